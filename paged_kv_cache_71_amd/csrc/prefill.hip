// prefill.hip -- causal paged attention for query chunks (chunked prefill).
//
// What is computed ("LLM inference, part 3: single node", ch. 13 secs. 1-2;
// CS349D lecture 3 sec. 7.2): row i of the chunk of sequence s sits at
// position context_lens[s] - Q_s + i and attends, through the block table, to
// the sequence's tokens 0 .. that position (earlier prompt chunks plus the
// chunk itself, already written by reshape_and_cache).
//
// 16-bit KV (bf16/f16): the only dense contraction of the path, so it runs on
// the gfx950 matrix cores (v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulation).
//  * Workgroup = 4 waves = 128 query rows of one (sequence, KV head): the rows
//    are (token, query head of the group) pairs, so the G heads that share a KV
//    head share every K/V tile (GQA reuse).  Each wave owns 32 rows.
//  * S^T = K Q^T per 32-token KV tile: K rows are the MFMA A operand and are
//    loaded straight from the paged pool into registers (each lane reads one
//    token row's contiguous half, 16 bytes at a time, its block found through
//    the table); Q^T is the B operand, loaded once.  In the 32x32 result each
//    lane holds 16 scores of ONE query row, so the softmax row max needs only
//    one cross-lane exchange (lane ^ 32).
//  * Online softmax in log2 units with a lazy rescale: the accumulator is only
//    rescaled when the running max grows by more than 2^8, so weights stay
//    <= 256 and most tiles skip the rescale.
//  * O^T = V^T P^T: the contraction runs over KV tokens, so V is staged in LDS
//    transposed ([d][token], double buffered, one barrier per tile) and read
//    as the A operand; the weights P^T come straight out of the score
//    registers as the B operand.  For bf16 the weights are split into
//    hi + lo bf16 parts (two MFMAs), keeping ~16 significant bits so the
//    result stays within fp32-accumulation accuracy even for peaked attention;
//    for f16 one f16 operand (11 bits) suffices.
//  * Workgroups of one (sequence, KV head) are mapped to the same XCD
//    (blockIdx % 8), so their shared K/V tiles are served from that XCD's L2.
//  * Positions past the row's causal limit, rows past the chunk and tokens
//    past the context are masked by selection (never multiplied), and memory
//    past the context is never dereferenced.
//
// fp32 KV: a plain vector-ALU kernel (one wave per query token and KV head).
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWG = 32 * kWaves;
constexpr int kKVT = 32;             // KV tokens per tile
constexpr int kVtPitch = kKVT + 4;   // LDS row pitch of V^T (elements), 8-byte aligned rows
constexpr float kRescaleThreshold = 8.0f;  // log2 units

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ uint4 ld16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

template <int DT>
__device__ __forceinline__ f32x16_t mfma32(const u32x4_t a, const u32x4_t b, f32x16_t c) {
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

// Two fp32 values -> one word of two 16-bit values of dtype DT (x in the low
// half), round to nearest even, with one packed hardware conversion.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  if constexpr (DT == DT_BF16) {
    typedef __bf16 b16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{x, y}), b16x2_t));
  } else {
    typedef _Float16 h16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{x, y}), h16x2_t));
  }
}
// The two 16-bit values of a word back in fp32 (exact).
template <int DT>
__device__ __forceinline__ float lo16(uint32_t w) {
  if constexpr (DT == DT_BF16) return __uint_as_float(w << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)w);
}
template <int DT>
__device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (DT == DT_BF16) return __uint_as_float(w & 0xffff0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

template <bool V>
struct BoolTag {
  static constexpr bool value = V;
};

__device__ __forceinline__ u32x4_t as_v(uint4 x) { return u32x4_t{x.x, x.y, x.z, x.w}; }

template <int DT, int D, bool PSPLIT>
__global__ __launch_bounds__(kThreads) void prefill_mfma_kernel(const PrefillArgs a) {
  constexpr int ES = 2;
  constexpr int NKK = D / 16;   // QK MFMAs per tile (16 of D each)
  constexpr int HALF = D / 2;   // d-values each lane half supplies
  constexpr int NDT = D / 32;   // 32-row d tiles of the PV output
  constexpr int CPR = D / 8;    // 16-byte chunks per token row
  constexpr int VCH = kKVT * CPR / kThreads;  // V chunks staged per thread per tile
  static_assert(VCH >= 1 && kKVT * CPR % kThreads == 0, "staging split");

  __shared__ uint16_t vt[2][D][kVtPitch];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5;     // lane half: which k-slice this lane supplies
  const int c32 = lane & 31;

  const int G = a.Hq / a.Hkv;
  const int TQ = kRowsPerWG / G;  // query tokens per workgroup
  const int nqt = (a.max_query_len + TQ - 1) / TQ;
  const int n_pairs = a.S * a.Hkv;
  const int b = blockIdx.x;
  int pair, qt;
  if ((n_pairs & 7) == 0) {  // all workgroups of a (sequence, KV head) on one XCD
    const int r = b >> 3;
    pair = (r / nqt) * 8 + (b & 7);
    qt = nqt - 1 - r % nqt;
  } else {
    pair = b / nqt;
    qt = nqt - 1 - b % nqt;
  }
  const int s = pair / a.Hkv;
  const int kvh = pair % a.Hkv;
  const int q0 = a.cu_seqlens_q[s];
  const int Qs = a.cu_seqlens_q[s + 1] - q0;
  const int L = min(a.context_lens[s], a.max_ctx);  // a larger value would overrun the table
  const int tq0 = qt * TQ;
  if (tq0 >= Qs || Qs > L) return;

  // this lane's query row (a column of S^T)
  const int r = wave * 32 + c32;
  const int tok = r / G;
  const int g = r % G;
  const bool row_valid = tok < TQ && tq0 + tok < Qs;
  const int pos = row_valid ? L - Qs + tq0 + tok : -1;
  int pos_min = pos;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) pos_min = min(pos_min, __shfl_xor(pos_min, off));
  pos_min = __builtin_amdgcn_readfirstlane(pos_min);

  const int kv_end = L - Qs + min(tq0 + TQ, Qs);  // tokens any row of this workgroup sees
  const int ntiles = (kv_end + kKVT - 1) / kKVT;

  // Q^T fragments (B operand): lane supplies Q[row][HALF*hf + 8*kk + 0..7]
  u32x4_t qf[NKK];
  {
    const char* qp = static_cast<const char*>(a.q) +
                     (((int64_t)(q0 + tq0 + tok) * a.Hq + (int64_t)kvh * G + g) * D + HALF * hf) * ES;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = row_valid ? as_v(ld16(qp + kk * 16)) : u32x4_t{0, 0, 0, 0};
  }

  const int32_t* __restrict__ table = a.block_tables + (int64_t)s * a.max_nb;
  const int64_t row_stride = (int64_t)a.Hkv * D * ES;
  const char* kbase = static_cast<const char*>(a.k_cache) + (int64_t)kvh * D * ES;
  const char* vbase = static_cast<const char*>(a.v_cache) + (int64_t)kvh * D * ES;
  const int log2B = a.log2B;
  const int bmask = a.B - 1;

  auto slot_off = [&](int kv) -> int64_t {
    const int ph = table[kv >> log2B];
    return ((int64_t)ph * a.B + (kv & bmask)) * row_stride;
  };

  // K fragment (A operand) of tile j: lane supplies K[kv0 + c32][HALF*hf + 8*kk + 0..7]
  u32x4_t kf[NKK];
  auto load_k = [&](int j) {
    const int kv = j * kKVT + c32;
    if (kv < kv_end) {
      const char* kp = kbase + slot_off(kv) + HALF * hf * ES;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) kf[kk] = as_v(ld16(kp + kk * 16));
    } else {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) kf[kk] = u32x4_t{0, 0, 0, 0};
    }
  };

  // V staging: chunk c = threadIdx.x + 256*i covers token c / CPR, d = 8*(c % CPR)
  uint4 vs[VCH];
  auto load_v = [&](int j) {
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = threadIdx.x + kThreads * i;
      const int kv = j * kKVT + c / CPR;
      vs[i] = kv < kv_end ? ld16(vbase + slot_off(kv) + (c % CPR) * 16) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_vt = [&](int buf) {
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = threadIdx.x + kThreads * i;
      const int kl = c / CPR;
      const int d0 = (c % CPR) * 8;
      const uint32_t w[4] = {vs[i].x, vs[i].y, vs[i].z, vs[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vt[buf][d0 + 2 * e][kl] = (uint16_t)(w[e] & 0xffffu);
        vt[buf][d0 + 2 * e + 1][kl] = (uint16_t)(w[e] >> 16);
      }
    }
  };

  f32x16_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.f;
  float m = -__builtin_inff();
  float lsum = 0.f;

  if (ntiles > 0) {
    load_v(0);
    load_k(0);
    store_vt(0);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const int kv0 = j * kKVT;
    // S^T tile: rows = KV tokens kv0 + 8*(v/4) + 4*hf + v%4, column = this lane's query row
    f32x16_t sacc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) sacc = mfma32<DT>(kf[kk], qf[kk], sacc);

    const bool more = j + 1 < ntiles;
    if (more) {
      load_k(j + 1);
      load_v(j + 1);
    }

    float sc[16];
    const bool need_mask = kv0 + kKVT - 1 > pos_min;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      sc[v] = sacc[v] * a.scale_log2;
      if (need_mask) {
        const int kv = kv0 + 8 * (v >> 2) + 4 * hf + (v & 3);
        sc[v] = kv <= pos ? sc[v] : -__builtin_inff();
      }
    }
    float tmax = sc[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) tmax = fmaxf(tmax, sc[v]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mn = fmaxf(m, tmax);
    const bool grow = mn > m + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? fast_exp2(m - mn) : 1.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
      lsum *= alpha;
      m = grow ? mn : m;
    }
    const float mu = m == -__builtin_inff() ? 0.f : m;
    uint32_t ph[8], pl[8];
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const float p0 = fast_exp2(sc[v] - mu);
      const float p1 = fast_exp2(sc[v + 1] - mu);
      lsum += p0 + p1;
      const uint32_t h = pack2<DT>(p0, p1);
      ph[v / 2] = h;
      if constexpr (PSPLIT) pl[v / 2] = pack2<DT>(p0 - lo16<DT>(h), p1 - hi16<DT>(h));
    }
    // O^T += V^T P^T over the tile's 32 tokens (two MFMAs of 16 tokens each)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const u32x4_t pb = u32x4_t{ph[4 * c], ph[4 * c + 1], ph[4 * c + 2], ph[4 * c + 3]};
      u32x4_t pbl;
      if constexpr (PSPLIT) pbl = u32x4_t{pl[4 * c], pl[4 * c + 1], pl[4 * c + 2], pl[4 * c + 3]};
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint16_t* rowp = &vt[buf][dt * 32 + c32][0];
        const uint2 x0 = *reinterpret_cast<const uint2*>(rowp + 16 * c + 4 * hf);
        const uint2 x1 = *reinterpret_cast<const uint2*>(rowp + 16 * c + 8 + 4 * hf);
        const u32x4_t va = u32x4_t{x0.x, x0.y, x1.x, x1.y};
        o[dt] = mfma32<DT>(va, pb, o[dt]);
        if constexpr (PSPLIT) o[dt] = mfma32<DT>(va, pbl, o[dt]);
      }
    }
    if (more) store_vt(buf ^ 1);
    __syncthreads();
  }

  if (!row_valid) return;
  const float lt = lsum + __shfl_xor(lsum, 32);
  const float inv = 1.f / lt;
  const int64_t orow = ((int64_t)(q0 + tq0 + tok) * a.Hq + (int64_t)kvh * G + g) * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int d = dt * 32 + 8 * v4 + 4 * hf;
      const float r0 = o[dt][4 * v4] * inv, r1 = o[dt][4 * v4 + 1] * inv;
      const float r2 = o[dt][4 * v4 + 2] * inv, r3 = o[dt][4 * v4 + 3] * inv;
      if (a.out_dt == DT_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow + d) = make_float4(r0, r1, r2, r3);
      } else {
        const bool bf = a.out_dt == DT_BF16;
        const uint32_t w0 = bf ? (f32_to_bf16_bits(r0) | ((uint32_t)f32_to_bf16_bits(r1) << 16))
                               : (f32_to_f16_bits(r0) | ((uint32_t)f32_to_f16_bits(r1) << 16));
        const uint32_t w1 = bf ? (f32_to_bf16_bits(r2) | ((uint32_t)f32_to_bf16_bits(r3) << 16))
                               : (f32_to_f16_bits(r2) | ((uint32_t)f32_to_f16_bits(r3) << 16));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow + d) = make_uint2(w0, w1);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tile kernel (16-bit KV, block size >= 16): both products on the 16x16x32
// matrix cores with the query row in lane % 16 throughout.
//
//  * Workgroup = 4 waves x QB x 16 query rows of one (sequence, KV head); a row
//    is a (token, query head of the group) pair, so the G heads sharing a KV
//    head share every K/V tile.
//  * Per 32-token KV tile, all 256 threads stage K and V rows (16-byte loads,
//    the tile's one or two blocks looked up a tile ahead) into LDS,
//    double buffered; the loads of tile j + 2 (and the table entries of tile
//    j + 3) are in flight while tile j is computed.  Rows past the context are
//    clamped to the last visible row.
//  * S^T = K Q^T: K (A operand, row-major from LDS, 16-byte reads over a
//    4-bank row skew) times Q^T (B operand, in registers for the whole loop).
//    Lane (g, n) receives S[kv = 4g + i (+16)][q = n].
//  * Online softmax per lane (its query row), max across the four lane groups
//    with permlane swaps; lazy rescale (only when the max grows by 2^8).
//  * O^T += V^T P^T: V^T is the A operand, read from row-major LDS with the
//    gfx950 transposing read ds_read_b64_tr_b16 (8-bank row skew, conflict
//    free); P^T is the B operand straight from the score registers.  Both use
//    the same order of the 32 tile tokens (4g + k, then 16 + 4g + k), so the
//    product over them is unchanged.  bf16: P is split into hi + lo bf16 parts
//    (two MFMAs), keeping ~16 significant bits of the weights.
//  * Workgroups of one (sequence, KV head) are mapped to the same XCD.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) int32_t cint32_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kTileKV = 32;                 // KV tokens per tile
constexpr int kWaitLgkm0 = 0xC07F;          // s_waitcnt: LDS/scalar count 0, others at max

template <int DT>
__device__ __forceinline__ f32x4_t mfma16(const u32x4_t a, const u32x4_t b, f32x4_t c) {
  if constexpr (DT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Transposing LDS read: lane j of each 16-lane group points at 4 consecutive
// 16-bit elements; lane i receives element i % 4 of lanes 4k + i / 4, k < 4.
__device__ __forceinline__ uint2 lds_read_tr16(const char* p) {
  const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
  return __builtin_bit_cast(uint2, r);
}

template <int N>
__device__ __forceinline__ void pair_max(float& x) {
  const unsigned u = __float_as_uint(x);
  if constexpr (N == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
}
template <int N>
__device__ __forceinline__ void pair_sum(float& x) {
  const unsigned u = __float_as_uint(x);
  if constexpr (N == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

template <int DT, int D, int QB>
__global__ __launch_bounds__(kThreads) void prefill_tile_kernel(const PrefillArgs a) {
  constexpr int ES = 2;
  constexpr int NKK = D / 32;                 // k-steps of S^T = K Q^T
  constexpr int NDB = D / 16;                 // 16-wide d blocks of O^T
  constexpr int KP = D * ES + 16;             // K row pitch in LDS: 4-bank skew
  constexpr int VP = D * ES + 32;             // V row pitch in LDS: 8-bank skew
  constexpr int CPR = D * ES / 16;            // 16-byte chunks per row
  constexpr int NCH = kTileKV * CPR / kThreads;  // chunks per thread per tile, K and V each
  constexpr int RW = kWaves * 16 * QB;        // query rows per workgroup
  constexpr bool PSPLIT = DT == DT_BF16;
  static_assert(NCH >= 1 && kTileKV * CPR % kThreads == 0, "staging split");

  __shared__ __attribute__((aligned(16))) char lk[2][kTileKV * KP];
  __shared__ __attribute__((aligned(16))) char lv[2][kTileKV * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4;  // lane group
  const int n = lane & 15;   // query column of each q block

  const int G = a.Hq / a.Hkv;
  const int TQ = RW / G;  // query tokens per workgroup
  const int nqt = (a.max_query_len + TQ - 1) / TQ;
  const int n_pairs = a.S * a.Hkv;
  const int b = blockIdx.x;
  int pair, qt;
  if ((n_pairs & 7) == 0) {  // all workgroups of a (sequence, KV head) on one XCD
    const int r = b >> 3;
    pair = (r / nqt) * 8 + (b & 7);
    qt = nqt - 1 - r % nqt;
  } else {
    pair = b / nqt;
    qt = nqt - 1 - b % nqt;
  }
  const int s = pair / a.Hkv;
  const int kvh = pair % a.Hkv;
  const int q0 = a.cu_seqlens_q[s];
  const int Qs = a.cu_seqlens_q[s + 1] - q0;
  const int L = min(a.context_lens[s], a.max_ctx);
  const int tq0 = qt * TQ;
  if (tq0 >= Qs || Qs > L) return;  // uniform over the workgroup, before any barrier

  // this lane's query rows (one per q block)
  int pos[QB], orow[QB];
  bool valid[QB];
  int pos_min = 0x7fffffff;
#pragma unroll
  for (int c = 0; c < QB; ++c) {
    const int r = 16 * (QB * wave + c) + n;
    const int tok = r / G;
    const int hq = r - tok * G;
    valid[c] = tok < TQ && tq0 + tok < Qs;
    pos[c] = valid[c] ? L - Qs + tq0 + tok : -1;
    orow[c] = valid[c] ? ((q0 + tq0 + tok) * a.Hq + kvh * G + hq) : 0;
    if (valid[c]) pos_min = min(pos_min, pos[c]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) pos_min = min(pos_min, __shfl_xor(pos_min, off));
  pos_min = __builtin_amdgcn_readfirstlane(pos_min);

  const int kv_end = L - Qs + min(tq0 + TQ, Qs);  // tokens any row of the workgroup sees
  const int ntiles = (kv_end + kTileKV - 1) / kTileKV;

  // Q^T fragments: lane holds Q[row][32 kk + 8 g4 .. + 7]
  u32x4_t qf[QB][NKK];
#pragma unroll
  for (int c = 0; c < QB; ++c) {
    const char* qp = static_cast<const char*>(a.q) + ((int64_t)orow[c] * D + 8 * g4) * ES;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[c][kk] = valid[c] ? as_v(ld16(qp + kk * 64)) : u32x4_t{0, 0, 0, 0};
  }
  // q must have landed before the loop: left pending, the loop header (where
  // the entry path meets the back edge) would wait for every load each tile
#pragma unroll
  for (int c = 0; c < QB; ++c)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) asm volatile("" ::"v"(qf[c][kk]));

  const int64_t row_stride = (int64_t)a.Hkv * D * ES;
  const int64_t blk_stride = row_stride * a.B;
  const int rs32 = (int)row_stride;
  const int log2B = a.log2B;
  const int bmask = a.B - 1;
  const char* kpool = static_cast<const char*>(a.k_cache) + (int64_t)kvh * D * ES;
  const char* vpool = static_cast<const char*>(a.v_cache) + (int64_t)kvh * D * ES;

  // Table entries of a tile's one or two blocks, fetched a tile ahead through
  // the vector queue (lane 0: first block, lane 1: second block) so their
  // latency hides behind a whole tile instead of stalling the K/V loads.
  const int32_t* tbv = a.block_tables + (int64_t)s * a.max_nb;
  int ent = 0;
  auto ent_issue = [&](int j) __attribute__((always_inline)) {
    const int kv0 = j * kTileKV;
    const int idx = (lane & 1) ? min(kv0 + 16, kv_end - 1) >> log2B : kv0 >> log2B;
    ent = tbv[idx];
  };
  // global -> registers for tile j (entries from ent_issue(j))
  uint4 sk[NCH], sv[NCH];
  auto gload = [&](int j) __attribute__((always_inline)) {
    const int kv0 = j * kTileKV;
    const int b0 = kv0 >> log2B;
    const int64_t e0 = __builtin_amdgcn_readlane(ent, 0);
    const int64_t e1 = __builtin_amdgcn_readlane(ent, 1);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = tid + kThreads * i;
      const int row = ch / CPR;
      const int col = ch - row * CPR;
      const int kvc = min(kv0 + row, kv_end - 1);
      const int64_t base = ((kvc >> log2B) == b0 ? e0 : e1) * blk_stride;
      const unsigned off = (unsigned)((kvc & bmask) * rs32 + col * 16);
      sk[i] = ld16(kpool + base + off);
      sv[i] = ld16(vpool + base + off);
    }
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = tid + kThreads * i;
      const int row = ch / CPR;
      const int col = ch - row * CPR;
      *reinterpret_cast<uint4*>(&lk[buf][row * KP + col * 16]) = sk[i];
      *reinterpret_cast<uint4*>(&lv[buf][row * VP + col * 16]) = sv[i];
    }
  };
  // LDS writes of this thread are complete and every wave has arrived; global
  // loads already issued stay in flight (no memory fence on the barrier)
  auto lds_barrier = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x4_t o[NDB][QB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int c = 0; c < QB; ++c) o[d][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[QB], lsum[QB];
#pragma unroll
  for (int c = 0; c < QB; ++c) {
    m[c] = -__builtin_inff();
    lsum[c] = 0.f;
  }

  if (ntiles > 0) {
    ent_issue(0);
    gload(0);
    lstore(0);
    if (ntiles > 1) {
      ent_issue(1);
      gload(1);
      if (ntiles > 2) ent_issue(2);
    }
  }
  lds_barrier();

  // one KV tile; MASK: some token of the tile lies after some row's position
  auto tile = [&](const int j, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int buf = j & 1;
    const int kv0 = j * kTileKV;
    const char* K = lk[buf];
    const char* V = lv[buf];
    // S^T blocks: st[mb][c] holds S[kv0 + 16 mb + 4 g4 + i][q col n of block c]
    f32x4_t st[2][QB];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int c = 0; c < QB; ++c) st[mb][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const u32x4_t ka = as_v(*reinterpret_cast<const uint4*>(K + (16 * mb + n) * KP + 64 * kk + 16 * g4));
#pragma unroll
        for (int c = 0; c < QB; ++c) st[mb][c] = mfma16<DT>(ka, qf[c][kk], st[mb][c]);
      }
    }
    u32x4_t ph[QB], pl[QB];
    bool grow_any = false;
    float sc[QB][8], mnew[QB];
#pragma unroll
    for (int c = 0; c < QB; ++c) {
      float t = -__builtin_inff();
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = st[mb][c][i] * a.scale_log2;
          if constexpr (MASK) {
            const int kv = kv0 + 16 * mb + 4 * g4 + i;
            v = kv <= pos[c] ? v : -__builtin_inff();
          }
          sc[c][4 * mb + i] = v;
          t = fmaxf(t, v);
        }
      }
      pair_max<16>(t);
      pair_max<32>(t);
      mnew[c] = fmaxf(m[c], t);
      grow_any |= mnew[c] > m[c] + kRescaleThreshold;
    }
    if (__builtin_amdgcn_ballot_w64(grow_any)) {
#pragma unroll
      for (int c = 0; c < QB; ++c) {
        const bool grow = mnew[c] > m[c] + kRescaleThreshold;
        const float alpha = grow ? fast_exp2(m[c] - mnew[c]) : 1.f;
#pragma unroll
        for (int d = 0; d < NDB; ++d) o[d][c] *= alpha;
        lsum[c] *= alpha;
        m[c] = grow ? mnew[c] : m[c];
      }
    }
#pragma unroll
    for (int c = 0; c < QB; ++c) {
      const float mu = m[c] == -__builtin_inff() ? 0.f : m[c];
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int k = 0; k < 8; k += 2) {
        const float p0 = fast_exp2(sc[c][k] - mu);
        const float p1 = fast_exp2(sc[c][k + 1] - mu);
        lsum[c] += p0 + p1;
        const uint32_t h = pack2<DT>(p0, p1);
        hw[k / 2] = h;
        if constexpr (PSPLIT) lw[k / 2] = pack2<DT>(p0 - lo16<DT>(h), p1 - hi16<DT>(h));
      }
      ph[c] = u32x4_t{hw[0], hw[1], hw[2], hw[3]};
      if constexpr (PSPLIT) pl[c] = u32x4_t{lw[0], lw[1], lw[2], lw[3]};
    }
    // O^T += V^T P^T: A = V^T rows d0 + n, tokens 4 g4 + k and 16 + 4 g4 + k
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const char* vp = V + (4 * g4 + (n >> 2)) * VP + (16 * d + 4 * (n & 3)) * ES;
      const uint2 lo = lds_read_tr16(vp);
      const uint2 hi = lds_read_tr16(vp + 16 * VP);
      const u32x4_t va = u32x4_t{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int c = 0; c < QB; ++c) {
        o[d][c] = mfma16<DT>(va, ph[c], o[d][c]);
        if constexpr (PSPLIT) o[d][c] = mfma16<DT>(va, pl[c], o[d][c]);
      }
    }
    if (j + 1 < ntiles) {
      lstore(buf ^ 1);
      if (j + 2 < ntiles) {
        gload(j + 2);
        if (j + 3 < ntiles) ent_issue(j + 3);
      }
    }
    lds_barrier();
  };
  // tiles wholly at or before every row's position need no causal mask (a
  // wave without valid rows has pos_min = INT_MAX: no tile needs it)
  const int nfree = pos_min == 0x7fffffff ? ntiles : min(ntiles, (pos_min + 1) / kTileKV);
  for (int j = 0; j < nfree; ++j) tile(j, BoolTag<false>{});
  for (int j = nfree; j < ntiles; ++j) tile(j, BoolTag<true>{});

  // total weight of each row (the four lane groups hold different tokens)
#pragma unroll
  for (int c = 0; c < QB; ++c) {
    pair_sum<16>(lsum[c]);
    pair_sum<32>(lsum[c]);
  }
#pragma unroll
  for (int c = 0; c < QB; ++c) {
    if (!valid[c]) continue;
    const float inv = 1.f / lsum[c];
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const int64_t off = (int64_t)orow[c] * D + 16 * d + 4 * g4;
      const float r0 = o[d][c][0] * inv, r1 = o[d][c][1] * inv;
      const float r2 = o[d][c][2] * inv, r3 = o[d][c][3] * inv;
      if (a.out_dt == DT_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + off) = make_float4(r0, r1, r2, r3);
      } else {
        const bool bf = a.out_dt == DT_BF16;
        const uint32_t w0 = bf ? (f32_to_bf16_bits(r0) | ((uint32_t)f32_to_bf16_bits(r1) << 16))
                               : (f32_to_f16_bits(r0) | ((uint32_t)f32_to_f16_bits(r1) << 16));
        const uint32_t w1 = bf ? (f32_to_bf16_bits(r2) | ((uint32_t)f32_to_bf16_bits(r3) << 16))
                               : (f32_to_f16_bits(r2) | ((uint32_t)f32_to_f16_bits(r3) << 16));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + off) = make_uint2(w0, w1);
      }
    }
  }
}

// fp32 KV: one wave per (query token, KV head); each lane owns D/64 elements
// of every head of the group and the wave walks the visible tokens one by one.
template <int D, int GMAX>
__global__ __launch_bounds__(64) void prefill_f32_kernel(const PrefillArgs a) {
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x;
  const int row = blockIdx.x / a.Hkv;
  const int kvh = blockIdx.x % a.Hkv;
  int lo = 0, hi = a.S;  // sequence of this row: last s with cu[s] <= row
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_seqlens_q[mid] <= row) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int q0 = a.cu_seqlens_q[s];
  const int Qs = a.cu_seqlens_q[s + 1] - q0;
  const int L = min(a.context_lens[s], a.max_ctx);
  if (Qs > L) return;
  const int visible = L - Qs + (row - q0) + 1;
  const int G = a.Hq / a.Hkv;
  const int32_t* table = a.block_tables + (int64_t)s * a.max_nb;
  const float* qrow = static_cast<const float*>(a.q) + ((int64_t)row * a.Hq + (int64_t)kvh * G) * D;
  const float* kc = static_cast<const float*>(a.k_cache);
  const float* vc = static_cast<const float*>(a.v_cache);
  for (int g0 = 0; g0 < G; g0 += GMAX) {
    const int gn = min(GMAX, G - g0);
    float q[GMAX][EPL], acc[GMAX][EPL], m[GMAX], l[GMAX];
    for (int g = 0; g < GMAX; ++g) {
      m[g] = -__builtin_inff();
      l[g] = 0.f;
      for (int e = 0; e < EPL; ++e) {
        q[g][e] = g < gn ? qrow[(int64_t)(g0 + g) * D + lane * EPL + e] : 0.f;
        acc[g][e] = 0.f;
      }
    }
    for (int t = 0; t < visible; ++t) {
      const int64_t base = (((int64_t)table[t >> a.log2B] * a.B + (t & (a.B - 1))) * a.Hkv + kvh) * D;
      float kv[EPL], vv[EPL];
      for (int e = 0; e < EPL; ++e) {
        kv[e] = kc[base + lane * EPL + e];
        vv[e] = vc[base + lane * EPL + e];
      }
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        if (g >= gn) break;
        float z = 0.f;
        for (int e = 0; e < EPL; ++e) z = fmaf(q[g][e], kv[e], z);
        for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
        z *= a.scale_log2;
        const float mn = fmaxf(m[g], z);
        const float alpha = fast_exp2(m[g] - mn);
        const float p = fast_exp2(z - mn);
        l[g] = l[g] * alpha + p;
        for (int e = 0; e < EPL; ++e) acc[g][e] = acc[g][e] * alpha + p * vv[e];
        m[g] = mn;
      }
    }
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
      for (int e = 0; e < EPL && g < gn; ++e)
        store_out(a.out, a.out_dt, ((int64_t)row * a.Hq + (int64_t)kvh * G + g0 + g) * D + lane * EPL + e,
                  acc[g][e] / l[g]);
  }
}

constexpr int kTileQB = 2;  // q blocks of 16 rows per wave in the tile kernel

template <int DT, int D>
pkv_status launch_tile(const PrefillArgs& a, hipStream_t stream) {
  constexpr int RW = kWaves * 16 * kTileQB;
  const int G = a.Hq / a.Hkv;
  const int TQ = RW / G;
  const int64_t nqt = (a.max_query_len + TQ - 1) / TQ;
  const int64_t grid = nqt * a.S * a.Hkv;
  if (grid == 0) return PKV_OK;
  if (grid > 0x7fffffff) return fail(PKV_ERR_UNSUPPORTED, "prefill grid too large");
  hipLaunchKernelGGL((prefill_tile_kernel<DT, D, kTileQB>), dim3((unsigned)grid), dim3(kThreads), 0,
                     stream, a);
  return check_launch("paged_attention_prefill");
}

template <int DT, int D>
pkv_status launch_mfma(const PrefillArgs& a, hipStream_t stream) {
  // blocks of at least 16 tokens and groups that fit a workgroup: tile kernel
  if (a.B >= 16 && a.Hq / a.Hkv <= kWaves * 16 * kTileQB) return launch_tile<DT, D>(a, stream);
  const int G = a.Hq / a.Hkv;
  if (G > kRowsPerWG) return fail(PKV_ERR_UNSUPPORTED, "prefill: group size %d > %d", G, kRowsPerWG);
  const int TQ = kRowsPerWG / G;
  const int64_t nqt = (a.max_query_len + TQ - 1) / TQ;
  const int64_t grid = nqt * a.S * a.Hkv;
  if (grid == 0) return PKV_OK;
  if (grid > 0x7fffffff) return fail(PKV_ERR_UNSUPPORTED, "prefill grid too large");
  constexpr bool split = DT == DT_BF16;
  hipLaunchKernelGGL((prefill_mfma_kernel<DT, D, split>), dim3((unsigned)grid), dim3(kThreads), 0,
                     stream, a);
  return check_launch("paged_attention_prefill");
}

template <int D>
pkv_status launch_f32(const PrefillArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.Tq * a.Hkv;
  if (grid == 0) return PKV_OK;
  if (grid > 0x7fffffff) return fail(PKV_ERR_UNSUPPORTED, "prefill grid too large");
  hipLaunchKernelGGL((prefill_f32_kernel<D, 8>), dim3((unsigned)grid), dim3(64), 0, stream, a);
  return check_launch("paged_attention_prefill (f32)");
}

}  // namespace

pkv_status launch_prefill(int kv_dt, const PrefillArgs& a, hipStream_t stream) {
  if (kv_dt == DT_F32) {
    switch (a.D) {
      case 64: return launch_f32<64>(a, stream);
      case 128: return launch_f32<128>(a, stream);
    }
  } else if (kv_dt == DT_BF16) {
    switch (a.D) {
      case 64: return launch_mfma<DT_BF16, 64>(a, stream);
      case 128: return launch_mfma<DT_BF16, 128>(a, stream);
    }
  } else if (kv_dt == DT_F16) {
    switch (a.D) {
      case 64: return launch_mfma<DT_F16, 64>(a, stream);
      case 128: return launch_mfma<DT_F16, 128>(a, stream);
    }
  }
  return fail(PKV_ERR_UNSUPPORTED, "prefill: kv dtype %d, head_dim %d", kv_dt, a.D);
}

}  // namespace pkv
