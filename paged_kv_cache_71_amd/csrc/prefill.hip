// prefill.hip -- causal paged attention for query chunks (chunked prefill).
//
// What is computed ("LLM inference, part 3: single node", ch. 13 secs. 1-2;
// CS349D lecture 3 sec. 7.2): row i of the chunk of sequence s sits at
// position context_lens[s] - Q_s + i and attends, through the block table, to
// the sequence's tokens 0 .. that position (earlier prompt chunks plus the
// chunk itself, already written by reshape_and_cache).
//
// Kernels:
//  * prefill_tile_kernel -- 16-bit pools with blocks of >= 4 tokens, FP8
//    pools with blocks of >= 8:
//    the software-pipelined matrix-core kernel (both products on
//    v_mfma_f32_16x16x32, K/V staged through LDS); described above it.
//  * prefill_merge_kernel -- combines the partial results of launches whose
//    KV ranges were split (plan_prefill: few sequences, long contexts).
//  * prefill_mfma_kernel -- 16-bit pools with smaller blocks
//    (32x32x16 matrix-core kernel, K read straight from the pool).
//  * prefill_f32_kernel -- fp32 pools, a plain vector-ALU kernel.
// Positions past a row's causal limit, rows past the chunk and tokens past
// the context are masked by selection (never multiplied), and memory past the
// context is never dereferenced.
#include <algorithm>
#include <type_traits>

#include "pkv_internal.h"

namespace pkv {

// query-row boundary i of the launch's sequences (rows counted from q / out)
__device__ __forceinline__ int cu_at(const PrefillArgs& a, int i) {
  return a.cu_seqlens_q[i] - a.cu_base;
}
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
// The lo part of a 16-bit hi/lo split: x - (16-bit value in half H of w),
// where that value is x rounded to dtype DT.  The difference has at most 16
// significant bits, so it is exact in fp32 whatever the rounding of the sum;
// one packed dot2 instruction (w . (-1, -0) + x, or w . (+0, -1) + x)
// replaces an unpack and a subtraction (x is finite, so the zero factor adds
// nothing).  The low-half constant carries -0 in its high half: as (-1, +0)
// = 0x0000bf80 the compiler encodes the bf16 word as the inline constant
// -1.0, which the hardware reads as the fp32 pattern 0xbf800000, i.e. -1 in
// the high half (measured: wrong residuals); with -0 above it the word has no
// inline form and goes out as a literal.
template <int DT, int H>
__device__ __forceinline__ float residual16(float x, uint32_t w) {
  if constexpr (DT == DT_BF16) {
    typedef __bf16 b16x2_t __attribute__((ext_vector_type(2)));
    constexpr uint32_t kMinusOne = H == 0 ? 0x8000bf80u : 0xbf800000u;  // -1.0 in half H
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b16x2_t, w),
                                           __builtin_bit_cast(b16x2_t, kMinusOne), x, false);
  } else {
    typedef _Float16 h16x2_t __attribute__((ext_vector_type(2)));
    constexpr uint32_t kMinusOne = H == 0 ? 0x8000bc00u : 0xbc000000u;  // -1.0 in half H
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2_t, w),
                                  __builtin_bit_cast(h16x2_t, kMinusOne), x, false);
  }
}

template <bool V>
struct BoolTag {
  static constexpr bool value = V;
};

__device__ __forceinline__ u32x4_t as_v(uint4 x) { return u32x4_t{x.x, x.y, x.z, x.w}; }

// Blocks too small for the tile kernel (16-bit KV, B < 4):
// v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulation.
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
//  * O^T = V^T P^T: V is staged in LDS transposed ([d][token], double
//    buffered, one barrier per tile) and read as the A operand; the weights
//    P^T come straight out of the score registers as the B operand, split
//    into hi + lo 16-bit parts (two MFMAs), keeping ~16 significant bits of
//    the weights (bf16 and f16 alike: one f16 operand rounds a dominant
//    weight by up to 2^-12, which times |v| near 9 exceeds the 2e-3 bound).
//  * Workgroups of one (sequence, KV head) are mapped to the same XCD
//    (blockIdx % 8), so their shared K/V tiles are served from that XCD's L2.
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
  const int q0 = cu_at(a, s);
  const int Qs = cu_at(a, s + 1) - q0;
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
      if constexpr (PSPLIT) pl[v / 2] = pack2<DT>(residual16<DT, 0>(p0, h), residual16<DT, 1>(p1, h));
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
// Tile kernel (16-bit or FP8 KV, blocks of >= 4 or 8 tokens): both products on the 16x16x32
// matrix cores with the query row in lane % 16 throughout.
//
//  * Workgroup = 4 waves x 2 x 16 query rows of one (sequence, KV head); a row
//    is a (token, query head of the group) pair, so the G heads sharing a KV
//    head share every K/V tile.
//  * Per 32-token KV tile, all 256 threads stage K and V rows into LDS with
//    16-byte loads.  A wave's rows of one staging chunk lie in one 16-token
//    half of the tile, hence in one block: the address is a per-wave block
//    base (from the table entry, fetched one step ahead) plus a per-lane
//    offset; only the last tile clamps rows past the context to its last one.
//  * S^T = K Q^T: K (A operand, row-major from LDS, 16-byte reads) times Q^T
//    (B operand, in registers for the whole loop).  Lane (g, n) receives
//    S[kv = 4g + i (+16)][q = n].  Scores stay raw; the softmax scale enters
//    the exponent through one fma (a negative scale flips q's sign instead).
//  * Online softmax per lane (its query row), max across the four lane groups
//    with permlane swaps; lazy rescale (only when the max grows by 2^8).
//  * O^T += V^T P^T: V^T is the A operand, read from row-major LDS with the
//    gfx950 transposing read ds_read_b64_tr_b16; P^T is the B operand straight
//    from the score registers.  Both use the same order of the 32 tile tokens
//    (4g + k, then 16 + 4g + k), so the product over them is unchanged.  P
//    is split into hi + lo 16-bit parts (two MFMAs), keeping ~16 significant
//    bits of the weights, for f16 as for bf16 (see the kernel above).
//  * Software pipeline: in the step for tile j the matrix cores run
//    O += P(j-1) V(j-1) and S(j+1) = Q K(j+1)^T while the vector ALU runs the
//    softmax of S(j), all three independent, so each wave's instruction
//    stream interleaves matrix and vector work.  K runs two tiles ahead of V
//    in the LDS double buffers; one barrier per step.
//  * LDS rows carry 32 bytes of skew, which makes the K reads, the
//    transposing V reads and the staging writes conflict free.
//  * Workgroups of one (sequence, KV head) are mapped to the same XCD.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) int32_t cint32_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kTileKV = 32;                 // KV tokens per tile
constexpr int kWaitLgkm0 = 0xC07F;          // s_waitcnt: LDS/scalar count 0, others at max
constexpr int kTileQB = 2;                  // q blocks of 16 rows per wave
// Waves per tile-kernel workgroup.  16-bit D = 128 runs 8 waves, two per
// SIMD, as two groups of four that take turns between a step's matrix part
// and its vector part (see the kernel); the other instantiations run 4 waves,
// two workgroups per CU: D = 64, whose 16-byte staging does not split over
// 512 threads, and FP8 pools (8 waves with 8-byte code chunks measured
// 1.171 against 1.135 ms on the 8 x 512 batch).
__host__ __device__ constexpr int tile_waves(int D, bool F8, bool NARROW) {
  return (!F8 && !NARROW && D == 128) ? 8 : 4;
}
// The tile kernel adds the lo parts of the weights (second P.V product) only
// on tiles where some row's largest weight exceeds 4% of that row's running
// total (kLog2LoShare = log2(0.04)); see the softmax step.
constexpr float kLog2LoShare = -4.6438562f;

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

// Maximum of three fp32 values in one instruction.  Written as asm because
// fmaxf on matrix-core results is preceded by a canonicalising v_max(x, x)
// per operand (IEEE mode); no NaN reaches these maxima except through an
// input that is NaN already, and then the row is NaN either way.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// Row max across the four lane groups (lanes n, n + 16, n + 32, n + 48).
__device__ __forceinline__ float group_max_raw(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = max3_raw(__uint_as_float(r16[0]), __uint_as_float(r16[1]), __uint_as_float(r16[0]));
  const unsigned w = __float_as_uint(y);
  const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return max3_raw(__uint_as_float(r32[0]), __uint_as_float(r32[1]), __uint_as_float(r32[0]));
}

// F8: the pools hold OCP E4M3 codes (one scale per KV head); they are widened
// to DT (q's dtype, exact) as they go into LDS, so everything after the
// staging is the 16-bit kernel.
// NARROW (16-bit D = 64 over blocks of 4 tokens): 8-byte staging chunks, so a
// wave stages 4 rows per chunk and they lie in one block
template <int DT, int D, bool F8, bool NARROW = false>
__global__ __launch_bounds__(64 * tile_waves(D, F8, NARROW)) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_tile_kernel(
    const PrefillArgs a) {
  constexpr int TW = tile_waves(D, F8, NARROW);
  constexpr int TT = 64 * TW;      // threads
  constexpr bool PP = TW == 8;     // two groups of four waves, one phase apart
  constexpr int QB = kTileQB;
  constexpr int ES = 2;            // q and LDS element bytes
  constexpr int ESK = F8 ? 1 : 2;  // pool element bytes
  constexpr int NKK = D / 32;                 // k-steps of S^T = K Q^T
  constexpr int NDB = D / 16;                 // 16-wide d blocks of O^T
  // LDS row pitches: 32 bytes of skew per row make both the 16-byte K reads
  // and the transposing V reads conflict free (measured: a 16-byte skew
  // costs the K reads 1.6x)
  constexpr int KP = D * ES + 32;
  constexpr int VP = D * ES + 32;
  static_assert(!NARROW || (!F8 && D == 64), "8-byte chunks: 16-bit D = 64 only");
  constexpr int CPR = F8 ? 8 : D * ES / (NARROW ? 8 : 16);  // staging chunks per row
  constexpr int CBP = D * ESK / CPR;             // pool bytes per chunk (16, or 8 for FP8 D = 64)
  constexpr int CBL = D * ES / CPR;              // LDS bytes per chunk (16 or 32)
  constexpr int NCH = kTileKV * CPR / TT;  // chunks per thread per tile, K and V each
  using Chunk = std::conditional_t<CBP == 16, uint4, uint2>;
  static_assert(CBP == 16 || CBP == 8, "staging chunk");
  constexpr int RW = TW * 16 * QB;        // query rows per workgroup
  constexpr bool PSPLIT = true;  // hi + lo parts of P for both 16-bit dtypes
  static_assert(NCH >= 1 && NCH <= 2 && kTileKV * CPR % TT == 0, "staging split");
  static_assert(16 % (64 / CPR) == 0, "a wave's staged rows must lie in one 16-token half");

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
  const int ns = a.n_split;
  const int units = nqt * ns;  // workgroups per (sequence, KV head): query tiles x splits
  const int n_pairs = a.S * a.Hkv;
  const int b = blockIdx.x;
  int pair, u;
  if ((n_pairs & 7) == 0) {  // all workgroups of a (sequence, KV head) on one XCD
    const int r = b >> 3;
    pair = (r / units) * 8 + (b & 7);
    u = r % units;
  } else {
    pair = b / units;
    u = b % units;
  }
  const int qt = nqt - 1 - u / ns;  // longest query tiles first
  const int sp = u % ns;
  const int s = pair / a.Hkv;
  const int kvh = pair % a.Hkv;
  const int q0 = cu_at(a, s);
  const int Qs = cu_at(a, s + 1) - q0;
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
  const int ntiles = (kv_end + kTileKV - 1) / kTileKV;  // >= 1 here
  // this workgroup's tiles t0 .. tl (split sp of the rows' range)
  const int tps = ns > 1 ? a.tiles_per_split : ntiles;
  const int t0 = sp * tps;
  if (t0 >= ntiles) return;  // past the rows' last tile; uniform, before any barrier
  const int tl = min(ntiles, t0 + tps) - 1;
  const bool partial = ntiles > tps;  // the rows' range spans several splits

  // Scores are kept as raw q.k; the softmax scale enters the exponent through
  // one fma.  A negative scale flips the sign of q instead (exact for 16-bit
  // values), so the factor used is |scale| and the running max stays a max.
  // FP8 pools: the K scale joins the softmax scale, the V scale the output.
  const float kscale = F8 ? a.k_scale[kvh] : 1.f;
  const float oscale = F8 ? a.v_scale[kvh] : 1.f;
  const float sl = fabsf(a.scale_log2 * kscale);
  const uint32_t qflip = a.scale_log2 * kscale < 0.f ? 0x80008000u : 0u;

  // Q^T fragments: lane holds Q[row][32 kk + 8 g4 .. + 7]
  u32x4_t qf[QB][NKK];
#pragma unroll
  for (int c = 0; c < QB; ++c) {
    const char* qp = static_cast<const char*>(a.q) + ((int64_t)orow[c] * D + 8 * g4) * ES;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[c][kk] = valid[c] ? (as_v(ld16(qp + kk * 64)) ^ qflip) : u32x4_t{0, 0, 0, 0};
  }
  // q must have landed before the loop: left pending, the loop header (where
  // the entry path meets the back edge) would wait for every load each step
#pragma unroll
  for (int c = 0; c < QB; ++c)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) asm volatile("" ::"v"(qf[c][kk]));

  const int64_t row_stride = (int64_t)a.Hkv * D * ESK;
  const int64_t blk_stride = row_stride * a.B;
  const int rs32 = (int)row_stride;
  const int log2B = a.log2B;
  const int bmask = a.B - 1;
  const char* kpool = static_cast<const char*>(a.k_cache) + (int64_t)kvh * D * ESK;
  const char* vpool = static_cast<const char*>(a.v_cache) + (int64_t)kvh * D * ESK;
  const int32_t* tbv = a.block_tables + (int64_t)s * a.max_nb;

  // Staging: chunk i of a thread is column ch % CPR of tile row ch / CPR
  // (ch = tid + 256 i): CBP pool bytes, CBL bytes in LDS.  The rows a wave
  // stages for one chunk are 64 / CPR consecutive rows, aligned, so they lie
  // in one block whenever B >= 64 / CPR (the host launches this kernel only
  // then): a chunk's pool address is a per-wave block base plus a per-lane
  // offset.  Tiles start at multiples of 32 >= B, so a row's place in its
  // block is its tile row & (B - 1).
  const int log2E = log2B < 4 ? log2B : 4;  // tokens per table entry read: min(B, 16)
  int crow[NCH], ccol[NCH], csel[NCH];
  uint32_t loff[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int ch = tid + TT * i;
    crow[i] = ch / CPR;
    ccol[i] = ch - crow[i] * CPR;
    csel[i] = __builtin_amdgcn_readfirstlane(crow[i] >> log2E);  // entry of this wave's rows
    loff[i] = (uint32_t)((crow[i] & bmask) * rs32 + ccol[i] * CBP);
  }
  // Block table entry of chunk i's rows in tile t: the block of token
  // 32 t + min(B, 16) csel[i], clamped to the last visible token (so the
  // table is never read past the sequence's blocks, and a run of rows past
  // the context finds the block of the row it is clamped to).  Wave-uniform:
  // a scalar load through the constant address space, no vector work.
  const cint32_t* tbs = (const cint32_t*)tbv;
  auto ent = [&](int t, int i) __attribute__((always_inline)) -> int {
    const int kv = min(t * kTileKV + (csel[i] << log2E), kv_end - 1);
    return tbs[kv >> log2B];
  };
  // global -> registers: the chunks of tile t (entry e0 for chunk 0, e1 for
  // chunk 1).
  // Rows past the visible range (last tile only) repeat its last row.  The
  // block base is an unsigned 32 x 32 -> 64-bit product: entries reached here
  // are physical block ids (>= 0) and a block is under 2 GiB (checked on the
  // host), which spares the signed 64-bit multiply's scalar instructions.
  auto ldc = [](const char* p) __attribute__((always_inline)) -> Chunk {
    return *reinterpret_cast<const Chunk*>(p);
  };
  auto gload = [&](Chunk (&dst)[NCH], const char* pool, int t, int e0, int e1)
      __attribute__((always_inline)) {
    const int kv0 = t * kTileKV;
    const bool full = kv0 + kTileKV <= kv_end;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      // uniform block base (scalar registers) + a 32-bit per-lane offset
      const char* base = pool + (uint64_t)(uint32_t)(i ? e1 : e0) * (uint32_t)blk_stride;
      uint32_t off = loff[i];
      if (!full) off = (uint32_t)((min(kv0 + crow[i], kv_end - 1) & bmask) * rs32 + ccol[i] * CBP);
      dst[i] = ldc(base + off);
    }
  };
  auto lstore = [&](char* buf, int pitch, const Chunk (&src)[NCH]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      char* dst = buf + crow[i] * pitch + ccol[i] * CBL;
      if constexpr (!F8 && CBP == 8) {
        *reinterpret_cast<uint2*>(dst) = src[i];
      } else if constexpr (!F8) {
        *reinterpret_cast<uint4*>(dst) = src[i];
      } else if constexpr (CBP == 16) {
        *reinterpret_cast<uint4*>(dst) = fp8x8_to16<DT>(make_uint2(src[i].x, src[i].y));
        *reinterpret_cast<uint4*>(dst + 16) = fp8x8_to16<DT>(make_uint2(src[i].z, src[i].w));
      } else {
        *reinterpret_cast<uint4*>(dst) = fp8x8_to16<DT>(src[i]);
      }
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

  // o[d][c]: O^T blocks of q block c; o[NDB][c]: the row sums of the weights
  f32x4_t o[NDB + 1][QB];
#pragma unroll
  for (int d = 0; d <= NDB; ++d)
#pragma unroll
    for (int c = 0; c < QB; ++c) o[d][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // running maxima (log2 units); -FLT_MAX before a row's first visible token:
  // the first visible score always grows it, and weights are only formed
  // from visible scores (masked ones are selected to 0)
  float m[QB];
#pragma unroll
  for (int c = 0; c < QB; ++c) m[c] = -__FLT_MAX__;

  // Software pipeline over KV tiles.  Step j (j = -1 .. ntiles):
  //   1. stage K(j+2) and V(j) into LDS (loaded during step j-1), then issue
  //      the loads of K(j+3) and V(j+1) and of the table entries of tile j+4;
  //   2. matrix cores: O^T += V(j-1)^T P(j-1)^T (with the row sums of
  //      P(j-1)) and S(j+1)^T = K(j+1) Q^T;
  //   3. vector ALU, independent of 2: softmax of S(j) into P(j);
  //   4. rare: rescale O when some row's max grew; barrier.
  // So the softmax of one tile runs while the matrix cores work on the tiles
  // on either side of it.  K(t) sits in LDS buffer t % 2 during steps t-2 ..
  // t-1, V(t) in buffer t % 2 during steps t .. t+1.  Tile indices past the
  // last tile are clamped to it (their loads repeat it and are never used).
  Chunk sk[NCH], sv[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) sv[i] = Chunk{};
  // entries (chunk 0, chunk NCH - 1) of tiles j+1, j+2 and j+3 at step j
  int ea0 = ent(t0, 0), ea1 = ent(t0, NCH - 1);
  int eb0 = ent(min(t0 + 1, tl), 0), eb1 = ent(min(t0 + 1, tl), NCH - 1);
  int en0 = ent(min(t0 + 2, tl), 0), en1 = ent(min(t0 + 2, tl), NCH - 1);
  gload(sk, kpool, t0, ea0, ea1);
  lstore(lk[t0 & 1], KP, sk);
  gload(sk, kpool, min(t0 + 1, tl), eb0, eb1);
  lds_barrier();

  f32x4_t SA[2][QB], SB[2][QB];   // S of the tile being softmaxed / of the next one
  u32x4_t PAh[QB], PAl[QB], PBh[QB], PBl[QB];  // P of the previous tile / of this one
  bool FA = false, FB = false;   // whether that P has its lo parts (uniform)

  auto step = [&](const int j, auto ld_tag, auto pv_tag, auto qk_tag, auto sm_tag, auto mask_tag,
                  f32x4_t (&s_cur)[2][QB], f32x4_t (&s_nxt)[2][QB], const u32x4_t (&pph)[QB],
                  const u32x4_t (&ppl)[QB], u32x4_t (&nph)[QB], u32x4_t (&npl)[QB], bool pflag,
                  bool& nflag)
      __attribute__((always_inline)) {
    constexpr bool LD = decltype(ld_tag)::value;
    constexpr bool PV = decltype(pv_tag)::value;
    constexpr bool QK = decltype(qk_tag)::value;
    constexpr bool SM = decltype(sm_tag)::value;
    constexpr bool MASK = decltype(mask_tag)::value;
    if constexpr (LD) {
      lstore(lk[j & 1], KP, sk);
      lstore(lv[j & 1], VP, sv);
      const int ec0 = en0, ec1 = en1;
      // two groups: the entries of tile j+4 are fetched in the vector part,
      // so no scalar load is pending while the matrix part waits for its LDS
      // reads (the shared counter would make it wait for all of them)
      if constexpr (!PP) {
        en0 = ent(min(j + 4, tl), 0);
        en1 = ent(min(j + 4, tl), NCH - 1);
      }
      gload(sk, kpool, min(j + 3, tl), ec0, ec1);
      gload(sv, vpool, min(j + 1, tl), ea0, ea1);
      ea0 = eb0;
      ea1 = eb1;
      eb0 = ec0;
      eb1 = ec1;
    }
    // K fragments of tile j+1, read before the P.V products are issued so
    // their LDS latency hides behind them (1.116 -> 1.072 ms on 8 x 512
    // chunks, against reading each pair right before its two products)
    u32x4_t kfr[2][NKK];
    if constexpr (QK) {
      const char* K = lk[(j + 1) & 1];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          kfr[mb][kk] = as_v(*reinterpret_cast<const uint4*>(K + (16 * mb + n) * KP + 64 * kk + 16 * g4));
    }
    // O^T += V^T P^T over the D columns of V and a block of ones (an A
    // operand of 1.0 in every element, from registers), so o[NDB][c] holds
    // every row's sum of its weights as they entered the product.  A = V^T
    // rows 16 d + n, tokens 4 g4 + k and 16 + 4 g4 + k.
    const char* V = lv[(j - 1) & 1];
    auto pv_pass = [&](const u32x4_t (&pp)[QB]) __attribute__((always_inline)) {
#pragma unroll
      for (int d = 0; d <= NDB; ++d) {
        u32x4_t va;
        if (d < NDB) {
          const char* vp = V + (4 * g4 + (n >> 2)) * VP + (16 * d + 4 * (n & 3)) * ES;
          const uint2 lo = lds_read_tr16(vp);
          const uint2 hi = lds_read_tr16(vp + 16 * VP);
          va = u32x4_t{lo.x, lo.y, hi.x, hi.y};
        } else {
          const uint32_t one2 = DT == DT_BF16 ? 0x3f803f80u : 0x3c003c00u;
          va = u32x4_t{one2, one2, one2, one2};
        }
#pragma unroll
        for (int c = 0; c < QB; ++c) o[d][c] = mfma16<DT>(va, pp[c], o[d][c]);
      }
    };
    // each row's total weight through P(j-2) (P(j-1) is added below)
    float lprev[QB];
    if constexpr (SM) {
#pragma unroll
      for (int c = 0; c < QB; ++c) lprev[c] = o[NDB][c][0];
    }
    if constexpr (PV) pv_pass(pph);
    // two groups: the lo parts of P(j-1) join this step's matrix part
    if constexpr (PP && PV) {
      if (pflag) pv_pass(ppl);
    }
    if constexpr (QK) {
      // S^T blocks: s_nxt[mb][c] holds S[16 mb + 4 g4 + i][q col n of block c]
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int c = 0; c < QB; ++c) s_nxt[mb][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
          for (int c = 0; c < QB; ++c) s_nxt[mb][c] = mfma16<DT>(kfr[mb][kk], qf[c][kk], s_nxt[mb][c]);
      }
    }
    // two groups: the matrix part ends here (its results are taken as
    // complete, so the compiler moves none of it, nor of the vector part,
    // across the barrier); the other group's matrix part runs while this
    // group's vector part does
    if constexpr (PP && LD) {
#pragma unroll
      for (int c = 0; c < QB; ++c) {
#pragma unroll
        for (int d = 0; d <= NDB; ++d) asm volatile("" ::"v"(o[d][c]));
        if constexpr (QK) asm volatile("" ::"v"(s_nxt[0][c]), "v"(s_nxt[1][c]));
      }
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      en0 = ent(min(j + 4, tl), 0);
      en1 = ent(min(j + 4, tl), NCH - 1);
    }
    bool grow[QB];
    uint64_t grow_mask = 0, lo_mask = 0;  // lanes whose row's max grew / that want the lo parts
    float mold[QB], pk[QB][8];  // previous maxima; this tile's weights (for their lo parts)
    if constexpr (SM) {
      const int kv0 = j * kTileKV;
#pragma unroll
      for (int c = 0; c < QB; ++c) {
        float r[8];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = s_cur[mb][c][i];
            if constexpr (MASK) v = kv0 + 16 * mb + 4 * g4 + i <= pos[c] ? v : -__builtin_inff();
            r[4 * mb + i] = v;
          }
        const float t = group_max_raw(
            max3_raw(max3_raw(r[0], r[1], r[2]), max3_raw(r[3], r[4], r[5]), max3_raw(r[6], r[7], r[7])));
        // the max grows (lazily) when the tile's exceeds it by the threshold,
        // and is then the tile's; tsl is NaN only when all masked and scale 0
        // (no growth then)
        const float tsl = t * sl;
        grow[c] = tsl > m[c] + kRescaleThreshold;
        mold[c] = m[c];
        m[c] = grow[c] ? tsl : m[c];
        grow_mask |= __builtin_amdgcn_ballot_w64(grow[c]);
        const float mu = m[c];
        uint32_t hw[4];
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
          float p0 = fast_exp2(__builtin_fmaf(r[k], sl, -mu));
          float p1 = fast_exp2(__builtin_fmaf(r[k + 1], sl, -mu));
          if constexpr (MASK) {
            const int kv = kv0 + 16 * (k >> 2) + 4 * g4 + (k & 3);
            p0 = kv <= pos[c] ? p0 : 0.f;
            p1 = kv + 1 <= pos[c] ? p1 : 0.f;
          }
          pk[c][k] = p0;
          pk[c][k + 1] = p1;
          hw[k / 2] = pack2<DT>(p0, p1);
        }
        nph[c] = u32x4_t{hw[0], hw[1], hw[2], hw[3]};
        if constexpr (PSPLIT) {
          // Rounding the weights w_i to 16 bits (by d_i, |d_i| <= eps w_i)
          // moves the row's result by sum_i d_i (v_i - o) / total (the total
          // is the sum of the same rounded weights, so a dominant weight's
          // rounding cancels).  The roundings of different weights are
          // independent, so the shift is of order eps sqrt(sum_i (w_i /
          // total)^2) |v - o| <= eps sqrt(p) |v - o| when no weight exceeds a
          // share p of the total.  Where the largest weight of every row is
          // at most 4% of the row's total (a lower bound of it: the total two
          // tiles back), that is a fifth of one weight's rounding, well inside
          // the tolerance, and the lo parts are skipped; else this tile
          // carries them (about 16 significant bits per weight).  A grown
          // maximum (a new dominant token) always does.
          // The test is taken in log2 units: the row's largest weight is
          // 2^(tsl - mu); log2(0.04 * total) comes from the total's bits
          // (e + f - 127 for 2^(e - 127) (1 + f), at most 0.087 below log2,
          // so it errs towards carrying the lo parts).  All masked or scale
          // 0: -inf or NaN, no lo parts.
          const float lg = (float)__float_as_int(lprev[c]) * 0x1p-23f + (kLog2LoShare - 127.f);
          lo_mask |= __builtin_amdgcn_ballot_w64(tsl - mu > lg);
        }
      }
    }
    // the lo parts of P(j-1): a second pass over the same V tile
    if constexpr (!PP && PV) {
      if (pflag) pv_pass(ppl);
    }
    if constexpr (SM) {
      nflag = PSPLIT && (lo_mask | grow_mask) != 0;
      if (nflag) {
#pragma unroll
        for (int c = 0; c < QB; ++c) {
          uint32_t lw[4];
#pragma unroll
          for (int k = 0; k < 8; k += 2) {
            const uint32_t h = nph[c][k / 2];
            lw[k / 2] = pack2<DT>(residual16<DT, 0>(pk[c][k], h), residual16<DT, 1>(pk[c][k + 1], h));
          }
          npl[c] = u32x4_t{lw[0], lw[1], lw[2], lw[3]};
        }
      }
      // O now includes P(j-1) V(j-1): bring it (and the row sums) to the new max
      if (grow_mask) {
#pragma unroll
        for (int c = 0; c < QB; ++c) {
          const float alpha = grow[c] ? fast_exp2(mold[c] - m[c]) : 1.f;
#pragma unroll
          for (int d = 0; d <= NDB; ++d) o[d][c] *= alpha;
        }
      }
    }
    if constexpr (LD) lds_barrier();
  };
  using T = BoolTag<true>;
  using F = BoolTag<false>;
  auto copy_back = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < QB; ++c) {
      SA[0][c] = SB[0][c];
      SA[1][c] = SB[1][c];
      PAh[c] = PBh[c];
      if constexpr (PSPLIT) PAl[c] = PBl[c];
    }
    FA = FB;
  };

  // Two groups (8 waves): waves 4-7 run one phase behind waves 0-3 -- one
  // barrier more here, waves 0-3 one more after the loop -- so while one
  // group issues a step's matrix part the other issues its vector part.
  // Every staging step has two barriers (after each part).  A tile's staging
  // is written half by each group, in consecutive phases, and read two
  // phases later; buffer reuse keeps the one-group distances (K(t) written
  // in the steps of tile t-2, V(t) in those of tile t, both read in the next).
  if constexpr (PP) {
    if (wave >= 4) __builtin_amdgcn_s_barrier();
  }
  // step t0-1: S(t0) into SB; step t0: softmax(t0), S(t0+1) into SA, P(t0) into PA
  step(t0 - 1, T{}, F{}, T{}, F{}, F{}, SA, SB, PAh, PAl, PBh, PBl, FA, FB);
  step(t0, T{}, F{}, T{}, T{}, T{}, SB, SA, PBh, PBl, PAh, PAl, FB, FA);
  if (tl > t0) {
    // steady state, unrolled by two so S and P alternate between the A and B
    // registers; tiles wholly at or before every row's position skip the mask
    const int nfree = pos_min == 0x7fffffff ? tl : max(t0 + 1, min(tl, (pos_min + 1) / kTileKV));
    int j = t0 + 1;
    for (; j + 1 < nfree; j += 2) {
      step(j, T{}, T{}, T{}, T{}, F{}, SA, SB, PAh, PAl, PBh, PBl, FA, FB);
      step(j + 1, T{}, T{}, T{}, T{}, F{}, SB, SA, PBh, PBl, PAh, PAl, FB, FA);
    }
    if (j < nfree) {
      step(j, T{}, T{}, T{}, T{}, F{}, SA, SB, PAh, PAl, PBh, PBl, FA, FB);
      copy_back();
      ++j;
    }
    for (; j < tl; ++j) {
      step(j, T{}, T{}, T{}, T{}, T{}, SA, SB, PAh, PAl, PBh, PBl, FA, FB);
      copy_back();
    }
    // last tile: no next S; P(tl) into PB, then its product
    step(tl, T{}, T{}, F{}, T{}, T{}, SA, SB, PAh, PAl, PBh, PBl, FA, FB);
    step(tl + 1, F{}, T{}, F{}, F{}, F{}, SA, SB, PBh, PBl, PAh, PAl, FB, FA);
  } else {
    step(t0 + 1, F{}, T{}, F{}, F{}, F{}, SA, SB, PAh, PAl, PBh, PBl, FA, FB);
  }
  if constexpr (PP) {
    if (wave < 4) __builtin_amdgcn_s_barrier();
  }

  // total weight of each row: the ones block of O (in every lane of the row)
  float lsum[QB];
#pragma unroll
  for (int c = 0; c < QB; ++c) lsum[c] = o[NDB][c][0];
  if (partial) {
    // unnormalised output, running max and weight sum of this split
    const int64_t rec = (int64_t)sp * a.Tq * a.Hq;
#pragma unroll
    for (int c = 0; c < QB; ++c) {
      if (!valid[c]) continue;
      float* po = a.ws_o + (rec + orow[c]) * D;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
        *reinterpret_cast<float4*>(po + 16 * d + 4 * g4) =
            make_float4(o[d][c][0] * oscale, o[d][c][1] * oscale, o[d][c][2] * oscale,
                        o[d][c][3] * oscale);
      if (g4 == 0) *reinterpret_cast<float2*>(a.ws_ml + (rec + orow[c]) * 2) = make_float2(m[c], lsum[c]);
    }
    return;
  }
#pragma unroll
  for (int c = 0; c < QB; ++c) {
    if (!valid[c]) continue;
    const float inv = F8 ? oscale / lsum[c] : 1.f / lsum[c];
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

// Merge of split prefill results ("Flash-Decoding" style log-sum-exp merge of
// partial softmax results over disjoint KV ranges): 16 lanes per output row
// (token, query head), 16 rows per workgroup, 16-byte loads; rows whose range
// was not split were written by the tile kernel and are skipped.  The splits'
// (m, l) pairs and partial outputs are loaded CH at a time, so a row costs one
// memory round trip for up to CH splits:
//   out = sum_i e^(m_i - M) o_i / sum_i e^(m_i - M) l_i.
// RW: query rows per workgroup of the tile kernel whose partials are merged
// (a row's query tile, hence its split count, follows from it).
template <int D, int RW>
__global__ __launch_bounds__(256) void prefill_merge_kernel(const PrefillArgs a) {
  constexpr int EPL = D / 16;  // outputs per lane: 8 or 4
  constexpr int NV = EPL / 4;  // float4 loads per lane and split
  constexpr int CH = 8;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c0 = (threadIdx.x & 15) * EPL;
  const int64_t nrows = (int64_t)a.Tq * a.Hq;
  if (row >= nrows) return;
  const int t = (int)(row / a.Hq);
  int lo = 0, hi = a.S;  // sequence of token t: last s with cu[s] <= t
  if (t >= cu_at(a, a.S)) return;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_at(a, mid) <= t) lo = mid; else hi = mid;
  }
  const int q0 = cu_at(a, lo);
  const int Qs = cu_at(a, lo + 1) - q0;
  const int L = min(a.context_lens[lo], a.max_ctx);
  if (Qs > L) return;  // skipped by the tile kernel as well
  const int TQ = RW / (a.Hq / a.Hkv);
  const int qt = (t - q0) / TQ;
  const int kv_end = L - Qs + min(qt * TQ + TQ, Qs);
  const int ntiles = (kv_end + kTileKV - 1) / kTileKV;
  const int nu = (ntiles + a.tiles_per_split - 1) / a.tiles_per_split;
  if (nu <= 1) return;
  const int64_t stride = nrows;
  float M = -__builtin_inff(), den = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int b0 = 0; b0 < nu; b0 += CH) {
    float2 ml[CH];
    float4 po[CH][NV];
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      if (b0 + q < nu) {
        const int64_t r = (int64_t)(b0 + q) * stride + row;
        ml[q] = *reinterpret_cast<const float2*>(a.ws_ml + r * 2);
#pragma unroll
        for (int v = 0; v < NV; ++v)
          po[q][v] = *reinterpret_cast<const float4*>(a.ws_o + r * D + c0 + 4 * v);
      }
    }
    float Mn = M;
#pragma unroll
    for (int q = 0; q < CH; ++q)
      if (b0 + q < nu) Mn = fmaxf(Mn, ml[q].x);
    // a split no row position reaches has m = -inf and weight 0
    const float rescale = M == -__builtin_inff() ? 0.f : fast_exp2(M - Mn);
    den *= rescale;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= rescale;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      if (b0 + q < nu) {
        const float w = fast_exp2(ml[q].x - Mn);
        den += w * ml[q].y;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          acc[4 * v] += w * po[q][v].x;
          acc[4 * v + 1] += w * po[q][v].y;
          acc[4 * v + 2] += w * po[q][v].z;
          acc[4 * v + 3] += w * po[q][v].w;
        }
      }
    }
    M = Mn;
  }
  const float inv = 1.f / den;
  float res[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) res[e] = acc[e] * inv;
  store_out_vec<EPL>(a.out, a.out_dt, row * D + c0, res);
}

// fp32 KV: one wave per (query token, KV head); each lane owns D/64 elements
// of every head of the group and the wave walks the visible tokens one by one,
// keeping the softmax's running sums in fp64 (a parity path for fp32 pools:
// the 1e-5 bound must hold over contexts of thousands of tokens).
template <int D, int GMAX>
__global__ __launch_bounds__(64) void prefill_f32_kernel(const PrefillArgs a) {
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x;
  const int row = blockIdx.x / a.Hkv;
  const int kvh = blockIdx.x % a.Hkv;
  int lo = 0, hi = a.S;  // sequence of this row: last s with cu[s] <= row
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_at(a, mid) <= row) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int q0 = cu_at(a, s);
  const int Qs = cu_at(a, s + 1) - q0;
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
    float q[GMAX][EPL], m[GMAX];
    double acc[GMAX][EPL], l[GMAX];
    for (int g = 0; g < GMAX; ++g) {
      m[g] = -__builtin_inff();
      l[g] = 0.0;
      for (int e = 0; e < EPL; ++e) {
        q[g][e] = g < gn ? qrow[(int64_t)(g0 + g) * D + lane * EPL + e] : 0.f;
        acc[g][e] = 0.0;
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
        // the scale enters the exponent through one fma (raw * scale - max), so
        // a large score is not rounded before the max is taken off
        const float mn = fmaxf(m[g], z * a.scale_log2);
        const float alpha = fast_exp2(m[g] - mn);
        const float p = fast_exp2(__builtin_fmaf(z, a.scale_log2, -mn));
        // running sums in fp64: over thousands of tokens the fp32 rounding of
        // a token-by-token sum reaches 1e-5 of a sharp softmax's output
        l[g] = l[g] * alpha + p;
        for (int e = 0; e < EPL; ++e) acc[g][e] = acc[g][e] * alpha + (double)p * vv[e];
        m[g] = mn;
      }
    }
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
      for (int e = 0; e < EPL && g < gn; ++e)
        store_out(a.out, a.out_dt, ((int64_t)row * a.Hq + (int64_t)kvh * G + g0 + g) * D + lane * EPL + e,
                  (float)(acc[g][e] / l[g]));
  }
}

template <int DT, int D, bool F8, bool NARROW = false>
pkv_status launch_tile(const PrefillArgs& a, hipStream_t stream) {
  constexpr int TW = tile_waves(D, F8, NARROW);
  constexpr int RW = TW * 16 * kTileQB;
  const int G = a.Hq / a.Hkv;
  const int TQ = RW / G;
  const int64_t nqt = (a.max_query_len + TQ - 1) / TQ;
  const int64_t grid = nqt * a.S * a.Hkv * a.n_split;
  if (grid == 0) return PKV_OK;
  if (grid > 0x7fffffff) return fail(PKV_ERR_UNSUPPORTED, "prefill grid too large");
  hipLaunchKernelGGL((prefill_tile_kernel<DT, D, F8, NARROW>), dim3((unsigned)grid), dim3(64 * TW), 0,
                     stream, a);
  pkv_status st = check_launch("paged_attention_prefill");
  if (st != PKV_OK || a.n_split <= 1) return st;
  const int64_t mgrid = ((int64_t)a.Tq * a.Hq + 15) / 16;  // 16 rows per workgroup
  if (mgrid > 0x7fffffff) return fail(PKV_ERR_UNSUPPORTED, "prefill merge grid too large");
  hipLaunchKernelGGL((prefill_merge_kernel<D, RW>), dim3((unsigned)mgrid), dim3(256), 0, stream, a);
  return check_launch("paged_attention_prefill (merge)");
}

// Whether the tile kernel can stage blocks of B tokens: a wave stages 64 / CPR
// consecutive rows per chunk (CPR = staging chunks per row: 16 for 16-bit
// D = 128, 8 for D = 64 and for FP8 codes, 16 of 8 bytes for the NARROW
// 16-bit D = 64 kernel) and they must lie in one block.  So B >= 4 for 16-bit
// pools, B >= 8 for FP8 (B <= 32 always).
bool tile_block_ok(int B, int /*D*/, bool fp8) { return B >= (fp8 ? 8 : 4); }

template <int DT, int D>
pkv_status launch_mfma(const PrefillArgs& a, hipStream_t stream) {
  // blocks of at least 16 tokens and groups that fit a workgroup: tile kernel
  if (tile_block_ok(a.B, D, false) && a.Hq / a.Hkv <= kWaves * 16 * kTileQB) {
    if constexpr (D == 64) {
      if (a.B == 4) return launch_tile<DT, D, false, true>(a, stream);
    }
    return launch_tile<DT, D, false>(a, stream);
  }
  const int G = a.Hq / a.Hkv;
  if (G > kRowsPerWG) return fail(PKV_ERR_UNSUPPORTED, "prefill: group size %d > %d", G, kRowsPerWG);
  const int TQ = kRowsPerWG / G;
  const int64_t nqt = (a.max_query_len + TQ - 1) / TQ;
  const int64_t grid = nqt * a.S * a.Hkv;
  if (grid == 0) return PKV_OK;
  if (grid > 0x7fffffff) return fail(PKV_ERR_UNSUPPORTED, "prefill grid too large");
  hipLaunchKernelGGL((prefill_mfma_kernel<DT, D, true>), dim3((unsigned)grid), dim3(kThreads), 0,
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

// Split plan.  A launch whose workgroups ((sequence, KV head) pairs x query
// tiles) would not fill the GPU with two per CU -- few sequences, e.g. one
// long prompt's chunk -- cuts every workgroup's KV range into splits of
// tiles_per_split tiles (at least kMinSplitTiles), up to two workgroups per
// CU in total: one round of resident workgroups.  (Four per CU, two rounds,
// measured 7-9% slower on single 256- to 1024-token chunks: twice the partial
// results to merge.)  Workgroups whose range fits one split write their rows
// directly; the others leave partial results for the merge kernel.
PrefillPlan plan_prefill(int kv_dt, int32_t S, int32_t Tq, int32_t max_query_len, int32_t Hq,
                         int32_t Hkv, int32_t D, int32_t B, int32_t max_ctx) {
  constexpr int kMinSplitTiles = 8;
  PrefillPlan p{1, 0, 0};
  const int G = Hkv > 0 ? Hq / Hkv : 0;
  const bool tile = kv_dt != DT_F32 && tile_block_ok(B, D, kv_dt == DT_FP8) && G >= 1 &&
                    G <= kWaves * 16 * kTileQB;
  if (!tile || S <= 0 || Tq <= 0 || max_query_len <= 0 || max_ctx <= 0) return p;
  const int TW = tile_waves(D, kv_dt == DT_FP8, false);  // the NARROW kernel runs 4 as well
  const int TQ = TW * 16 * kTileQB / G;
  const int64_t grid0 = (int64_t)((max_query_len + TQ - 1) / TQ) * S * Hkv;
  const int max_tiles = (max_ctx + kTileKV - 1) / kTileKV;
  // eight waves per CU: two 4-wave workgroups or one 8-wave workgroup (a
  // size query with no device to ask plans for the whole 256-CU gfx950)
  const int cu = device_cu_count();
  const int64_t target = (8 / TW) * (int64_t)(cu > 0 ? cu : 256);
  if (grid0 >= target) return p;
  int ns = (int)std::min<int64_t>((target + grid0 - 1) / grid0, std::max(1, max_tiles / kMinSplitTiles));
  if (ns <= 1) return p;
  const int tps = (max_tiles + ns - 1) / ns;
  ns = (max_tiles + tps - 1) / tps;
  if (ns <= 1) return p;
  p.n_split = ns;
  p.tiles_per_split = tps;
  p.workspace_bytes = (size_t)ns * Tq * Hq * (D + 2) * sizeof(float);
  return p;
}

pkv_status launch_prefill(int kv_dt, const PrefillArgs& a, hipStream_t stream) {
  if (kv_dt == DT_FP8) {
    // FP8 pools: the tile kernel only (blocks of >= 8 tokens, groups that fit
    // a workgroup), q in f16 or bf16
    if (!tile_block_ok(a.B, a.D, true) || a.Hq / a.Hkv > kWaves * 16 * kTileQB)
      return fail(PKV_ERR_UNSUPPORTED, "prefill_fp8: block_size %d / group %d", a.B, a.Hq / a.Hkv);
    if (a.q_dt == DT_BF16 && a.D == 128) return launch_tile<DT_BF16, 128, true>(a, stream);
    if (a.q_dt == DT_BF16 && a.D == 64) return launch_tile<DT_BF16, 64, true>(a, stream);
    if (a.q_dt == DT_F16 && a.D == 128) return launch_tile<DT_F16, 128, true>(a, stream);
    if (a.q_dt == DT_F16 && a.D == 64) return launch_tile<DT_F16, 64, true>(a, stream);
    return fail(PKV_ERR_UNSUPPORTED, "prefill_fp8: q dtype %d, head_dim %d", a.q_dt, a.D);
  }
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
