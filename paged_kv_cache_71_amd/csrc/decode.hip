// decode.hip -- paged attention for one query token per sequence (decode).
//
// What is computed (CS349D lecture 3 sec. 3.2; CMU 11-868 lecture 24 sec. 3.2):
// for every sequence s and query head h, softmax attention of q[s,h] over the
// sequence's context_lens[s] cached tokens, whose K/V rows are reached through
// the block table (physical = table[s][t / B], row t % B).  Scores are computed
// block by block and merged with an online (running-max) softmax; nothing is
// gathered into a contiguous buffer.  GQA: query head h reads KV head
// h / (Hq / Hkv) ("LLM inference, part 3: single node", ch. 9 sec. 1).
//
// Design (gfx950; decode is HBM-bound, every valid K/V row is read once):
//  * Work unit = a "tile" of TILE consecutive tokens of one row, a row being
//    (sequence, KV head, chunk of GC query heads).  All tiles of all rows are
//    numbered in one flat sequence and split into equal contiguous ranges, one
//    per wave of a persistent grid sized to the resident capacity of the GPU
//    (stream-K style).  Every wave therefore streams the same number of bytes
//    whatever the length mix (log-normal lengths would otherwise leave a long
//    tail), and no workgroup is launched without work.
//  * Each workgroup first turns context_lens into a prefix sum of tile counts
//    in LDS; a wave finds its first tile by binary search, then walks rows.
//  * A row that lies entirely inside one wave's range is finished by that wave
//    (output written directly, in any output dtype).  A row cut by range
//    boundaries leaves partial (max, sum, acc) states -- at most two per wave,
//    in fixed slots -- merged by a second small kernel in a fixed order.  Each
//    wave also records the row that its start cuts first, so the merge kernel
//    runs one wave per range boundary and finds its row with one load; rows
//    with nothing to attend get their zero output from the split kernel.  The
//    cut points depend only on the context lengths, so results are
//    bit-identical under any physical placement or aliasing of blocks.
//  * A token row of one KV head is D * elem bytes contiguous (256 B for bf16
//    D = 128); LPR lanes cover it with 16-byte loads, so one wave-load reads RPW
//    complete rows.  A tile is 4 such loads of K and 4 of V (8 KiB for bf16).
//  * Software pipeline: the loads of the next tile are issued before the
//    current tile is computed, and the table entries of the tile after that
//    are fetched with scalar loads.  Loads are never predicated: rows past the
//    context are clamped to the last valid row (always inside the same block)
//    and masked by selection afterwards, so the compiler can wait for exactly
//    one tile (vmcnt) instead of draining the queue.
//  * Each K/V load serves all GC query heads of the group (GQA reuse in
//    registers).  Matrix-core path (16-bit q, D = 128, groups of 4, 8 or 16
//    query heads, B >= 4; the Llama-3-8B batch): q . k on
//    v_mfma_f32_16x16x32 with the row's query heads as the 16 columns, P . V
//    on v_mfma_f32_16x16x16 over V staged per wave in LDS and read transposed
//    (ds_read_b64_tr_b16), three tiles in flight per wave.  Vector path (the
//    rest): the packed dot2 instructions for 16-bit KV (exact products, fp32
//    accumulation), then a DPP butterfly over the LPR lanes of the row.
//    Scores are kept in log2 units (scale * log2 e), and the accumulator is
//    rescaled only when some lane's running max grows (a wave vote), which is
//    bit-identical to rescaling by exp2(0) = 1 every tile.
//  * Rows past context_lens[s] and table entries past the last block are never
//    used (clamped loads read valid rows only), so stale or poisoned memory
//    there cannot reach the output.
//  * FP8 pools ("LLM inference, part 3", ch. 10): the F8 instantiations keep
//    every lane's element assignment of the 16-bit path with one code byte
//    per element, so a tile costs half the HBM bytes (on the matrix-core path
//    K codes come in 16-byte loads in a head-dimension order that q shares,
//    V codes in 16-byte loads restaged through LDS); the codes are widened
//    exactly in registers (gfx950 conversions) right before use, the K scale
//    of the row's KV head is folded into the score scale and the V scale
//    into the finished accumulator.
#include <atomic>
#include <type_traits>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLoadsPerTile = 4;
constexpr int kMaxSeqPerLaunch = 4096;  // LDS prefix capacity (sequences per launch)
constexpr int kMergeThreads = 256;
constexpr int kMaxGrid = 2048;          // workgroups of one split launch (8192 waves)
// s_waitcnt immediate: vector memory count 0, export and LDS/scalar counts
// left at their maxima (no wait on them)
constexpr int kWaitVmcnt0 = 0x0F70;

// DPP control words (row = 16 lanes).
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i within 16
constexpr int kDppRowRor8 = 0x128;       // lane i <- lane (i+8) mod 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// The two halves of a lane-pair exchange at lane distance 16 or 32 (gfx950
// permlane swaps): every lane receives (value of the lower partner, value of
// the upper partner), so a symmetric combine gives both partners the same bits.
template <int OFF>
__device__ __forceinline__ void pair_halves(float x, float& lo, float& hi) {
  static_assert(OFF == 16 || OFF == 32, "pair distance");
  const unsigned u = __float_as_uint(x);
  if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  }
}

// Sum over the LPR consecutive lanes that hold one token row; every lane of the
// row receives the same (bit-identical) total.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "row width");
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  if constexpr (LPR >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (LPR >= 32) {
    float lo, hi;
    pair_halves<16>(x, lo, hi);
    x = lo + hi;
  }
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// q . k over the 16 bytes one lane holds (8 x 16-bit or 4 x fp32 elements).
template <int DT>
__device__ __forceinline__ float dot16(const uint4 k, const uint4 q) {
  if constexpr (DT == DT_BF16) {
    float a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.x),
                                              __builtin_bit_cast(bf16x2_t, q.x), 0.f, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.y),
                                        __builtin_bit_cast(bf16x2_t, q.y), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.z),
                                        __builtin_bit_cast(bf16x2_t, q.z), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.w),
                                        __builtin_bit_cast(bf16x2_t, q.w), a, false);
    return a;
  } else if constexpr (DT == DT_F16) {
    float a = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, k.x),
                                     __builtin_bit_cast(f16x2_t, q.x), 0.f, false);
    a = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, k.y), __builtin_bit_cast(f16x2_t, q.y),
                               a, false);
    a = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, k.z), __builtin_bit_cast(f16x2_t, q.z),
                               a, false);
    a = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, k.w), __builtin_bit_cast(f16x2_t, q.w),
                               a, false);
    return a;
  } else {
    float a = __uint_as_float(k.x) * __uint_as_float(q.x);
    a = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), a);
    a = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), a);
    a = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), a);
    return a;
  }
}

// Widen the 16 bytes of V one lane holds to fp32.
template <int DT>
__device__ __forceinline__ void widen16(const uint4 v, float* f) {
  if constexpr (DT == DT_BF16) {
    f[0] = bf16_lo_to_f32(v.x); f[1] = bf16_hi_to_f32(v.x);
    f[2] = bf16_lo_to_f32(v.y); f[3] = bf16_hi_to_f32(v.y);
    f[4] = bf16_lo_to_f32(v.z); f[5] = bf16_hi_to_f32(v.z);
    f[6] = bf16_lo_to_f32(v.w); f[7] = bf16_hi_to_f32(v.w);
  } else if constexpr (DT == DT_F16) {
    f[0] = f16_lo_to_f32(v.x); f[1] = f16_hi_to_f32(v.x);
    f[2] = f16_lo_to_f32(v.y); f[3] = f16_hi_to_f32(v.y);
    f[4] = f16_lo_to_f32(v.z); f[5] = f16_hi_to_f32(v.z);
    f[6] = f16_lo_to_f32(v.w); f[7] = f16_hi_to_f32(v.w);
  } else {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
}

__device__ __forceinline__ uint4 ld16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

// K/V stream loads: every byte is read once per call, so they are marked
// non-temporal (they do not displace reusable lines in the caches); measured
// 7% faster than plain loads on the Llama-3-8B batch, 19% with cold caches.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const char* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ld8_stream(const char* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}

// 8 OCP E4M3 codes (one lane's V load) -> 8 fp32 values, exact.
__device__ __forceinline__ void fp8x8_to_f32(const uint2 v, float* f) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(v.x, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(v.x, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(v.y, false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(v.y, true);
  f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
  f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// C += A B on the matrix cores, 16 x 16 x 32 with 16-bit operands (gfx950):
// lane l holds A[l % 16][8 (l / 16) + 0..7], B[8 (l / 16) + 0..7][l % 16] and
// receives C[4 (l / 16) + i][l % 16], i < 4.
template <int DT>
__device__ __forceinline__ f32x4_t mfma16(const uint4 a, const uint4 b, f32x4_t c) {
  if constexpr (DT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// C += A B on the matrix cores, 16 x 16 x 16 with 16-bit operands: lane l
// holds A[l % 16][4 (l / 16) + 0..3], B[4 (l / 16) + 0..3][l % 16] and
// receives C[4 (l / 16) + i][l % 16], i < 4.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
template <int DT>
__device__ __forceinline__ f32x4_t mfma16k16(const uint2 a, const uint2 b, f32x4_t c) {
  if constexpr (DT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}

// gfx950 transposed LDS read of 16-bit elements: within each 16-lane group,
// lane j addresses 4 consecutive elements; lane i receives element i % 4 of
// lanes 4k + i / 4 (k < 4).  Pointing lane j at row r0 + j / 4, column
// c0 + 4 (j % 4) of a row-major tile gives lane i the column c0 + i of rows
// r0 .. r0 + 3.
typedef short i16x4lds_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const char* p) {
  const i16x4lds_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4lds_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Two fp32 values -> one word of two 16-bit values of dtype DT (x low),
// round to nearest even; and the two halves of such a word back to fp32.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  if constexpr (DT == DT_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{x, y}), bf16x2_t));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{x, y}), f16x2_t));
}
template <int DT>
__device__ __forceinline__ float half_lo(uint32_t w) {
  if constexpr (DT == DT_BF16) return __uint_as_float(w << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)w);
}
template <int DT>
__device__ __forceinline__ float half_hi(uint32_t w) {
  if constexpr (DT == DT_BF16) return __uint_as_float(w & 0xffff0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

__device__ __forceinline__ int rfl(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Read-only view of device memory in the constant address space: a load from it
// with a wave-uniform address becomes a scalar (SMEM) load, which is counted
// apart from the vector loads of the K/V pipeline.
typedef const __attribute__((address_space(4))) int32_t cint32_t;
typedef const __attribute__((address_space(4))) float cfloat_t;

// Tile geometry of a (dtype, head_dim) pair.
template <int DT, int D>
struct Geo {
  static constexpr int ES = dt_bytes(DT);
  static constexpr int EPL = 16 / ES;      // elements per lane per load
  static constexpr int LPR = D * ES / 16;  // lanes per token row
  static constexpr int RPW = 64 / LPR;     // token rows per wave-load
  static constexpr int NLD = kLoadsPerTile;
  static constexpr int TILE = NLD * RPW;   // tokens per tile
};

template <bool V>
struct BoolTag {
  static constexpr bool value = V;
};
template <int V>
struct IntTag {
  static constexpr int value = V;
};
// f(IntTag<0>), f(IntTag<1>), ..., f(IntTag<N - 1>), in order
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(IntTag<N - 1>{});
  }
}

// Where a wave is in the flat tile sequence (all fields wave-uniform).
struct Cursor {
  int s;    // sequence
  int rho;  // row of the sequence: kv head * n_hchunks + head chunk
  int j;    // tile within the row
  int nt;   // tiles per row of this sequence
  int st;   // first token attended (0 unless a start per sequence is given)
  int L;    // context length of the sequence (one past the last token attended)
  int kvh;  // KV head of the row
  int h0;   // first query head of the row
  float zs; // FP8 pools: score scale of the row (softmax scale * log2 e * K scale)
  float vs; // FP8 pools: V scale of the row
};

// Split kernel.  UNI: every wave-load lies in one block (B >= RPW), so its
// table entry is one scalar; otherwise each lane looks up its own row's block.
// MF (16-bit KV, D = 128, a GQA group of 4 query heads, B >= 16, or 8 or 4 with
// two or four blocks per tile): q . k runs on
// the matrix cores; everything else as in the vector path (see below).
// F8: the pools hold E4M3 codes (DT is then the dtype of q and of the widened
// elements); the lane layout is DT's, with 8-byte instead of 16-byte loads.
// The two-waves-per-SIMD bound keeps the matrix-core results in ordinary
// VGPRs (no accumulation registers, hence no copies out of them before the
// softmax): FP8 decode 176 -> 173 us on the Llama-3-8B batch, bf16 unchanged.
// BPT: blocks per 16-token tile on the matrix-core path (1 for B >= 16, 2 for
// B = 8, 4 for B = 4)
template <int DT, int D, int GC, bool UNI, bool MF, bool F8, int BPT = 1>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_split_kernel(
    const DecodeArgs a) {
  using Gm = Geo<DT, D>;
  constexpr int ES = Gm::ES, EPL = Gm::EPL, LPR = Gm::LPR, RPW = Gm::RPW;
  constexpr int NLD = Gm::NLD, TILE = Gm::TILE;
  static_assert(!F8 || DT != DT_F32, "FP8 pools pair with a 16-bit q");
  constexpr int KS = F8 ? 1 : ES;   // bytes per cached element
  constexpr int LB = 16 * KS / ES;  // bytes of K or V per lane per load
  using KVT = std::conditional_t<F8, uint2, uint4>;
  static_assert(!MF || (DT != DT_F32 && D == 128 && (GC == 4 || GC == 8 || GC == 16) && UNI &&
                        TILE == 16),
                "matrix-core path: 16-bit q, D = 128, 4, 8 or 16 query heads, one block per tile");
  static_assert(BPT == 1 || (MF && (BPT == 2 || BPT == 4)), "several blocks per tile: matrix-core path");
  constexpr int QN = MF ? D / 32 : GC;  // q registers: k-steps of 32 (MF) or heads
  // tiles in flight per wave: three where the registers allow it
  constexpr int NBUF = (MF || GC <= 2) ? 3 : 2;

  __shared__ int sm_ps[kMaxSeqPerLaunch + 1];  // prefix of tile counts over sequences
  __shared__ int sm_len[kMaxSeqPerLaunch];     // tokens to attend per sequence
  __shared__ int sm_wsum[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = rfl(tid >> 6);
  const int row = lane / LPR;
  const int col = lane % LPR;
  const int S = a.S;
  const int R = a.rows_per_seq;

  // ---- prefix sum of per-sequence tile counts (R rows per sequence)
  {
    const int per = (S + kThreads - 1) / kThreads;
    const int b = min(S, tid * per);
    const int e = min(S, b + per);
    int local = 0;
    for (int i = b; i < e; ++i) {
      const int L = min(max(a.context_lens[i], 0), a.max_ctx);
      // tokens start .. L - 1 (start = 0 unless a start per sequence is given)
      const int n = a.seq_start ? max(L - a.seq_start[i], 0) : L;
      const int c = ((n + TILE - 1) / TILE) * R;
      sm_len[i] = n;
      sm_ps[i + 1] = c;
      local += c;
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == 63) sm_wsum[wave] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < wave; ++w) run += sm_wsum[w];
    if (tid == 0) sm_ps[0] = 0;
    for (int i = b; i < e; ++i) {
      run += sm_ps[i + 1];
      sm_ps[i + 1] = run;
    }
    __syncthreads();
    if (blockIdx.x == 0)
      for (int i = tid; i <= S; i += kThreads) a.ws_ps[i] = sm_ps[i];
  }

  // ---- decode step (16-bit pools, matrix-core path): the new tokens' K/V
  // rows go to their slots, one 16-byte chunk of K and one of V per thread and
  // round.  The first round is loaded here and stored when the wave is done
  // with its range, so neither its loads nor its stores hold up the tiles.
  // No wave of this launch reads those slots -- token L - 1 of every row is
  // taken from new_k/new_v (see issue) -- so the stores need no ordering
  // against the attention's loads.
  constexpr bool STEP = MF && !F8;
  const bool step_on = STEP && a.new_k != nullptr;  // uniform
  const int rc = a.Hkv * D * KS / 16;                // 16-byte chunks per token row
  const int n_items = step_on ? S * rc : 0;          // < 2^31 (checked on the host)
  const int gid = blockIdx.x * kThreads + tid;
  uint4 nk{}, nv{};
  int64_t nslot = -1;
  if (gid < n_items) {
    nslot = a.slot_mapping[gid / rc];
    nk = reinterpret_cast<const uint4*>(a.new_k)[gid];
    nv = reinterpret_cast<const uint4*>(a.new_v)[gid];
  }
  auto put_new_rows = [&]() __attribute__((always_inline)) {
    if (!step_on) return;
    uint4* const kw = static_cast<uint4*>(const_cast<void*>(a.k_cache));
    uint4* const vw = static_cast<uint4*>(const_cast<void*>(a.v_cache));
    auto put = [&](int i, int64_t slot, const uint4& k4, const uint4& v4) __attribute__((always_inline)) {
      if (slot >= 0 && slot < a.nslots) {
        const int64_t d = slot * rc + (i % rc);
        kw[d] = k4;
        vw[d] = v4;
      }
    };
    if (gid < n_items) put(gid, nslot, nk, nv);
    // (batches with more chunks than the grid has threads)
    const int nthreads = gridDim.x * kThreads;
    for (int i = gid + nthreads; i < n_items; i += nthreads)
      put(i, a.slot_mapping[i / rc], reinterpret_cast<const uint4*>(a.new_k)[i],
          reinterpret_cast<const uint4*>(a.new_v)[i]);
  };

  // sequences with nothing to attend: all-zero output, -inf log-sum-exp
  for (int i = blockIdx.x; i < S; i += gridDim.x) {
    if (rfl(sm_len[i]) != 0) continue;
    const int64_t ob = (int64_t)i * a.Hq * D;
    for (int j = tid; j < a.Hq * D; j += kThreads) store_out(a.out, a.out_dt, ob + j, 0.f);
    if (a.lse)
      for (int h = tid; h < a.Hq; h += kThreads) a.lse[(int64_t)i * a.Hq + h] = -__builtin_inff();
  }

  const int N = rfl(sm_ps[S]);
  const int NW = gridDim.x * kWaves;
  const int C = (N + NW - 1) / NW;
  // XCD-aware range order: workgroups are dispatched round-robin over the 8
  // XCDs (blockIdx % 8), so consecutive ranges -- neighbouring rows, e.g. the
  // samples of one prompt aliasing the same prefix blocks -- go to workgroups
  // of the same XCD and share its L2 (measured 3-5% faster on aliased batches,
  // neutral otherwise).
  const int nwg = gridDim.x;
  const int wg_rank = (nwg % 8 == 0) ? (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8 : blockIdx.x;
  const int w = wg_rank * kWaves + wave;
  const int x0 = w * C;
  const int x1 = min(x0 + C, N);
  if (x0 >= x1) {
    if (lane == 0) a.ws_rec[w] = make_int4(-1, 0, 0, 0);  // nothing cut here
    put_new_rows();
    return;
  }

  const int G = a.Hq / a.Hkv;
  const int nhc = a.n_hchunks;
  const int log2B = a.log2B;
  const int bmask = a.B - 1;
  const int64_t row_stride = (int64_t)a.Hkv * D * KS;  // bytes between consecutive slots
  const int64_t blk_stride = row_stride * a.B;
  const int row_stride32 = (int)row_stride;  // B * row_stride < 2^31 (checked on the host)
  const char* const kpool = static_cast<const char*>(a.k_cache);
  const char* const vpool = static_cast<const char*>(a.v_cache);
  const float c_scale = a.scale_log2;  // softmax scale * log2(e): scores in log2 units

  auto set_row = [&](Cursor& c) __attribute__((always_inline)) {
    c.kvh = c.rho / nhc;
    c.h0 = c.kvh * G + (c.rho - c.kvh * nhc) * GC;
    if constexpr (F8) {  // scalar loads (uniform address, constant space)
      c.zs = c_scale * ((cfloat_t*)a.k_scale)[c.kvh];
      c.vs = ((cfloat_t*)a.v_scale)[c.kvh];
    }
  };
  auto set_seq = [&](Cursor& c) __attribute__((always_inline)) {
    const int n = rfl(sm_len[c.s]);
    c.st = a.seq_start ? ((cint32_t*)a.seq_start)[c.s] : 0;  // scalar load, uniform
    c.L = c.st + n;
    c.nt = (n + TILE - 1) / TILE;
  };
  auto advance = [&](Cursor c) __attribute__((always_inline)) -> Cursor {
    if (++c.j == c.nt) {
      c.j = 0;
      if (++c.rho == R) {
        c.rho = 0;
        do {
          ++c.s;
        } while (c.s + 1 < S && rfl(sm_len[c.s]) == 0);
        set_seq(c);
      }
      set_row(c);
    }
    return c;
  };

  // locate x0: the largest s with ps[s] <= x0 (then ps[s + 1] > x0)
  Cursor c0;
  {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (rfl(sm_ps[mid]) <= x0) lo = mid;
      else hi = mid - 1;
    }
    c0.s = lo;
    set_seq(c0);
    const int u = x0 - rfl(sm_ps[lo]);
    c0.rho = u / c0.nt;
    c0.j = u - c0.rho * c0.nt;
    set_row(c0);
  }
  // the merge kernel's work list: x0 cuts the row holding it when the row
  // starts earlier (j > 0); the row is listed at its first cut only, the one
  // whose previous boundary x0 - C lies at or before the row's start
  if (lane == 0)
    a.ws_rec[w] = c0.j > 0 && c0.j <= C ? make_int4(c0.s * R + c0.rho, x0 - c0.j, c0.nt, C)
                                        : make_int4(-1, 0, 0, 0);

  // table entries of a tile: one per wave-load (UNI) -- scalar loads
  struct Ent {
    int e[NLD];
  };
  auto entries = [&](const Cursor& c) __attribute__((always_inline)) -> Ent {
    Ent r;
    if constexpr (MF) {
      const cint32_t* tb = (const cint32_t*)(a.block_tables + (int64_t)c.s * a.max_nb);
      r.e[0] = tb[(c.st + c.j * TILE) >> log2B];
#pragma unroll
      for (int i = 1; i < NLD; ++i) r.e[i] = r.e[0];
      // blocks of 8 or 4: the blocks of the tile's later 8- or 4-token parts
      // (clamped to the last token, so a clamped row finds the block holding it)
#pragma unroll
      for (int k = 1; k < BPT; ++k) r.e[k] = tb[min(c.st + c.j * TILE + k * (TILE / BPT), c.L - 1) >> log2B];
    } else if constexpr (UNI) {
      const cint32_t* tb = (const cint32_t*)(a.block_tables + (int64_t)c.s * a.max_nb);
      const int ts = c.st + c.j * TILE;
#pragma unroll
      for (int i = 0; i < NLD; ++i) r.e[i] = tb[min(ts + i * RPW, c.L - 1) >> log2B];
    } else {
#pragma unroll
      for (int i = 0; i < NLD; ++i) r.e[i] = 0;
    }
    return r;
  };

  // K/V loads of one tile; rows past the context read the last valid row
  auto ldkv = [&](const char* p) __attribute__((always_inline)) -> KVT {
    if constexpr (F8) return ld8_stream(p);
    else return ld16_stream(p);
  };
  auto issue = [&](const Cursor& c, const Ent& en, KVT (&kb)[NLD], KVT (&vb)[NLD]) __attribute__((always_inline)) {
    const int ts = c.st + c.j * TILE;
    const int head_off = c.kvh * D * KS + col * LB;
    if constexpr (MF) {
      // the whole tile lies in one block.  K as the MFMA A operand: lane l
      // holds token l % 16, elements 32 kk + 8 (l / 16) .. + 7.  V rows as in
      // the vector path but with token 4 * row + i in load i, which is where
      // the MFMA result leaves that token's scores.
      // wave-uniform; unsigned 32 x 32 -> 64 bits: block ids are >= 0 and a
      // block is under 2 GiB (checked on the host)
      const uint64_t base = (uint64_t)(uint32_t)en.e[0] * (uint32_t)blk_stride;
      // blocks of 8 or 4 tokens: a load's token t (already clamped) lies in
      // the block of entry (t - ts) >> log2 B -- a per-lane choice of base
      [[maybe_unused]] const uint64_t base1 = (uint64_t)(uint32_t)en.e[1] * (uint32_t)blk_stride;
      [[maybe_unused]] const uint64_t base2 = (uint64_t)(uint32_t)en.e[2] * (uint32_t)blk_stride;
      [[maybe_unused]] const uint64_t base3 = (uint64_t)(uint32_t)en.e[3] * (uint32_t)blk_stride;
      auto bsel = [&](int t) __attribute__((always_inline)) -> uint64_t {
        if constexpr (BPT == 2) {
          return t - ts >= 8 ? base1 : base;
        } else if constexpr (BPT == 4) {
          // two bit tests, so the choice stays in registers (selects)
          const int k = (t - ts) >> 2;
          const uint64_t lo = (k & 1) ? base1 : base;
          const uint64_t hi = (k & 1) ? base3 : base2;
          return (k & 2) ? hi : lo;
        } else {
          return base;
        }
      };
      const int kvoff = c.kvh * D * KS;
      const int tk = min(ts + col, c.L - 1);
      if constexpr (F8) {
        // FP8: lane (token col, group row) takes the 32 contiguous codes
        // 32 row .. 32 row + 31 of its token in two 16-byte loads; k-step kk
        // uses codes 32 row + 8 kk .. + 7 (q is loaded with the same order).
        // Each load instruction then reads half of every token's 128-byte
        // line instead of a quarter: half the cache-line requests.
        const unsigned koff = (unsigned)((tk & bmask) * row_stride32 + kvoff + row * 32);
        const uint64_t kbase = bsel(tk);
        const uint4 k0 = ld16_stream(kpool + kbase + koff);
        const uint4 k1 = ld16_stream(kpool + kbase + koff + 16);
        kb[0] = make_uint2(k0.x, k0.y);
        kb[1] = make_uint2(k0.z, k0.w);
        kb[2] = make_uint2(k1.x, k1.y);
        kb[3] = make_uint2(k1.z, k1.w);
      }
      if constexpr (F8) {
        // FP8 V goes through LDS, so its load layout is free: two 16-byte
        // loads per lane, lane (row, col) taking codes 16 (col % 8) .. + 15 of
        // token 8 j + 2 row + col / 8 (whole 128-byte rows per 8 lanes)
#pragma unroll
        for (int jv = 0; jv < 2; ++jv) {
          const int tv = min(ts + 8 * jv + 2 * row + (col >> 3), c.L - 1);
          const unsigned voff = (unsigned)((tv & bmask) * row_stride32 + kvoff + (col & 7) * 16);
          const uint4 v4 = ld16_stream(vpool + bsel(tv) + voff);
          vb[2 * jv] = make_uint2(v4.x, v4.y);
          vb[2 * jv + 1] = make_uint2(v4.z, v4.w);
        }
      } else {
        // SUB: the tile holding token L - 1 of a decode step, whose K/V row
        // comes from new_k/new_v (lanes that would read it, clamped rows
        // included, read it there; a per-lane choice of address)
        auto ld16 = [&](auto sub_tag) __attribute__((always_inline)) {
          constexpr bool SUB = decltype(sub_tag)::value;
          const unsigned koff = (unsigned)((tk & bmask) * row_stride32 + kvoff + row * LB);
          const char* kp = kpool + bsel(tk) + koff;
          if constexpr (SUB) {
            if (tk == c.L - 1)
              kp = static_cast<const char*>(a.new_k) + (int64_t)c.s * row_stride + kvoff + row * LB;
          }
#pragma unroll
          for (int kk = 0; kk < NLD; ++kk) kb[kk] = ldkv(kp + kk * 4 * LB);
#pragma unroll
          for (int i = 0; i < NLD; ++i) {
            const int tv = min(ts + 4 * row + i, c.L - 1);
            const unsigned voff = (unsigned)((tv & bmask) * row_stride32 + kvoff + col * LB);
            const char* vp = vpool + bsel(tv) + voff;
            if constexpr (SUB) {
              if (tv == c.L - 1)
                vp = static_cast<const char*>(a.new_v) + (int64_t)c.s * row_stride + kvoff + col * LB;
            }
            vb[i] = ldkv(vp);
          }
        };
        if (step_on && c.j == c.nt - 1) ld16(BoolTag<true>{});
        else ld16(BoolTag<false>{});
      }
    } else if constexpr (UNI) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int tok = min(ts + i * RPW + row, c.L - 1);
        const uint64_t base = (uint64_t)(uint32_t)en.e[i] * (uint32_t)blk_stride;  // as above
        const unsigned off = (unsigned)((tok & bmask) * row_stride32 + head_off);
        kb[i] = ldkv(kpool + base + off);
        vb[i] = ldkv(vpool + base + off);
      }
    } else {
      const int32_t* tb = a.block_tables + (int64_t)c.s * a.max_nb;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int tok = min(ts + i * RPW + row, c.L - 1);
        const int ph = tb[tok >> log2B];
        const int64_t off =
            (int64_t)ph * blk_stride + (int64_t)(tok & bmask) * row_stride + head_off;
        kb[i] = ldkv(kpool + off);
        vb[i] = ldkv(vpool + off);
      }
    }
  };

  auto load_q = [&](const Cursor& c, uint4 (&qv)[QN]) __attribute__((always_inline)) {
    if constexpr (MF) {
      // q^T as the MFMA B operand, the GC heads repeated across the 16
      // columns: lane l holds head (l % 16) % GC, elements 32 kk + 8 (l / 16) ..
      // (FP8 pools: elements 32 (l / 16) + 8 kk .., the order of the K loads)
      const char* qp = static_cast<const char*>(a.q) +
                       (((int64_t)c.s * a.Hq + c.h0 + (col % GC)) * D) * ES + row * (F8 ? 64 : 16);
#pragma unroll
      for (int kk = 0; kk < QN; ++kk) qv[kk] = ld16(qp + kk * (F8 ? 16 : 64));
    } else {
      const char* qp = static_cast<const char*>(a.q) +
                       (((int64_t)c.s * a.Hq + c.h0) * D) * ES + col * 16;
#pragma unroll
      for (int g = 0; g < GC; ++g) qv[g] = ld16(qp + (int64_t)g * D * ES);
    }
  };

  // online-softmax state of this lane's token row (m: running max of the
  // scaled scores, log2 units)
  // Matrix-core path: one query column per lane (col % GC), m and l of that
  // column, and oacc[db][i] = output element 16 db + 4 row + i of the column.
  constexpr int NS = MF ? 1 : GC;
  float m[NS], l[NS], acc[MF ? 1 : GC][EPL];
  f32x4_t oacc[MF ? D / 16 : 1];
  auto reset_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < NS; ++g) {
      m[g] = -__builtin_inff();
      l[g] = 0.f;
    }
    if constexpr (MF) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
      for (int g = 0; g < GC; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }
  };
  // Matrix-core path: this wave's rows of LDS, the V tile (16 tokens x D,
  // 16-bit) staged for transposed reads; rows padded by 32 bytes so the four
  // rows one read touches fall on distinct banks.
  constexpr int kVP = D * 2 + 32;
  __shared__ __attribute__((aligned(16))) char sm_v[MF ? kWaves * 16 * kVP : 16];
  char* const vs = sm_v + (MF ? wave * 16 * kVP : 0);

  // One tile.  FULL: every row of the tile is a valid token.
  // K as 16-bit elements and V as fp32 (FP8 codes widened exactly)
  auto kfrag = [&](const KVT& x) __attribute__((always_inline)) -> uint4 {
    if constexpr (F8) return fp8x8_to16<DT>(x);
    else return x;
  };
  auto vwiden = [&](const KVT& x, float* vf) __attribute__((always_inline)) {
    if constexpr (F8) fp8x8_to_f32(x, vf);
    else widen16<DT>(x, vf);
  };
  auto compute = [&](const Cursor& c, const uint4 (&qv)[QN], const KVT (&kb)[NLD],
                     const KVT (&vb)[NLD], auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int ts = c.st + c.j * TILE;
    float zsc;
    if constexpr (F8) zsc = c.zs;
    else zsc = c_scale;
    if constexpr (MF) {
      // S = K q^T on the matrix cores: lane (row, col) receives the scores of
      // tokens 4 * row + i (i < 4) for query column col (head h0 + col % GC).
      // The running max m[0] of the column is shared by its four lanes (max
      // over the 16 tokens of the tile, across lane rows); l[0] is this lane's
      // partial sum over its 4 tokens.
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NLD; ++kk) sacc = mfma16<DT>(kfrag(kb[kk]), qv[kk], sacc);
      float z[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float zz = sacc[i] * zsc;
        if constexpr (FULL) z[i] = zz;
        else z[i] = (ts + 4 * row + i < c.L) ? zz : -__builtin_inff();
      }
      float t = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      float lo, hi;
      pair_halves<16>(t, lo, hi);
      t = fmaxf(lo, hi);
      pair_halves<32>(t, lo, hi);
      t = fmaxf(lo, hi);
      const float mn = fmaxf(m[0], t);  // finite: a tile holds at least one valid token
      if (__builtin_amdgcn_ballot_w64(mn > m[0])) {
        const float alpha = fast_exp2(m[0] - mn);  // this lane's own column
        l[0] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) oacc[db] *= alpha;
        m[0] = mn;
      }
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pe = fast_exp2(z[i] - m[0]);
        if constexpr (FULL) p[i] = pe;
        else p[i] = (ts + 4 * row + i < c.L) ? pe : 0.f;
      }
      l[0] += (p[0] + p[1]) + (p[2] + p[3]);
      // O^T += V^T P^T on the matrix cores (16 x 16 x 16 per 16 output
      // elements): B = P^T is this lane's p (tokens 4 row + j, column col), in
      // hi + lo 16-bit parts (about 16 significant bits); A = V^T comes from
      // the tile staged in LDS through transposed reads.
      const uint32_t h01 = pack2<DT>(p[0], p[1]), h23 = pack2<DT>(p[2], p[3]);
      const uint2 ph = make_uint2(h01, h23);
      const uint2 pl = make_uint2(pack2<DT>(p[0] - half_lo<DT>(h01), p[1] - half_hi<DT>(h01)),
                                  pack2<DT>(p[2] - half_lo<DT>(h23), p[3] - half_hi<DT>(h23)));
      // (the wave's own LDS rows, written and read in order by this wave only)
      if constexpr (F8) {
#pragma unroll
        for (int jv = 0; jv < 2; ++jv) {
          char* dst = vs + (8 * jv + 2 * row + (col >> 3)) * kVP + (col & 7) * 32;
          *reinterpret_cast<uint4*>(dst) = kfrag(vb[2 * jv]);
          *reinterpret_cast<uint4*>(dst + 16) = kfrag(vb[2 * jv + 1]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NLD; ++i)
          *reinterpret_cast<uint4*>(vs + (4 * row + i) * kVP + col * 16) = kfrag(vb[i]);
      }
      const char* vrd = vs + (4 * row + (col >> 2)) * kVP + (col & 3) * 8;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const uint2 va = lds_read_tr16(vrd + db * 32);
        oacc[db] = mfma16k16<DT>(va, ph, oacc[db]);
        oacc[db] = mfma16k16<DT>(va, pl, oacc[db]);
      }
      return;
    }
    float z[NLD][GC];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const uint4 kx = kfrag(kb[i]);
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        const float zz = row_sum<LPR>(dot16<DT>(kx, qv[g])) * zsc;
        if constexpr (FULL) z[i][g] = zz;
        else z[i][g] = (ts + i * RPW + row < c.L) ? zz : -__builtin_inff();
      }
    }
    float mn[GC];
    bool grow = false;
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      float t = z[0][g];
#pragma unroll
      for (int i = 1; i < NLD; ++i) t = fmaxf(t, z[i][g]);
      mn[g] = fmaxf(m[g], t);
      grow |= mn[g] > m[g];
    }
    // Rescale only when some lane's max grew: otherwise the factor would be
    // exp2(0) = 1 exactly, so skipping it changes no bit.
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        // a lane row with no valid token yet keeps m = -inf and zero state
        const float alpha = mn[g] == -__builtin_inff() ? 1.f : fast_exp2(m[g] - mn[g]);
        l[g] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
        m[g] = mn[g];
      }
    }
    float p[NLD][GC];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const float pe = fast_exp2(z[i][g] - m[g]);
        if constexpr (FULL) p[i][g] = pe;
        else p[i][g] = (ts + i * RPW + row < c.L) ? pe : 0.f;
        ps += p[i][g];
      }
      l[g] += ps;
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      float vf[EPL];
      vwiden(vb[i], vf);
#pragma unroll
      for (int g = 0; g < GC; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p[i][g], vf[e], acc[g][e]);
    }
  };

  // merge two lane-row states (symmetric, so both partners get the same bits)
  auto merge_pair = [&](float cm_a, float l_a, const float* acc_a, float cm_b, float l_b,
                        const float* acc_b, float& cm_o, float& l_o, float* acc_o) __attribute__((always_inline)) {
    const float M = fmaxf(cm_a, cm_b);
    const float mu = M == -__builtin_inff() ? 0.f : M;
    const float sa = fast_exp2(cm_a - mu);
    const float sb = fast_exp2(cm_b - mu);
    l_o = l_a * sa + l_b * sb;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc_o[e] = acc_a[e] * sa + acc_b[e] * sb;
    cm_o = M;
  };

  // finish the row of cursor c: merge the RPW lane rows, then write the output
  // (row complete in this wave) or a partial state (slot 2w: the row holding
  // x0, slot 2w+1: the row holding x1 - 1)
  auto epilogue = [&](const Cursor& c, int row_xb) __attribute__((always_inline)) {
    if constexpr (MF) {
      // the four lanes of a column share its running max: their partial sums
      // add up; the matrix cores already summed the accumulators over tokens
      float lo, hi;
      pair_halves<16>(l[0], lo, hi);
      pair_halves<32>(lo + hi, lo, hi);
      l[0] = lo + hi;  // total weight of column col
      const bool complete = row_xb >= x0 && row_xb + c.nt <= x1;
      if constexpr (F8) {
#pragma unroll
        for (int db = 0; db < D / 16; ++db) oacc[db] *= c.vs;
      }
      if (col < GC) {  // one of the identical copies of each query column
        if (complete) {
          const int64_t o = ((int64_t)c.s * a.Hq + c.h0 + col) * D + 4 * row;
          if (a.lse && row == 0) a.lse[(int64_t)c.s * a.Hq + c.h0 + col] = m[0] + __log2f(l[0]);
#pragma unroll
          for (int db = 0; db < D / 16; ++db) {
            const float r4[4] = {oacc[db][0] / l[0], oacc[db][1] / l[0], oacc[db][2] / l[0],
                                 oacc[db][3] / l[0]};
            store_out_vec<4>(a.out, a.out_dt, o + 16 * db, r4);
          }
        } else {
          const int slot = row_xb <= x0 ? 2 * w : 2 * w + 1;
          const int64_t o = ((int64_t)slot * GC + col) * D + 4 * row;
#pragma unroll
          for (int db = 0; db < D / 16; ++db)
            *reinterpret_cast<float4*>(a.ws_acc + o + 16 * db) =
                make_float4(oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]);
          if (row == 0)
            *reinterpret_cast<float2*>(a.ws_ml + ((int64_t)slot * GC + col) * 2) = make_float2(m[0], l[0]);
        }
      }
      reset_state();
    } else {
    if constexpr (LPR == 8) {
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        float accb[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) accb[e] = dpp<kDppRowRor8>(acc[g][e]);
        const float cmb = dpp<kDppRowRor8>(m[g]);
        const float lb = dpp<kDppRowRor8>(l[g]);
        merge_pair(m[g], l[g], acc[g], cmb, lb, accb, m[g], l[g], acc[g]);
      }
    }
    if constexpr (LPR <= 16) {
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        float a0[EPL], a1[EPL], c0v, c1v, l0, l1;
#pragma unroll
        for (int e = 0; e < EPL; ++e) pair_halves<16>(acc[g][e], a0[e], a1[e]);
        pair_halves<16>(m[g], c0v, c1v);
        pair_halves<16>(l[g], l0, l1);
        merge_pair(c0v, l0, a0, c1v, l1, a1, m[g], l[g], acc[g]);
      }
    }
    {
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        float a0[EPL], a1[EPL], c0v, c1v, l0, l1;
#pragma unroll
        for (int e = 0; e < EPL; ++e) pair_halves<32>(acc[g][e], a0[e], a1[e]);
        pair_halves<32>(m[g], c0v, c1v);
        pair_halves<32>(l[g], l0, l1);
        merge_pair(c0v, l0, a0, c1v, l1, a1, m[g], l[g], acc[g]);
      }
    }
    // A row lying inside this wave's range is final here and written
    // directly.  A row cut by the range leaves its state in slot 2w (the row
    // holding x0) or 2w + 1 (the row holding x1 - 1) for the merge kernel.
    if constexpr (F8) {  // V scale of the row's KV head (common to all its partial states)
#pragma unroll
      for (int g = 0; g < GC; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= c.vs;
    }
    const bool complete = row_xb >= x0 && row_xb + c.nt <= x1;
    if (complete) {
      if (a.lse && row == 0 && col == 0) {  // log2-sum-exp of the scaled scores, per head
#pragma unroll
        for (int g = 0; g < GC; ++g) a.lse[(int64_t)c.s * a.Hq + c.h0 + g] = m[g] + __log2f(l[g]);
      }
      if (row == 0) {
#pragma unroll
        for (int g = 0; g < GC; ++g) {
          const float lg = l[g];
          const int64_t o = ((int64_t)c.s * a.Hq + c.h0 + g) * D + col * EPL;
#pragma unroll
          for (int e = 0; e < EPL / 4; ++e) {
            const float r4[4] = {acc[g][4 * e] / lg, acc[g][4 * e + 1] / lg, acc[g][4 * e + 2] / lg,
                                 acc[g][4 * e + 3] / lg};
            store_out_vec<4>(a.out, a.out_dt, o + 4 * e, r4);
          }
        }
      }
    } else {
      const int slot = row_xb <= x0 ? 2 * w : 2 * w + 1;
      if (row == 0) {
#pragma unroll
        for (int g = 0; g < GC; ++g) {
          float4* dst = reinterpret_cast<float4*>(a.ws_acc + ((int64_t)slot * GC + g) * D + col * EPL);
#pragma unroll
          for (int e = 0; e < EPL / 4; ++e)
            dst[e] = make_float4(acc[g][4 * e], acc[g][4 * e + 1], acc[g][4 * e + 2], acc[g][4 * e + 3]);
        }
        if (col == 0) {
#pragma unroll
          for (int g = 0; g < GC; ++g)
            *reinterpret_cast<float2*>(a.ws_ml + ((int64_t)slot * GC + g) * 2) = make_float2(m[g], l[g]);
        }
      }
    }
    reset_state();
    }
  };

  using TrueT = BoolTag<true>;
  using FalseT = BoolTag<false>;

  reset_state();
  int row_xb = x0 - c0.j;  // flat index of the first tile of c0's row

  // compute tile x (cursor cc), then finish the row if it ends here.  last: x
  // is the wave's final tile (a constant false inside the main loop).  At a row
  // switch the next row's q is loaded (and waited for): once per row.
  auto finish = [&](int x, const Cursor& cc, const Cursor& cn, const KVT (&kbc)[NLD],
                    const KVT (&vbc)[NLD], uint4 (&qv)[QN], bool last) __attribute__((always_inline)) {
    if (!MF && cc.st + (cc.j + 1) * TILE <= cc.L) compute(cc, qv, kbc, vbc, TrueT{});
    else compute(cc, qv, kbc, vbc, FalseT{});  // (the matrix-core path always masks: 8 selects)
    if (last || cn.j == 0) {
      epilogue(cc, row_xb);
      if (!last) {
        load_q(cn, qv);
        // wait for q here, on this rare path: left pending it would make every
        // later tile wait as if it had just been loaded behind q
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        row_xb = x + 1;
      }
    }
  };

  // The K/V loads are never conditional and never overwrite a register with a
  // load in flight, so the compiler waits for exactly the tile being computed.
  // The main loop runs whole groups of NBUF steps with a single exit at the
  // bottom (no path reaches its header with a buffer set's loads unconsumed);
  // the last 1 .. NBUF tiles are peeled after it.  Cursors past the wave's last
  // tile repeat it (harmless reloads).
  uint4 qv[QN];
  load_q(c0, qv);
  // NBUF buffer sets: tiles x + 1 .. x + NBUF - 1 load while tile x is computed.
  KVT kb[NBUF][NLD], vb[NBUF][NLD];
  Cursor cs[NBUF];  // cs[k]: cursor of tile x + k
  cs[0] = c0;
  issue(cs[0], entries(cs[0]), kb[0], vb[0]);
#pragma unroll
  for (int k = 1; k < NBUF; ++k) {
    cs[k] = (x0 + k < x1) ? advance(cs[k - 1]) : cs[k - 1];
    if (k < NBUF - 1) issue(cs[k], entries(cs[k]), kb[k], vb[k]);
  }
  Ent en = entries(cs[NBUF - 1]);
  // Step U of a group: tile x + NBUF - 1 is issued into set (U + NBUF - 1) % NBUF,
  // then tile x (set U) is computed.
  auto step = [&](int x, auto u_tag, bool last) __attribute__((always_inline)) {
    constexpr int U = decltype(u_tag)::value;
    constexpr int I = (U + NBUF - 1) % NBUF;
    issue(cs[NBUF - 1], en, kb[I], vb[I]);
    const Cursor nx = (x + NBUF < x1) ? advance(cs[NBUF - 1]) : cs[NBUF - 1];
    en = entries(nx);
    finish(x, cs[0], cs[1], kb[U], vb[U], qv, last);
#pragma unroll
    for (int k = 0; k + 1 < NBUF; ++k) cs[k] = cs[k + 1];
    cs[NBUF - 1] = nx;
  };
  int x = x0;
  while (x1 - x > NBUF) {
    static_for<NBUF>([&](auto u) __attribute__((always_inline)) { step(x + decltype(u)::value, u, false); });
    x += NBUF;
  }
  const int r = x1 - x;  // 1 .. NBUF tiles left
  static_for<NBUF>([&](auto u) __attribute__((always_inline)) {
    constexpr int U = decltype(u)::value;
    if (U < r) step(x + U, u, U == r - 1);
  });
  put_new_rows();
}

// Merge: one wave per range boundary b = 1 .. n_waves - 1.  The split kernel's
// wave b recorded the row that its start cuts first (or nothing); that row's
// states lie in slot 2(b-1)+1 (or 2(b-1) when the row starts exactly at wave
// b-1's start) and then in slot 2w of each following wave w up to the one
// holding the row's last tile.  They are combined in wave order,
//   out = sum_w e^(m_w - M) acc_w / sum_w e^(m_w - M) l_w   (log2 units),
// in batches of CH states whose loads are issued together: one running max
// per batch, then each state's weight.  Lane l owns the NPL consecutive
// outputs from l * NPL on (all of one query head of the row).
template <int D, int GC>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(const DecodeArgs a) {
  constexpr int NPL = GC * D / 64;      // outputs per lane
  constexpr int CH = NPL <= 8 ? 8 : 2;  // states per batch (register budget)
  static_assert(NPL >= 1 && D % NPL == 0, "a lane's outputs belong to one head");
  const int b = blockIdx.x * (kMergeThreads / 64) + rfl(threadIdx.x >> 6) + 1;
  if (b >= a.n_waves) return;
  const int4 r = a.ws_rec[b];
  if (r.x < 0) return;
  const int lane = threadIdx.x & 63;
  const int R = a.rows_per_seq;
  const int s = r.x / R;
  const int rho = r.x - s * R;
  const int kvh = rho / a.n_hchunks;
  const int h0 = kvh * (a.Hq / a.Hkv) + (rho - kvh * a.n_hchunks) * GC;
  const int xb = r.y, nt = r.z, C = r.w;
  const int w0 = b - 1;                     // the wave holding the row's first tile
  const int ns = (xb + nt - 1) / C - w0 + 1;  // states of this row, in wave order
  auto slot_of = [&](int k) __attribute__((always_inline)) -> int {
    return k == 0 ? (xb != w0 * C ? 2 * w0 + 1 : 2 * w0) : 2 * (w0 + k);
  };
  const int j0 = lane * NPL;
  const int g = j0 / D;
  float M = -__builtin_inff(), den = 0.f, num[NPL];
#pragma unroll
  for (int e = 0; e < NPL; ++e) num[e] = 0.f;
  for (int b0 = 0; b0 < ns; b0 += CH) {
    float2 ml[CH];
    float av[CH][NPL];
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      if (b0 + q < ns) {
        const int64_t st = (int64_t)slot_of(b0 + q) * GC + g;
        ml[q] = *reinterpret_cast<const float2*>(a.ws_ml + st * 2);
        const float* src = a.ws_acc + st * D + (j0 - g * D);
        if constexpr (NPL % 4 == 0) {
#pragma unroll
          for (int e = 0; e < NPL; e += 4) {
            const float4 v4 = *reinterpret_cast<const float4*>(src + e);
            av[q][e] = v4.x;
            av[q][e + 1] = v4.y;
            av[q][e + 2] = v4.z;
            av[q][e + 3] = v4.w;
          }
        } else {
#pragma unroll
          for (int e = 0; e < NPL; ++e) av[q][e] = src[e];
        }
      }
    }
    float Mn = M;
#pragma unroll
    for (int q = 0; q < CH; ++q)
      if (b0 + q < ns) Mn = fmaxf(Mn, ml[q].x);
    const float rescale = M == -__builtin_inff() ? 0.f : fast_exp2(M - Mn);
    float d = den * rescale;
#pragma unroll
    for (int e = 0; e < NPL; ++e) num[e] *= rescale;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      if (b0 + q < ns) {
        const float wq = fast_exp2(ml[q].x - Mn);
        d += ml[q].y * wq;
#pragma unroll
        for (int e = 0; e < NPL; ++e) num[e] += av[q][e] * wq;
      }
    }
    M = Mn;
    den = d;
  }
  const int64_t o = ((int64_t)s * a.Hq + h0) * D + j0;
  float res[NPL];
#pragma unroll
  for (int e = 0; e < NPL; ++e) res[e] = num[e] / den;
  if constexpr (NPL % 8 == 0) {
#pragma unroll
    for (int e = 0; e < NPL; e += 8) store_out_vec<8>(a.out, a.out_dt, o + e, res + e);
  } else if constexpr (NPL == 4) {
    store_out_vec<4>(a.out, a.out_dt, o, res);
  } else {
#pragma unroll
    for (int e = 0; e < NPL; ++e) store_out(a.out, a.out_dt, o + e, res[e]);
  }
  if (a.lse && j0 % D == 0) a.lse[(int64_t)s * a.Hq + h0 + g] = M + __log2f(den);
}

// ---- host side -----------------------------------------------------------------

// (the caches below may be filled by several host threads at once: atomics,
// every writer stores the same value)
template <int DT, int D, int GC, bool UNI, bool MF, bool F8, int BPT = 1>
int occupancy_of() {
  static std::atomic<int> occ{-1};
  int o = occ.load(std::memory_order_relaxed);
  if (o < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(&decode_split_kernel<DT, D, GC, UNI, MF, F8, BPT>), kThreads,
            0) != hipSuccess ||
        n < 1)
      n = 1;
    occ.store(n, std::memory_order_relaxed);
    o = n;
  }
  return o;
}

// Split launch (one resident wave set: CUs x occupancy, capped by grid_cap)
// followed by the merge launch.
template <int DT, int D, int GC, bool UNI, bool MF, bool F8, int BPT = 1>
pkv_status launch_split(DecodeArgs a, int grid_cap, int ncu, hipStream_t stream, int* waves_only) {
  // Matrix-core path: one workgroup (one wave per SIMD, three tiles in
  // flight each) per CU measured fastest -- 3-7% ahead of two per CU on the
  // Llama-3-8B batch for 16-bit pools, 168.5 -> 163.8 us for FP8 pools (four
  // tiles in flight at one workgroup: 162-164 us; at two workgroups, 171).
  // Vector path: every resident workgroup.
  int64_t grid = (int64_t)ncu * (MF ? 1 : occupancy_of<DT, D, GC, UNI, MF, F8, BPT>());
  if (grid > grid_cap) grid = grid_cap;
  if (grid < 1) grid = 1;
  a.n_waves = (int)grid * kWaves;
  if (waves_only) {  // sizing pass: report the waves, launch nothing
    if (a.n_waves > *waves_only) *waves_only = a.n_waves;
    return PKV_OK;
  }
  hipLaunchKernelGGL((decode_split_kernel<DT, D, GC, UNI, MF, F8, BPT>), dim3((unsigned)grid),
                     dim3(kThreads), 0, stream, a);
  pkv_status st = check_launch("paged_attention_decode (split)");
  if (st != PKV_OK) return st;
  // one merge wave per range boundary (the first range has none)
  constexpr int kMergeWaves = kMergeThreads / 64;
  const int nb = a.n_waves - 1;
  hipLaunchKernelGGL((decode_merge_kernel<D, GC>), dim3((unsigned)((nb + kMergeWaves - 1) / kMergeWaves)),
                     dim3(kMergeThreads), 0, stream, a);
  return check_launch("paged_attention_decode (merge)");
}

template <int DT, int D, int GC, bool F8>
pkv_status launch_typed(const DecodeArgs& a, int grid_cap, int ncu, bool uni, hipStream_t stream,
                        int* waves_only) {
  // matrix cores: 16-bit q, D = 128, 4, 8 or 16 query heads per row, a tile in
  // one block (B >= 16), two (B = 8) or four (B = 4)
  if constexpr (DT != DT_F32 && D == 128 && (GC == 4 || GC == 8 || GC == 16)) {
    if (a.B >= 16)
      return launch_split<DT, D, GC, true, true, F8>(a, grid_cap, ncu, stream, waves_only);
    if (a.B == 8)
      return launch_split<DT, D, GC, true, true, F8, 2>(a, grid_cap, ncu, stream, waves_only);
    if (a.B == 4)
      return launch_split<DT, D, GC, true, true, F8, 4>(a, grid_cap, ncu, stream, waves_only);
  }
  if constexpr (GC == 16) {  // chunks of 16 heads exist on the matrix-core path only
    return fail(PKV_ERR_UNSUPPORTED, "decode: 16-head rows need the matrix-core path");
  } else {
    if (uni) return launch_split<DT, D, GC, true, false, F8>(a, grid_cap, ncu, stream, waves_only);
    return launch_split<DT, D, GC, false, false, F8>(a, grid_cap, ncu, stream, waves_only);
  }
}

template <int DT, int D, bool F8>
pkv_status launch_gc(const DecodeArgs& a, int grid_cap, int ncu, bool uni, hipStream_t stream,
                     int* waves_only) {
  switch (a.gc) {
    case 1: return launch_typed<DT, D, 1, F8>(a, grid_cap, ncu, uni, stream, waves_only);
    case 2: return launch_typed<DT, D, 2, F8>(a, grid_cap, ncu, uni, stream, waves_only);
    case 4: return launch_typed<DT, D, 4, F8>(a, grid_cap, ncu, uni, stream, waves_only);
    case 8: return launch_typed<DT, D, 8, F8>(a, grid_cap, ncu, uni, stream, waves_only);
    case 16: return launch_typed<DT, D, 16, F8>(a, grid_cap, ncu, uni, stream, waves_only);
  }
  return fail(PKV_ERR_UNSUPPORTED, "decode: head chunk %d", a.gc);
}

template <int DT, bool F8>
pkv_status launch_d(const DecodeArgs& a, int grid_cap, int ncu, bool uni, hipStream_t stream,
                    int* waves_only) {
  switch (a.D) {
    case 64: return launch_gc<DT, 64, F8>(a, grid_cap, ncu, uni, stream, waves_only);
    case 128: return launch_gc<DT, 128, F8>(a, grid_cap, ncu, uni, stream, waves_only);
  }
  return fail(PKV_ERR_UNSUPPORTED, "decode: head_dim %d", a.D);
}

// tokens per tile and token rows per wave-load of an instantiation
void tile_geometry(int kv_dt, int D, int* tile, int* rpw) {
  const int lpr = D * dt_bytes(kv_dt) / 16;
  *rpw = 64 / lpr;
  *tile = kLoadsPerTile * *rpw;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static std::atomic<int> cache[64];  // zero-initialised: not yet queried
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
  if (dev >= 0 && dev < 64 && n > 0) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

pkv_status plan_decode(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t /*B*/,
                       int32_t max_context_len, DecodePlan* plan) {
  const int G = Hq / Hkv;
  // query heads per row: the vector path takes the largest of 8, 4, 2 dividing
  // G (else 1); the matrix-core path the largest of 16, 8, 4 (else none)
  int gv = 1, gm = 0;
  for (int c : {8, 4, 2}) {
    if (G % c == 0) {
      gv = c;
      break;
    }
  }
  for (int c : {16, 8, 4}) {
    if (G % c == 0) {
      gm = c;
      break;
    }
  }
  plan->gc_vec = gv;
  plan->gc_mf = gm;
  const int gc_min = gm > 0 && gm < gv ? gm : gv;
  const int gc_max = gm > gv ? gm : gv;
  const int64_t rows_max = (int64_t)Hkv * (G / gc_min);
  // Tiles of a row with the smallest tile of any dtype (8 tokens): an upper
  // bound of the flat tile count, so the plan depends on the arguments only.
  const int64_t nt_max = ((int64_t)max_context_len + 7) / 8;
  const int64_t per_seq = nt_max * rows_max;
  // Sequences per launch: the LDS prefix capacity, and the flat tile count plus
  // the wave count must stay below 2^31.
  const int64_t limit = (int64_t)0x7fffffff - (int64_t)kMaxGrid * kWaves;
  int64_t sc = per_seq > 0 ? limit / per_seq : kMaxSeqPerLaunch;
  if (sc > kMaxSeqPerLaunch) sc = kMaxSeqPerLaunch;
  if (sc > S) sc = S;
  if (sc < 1 && S > 0) return fail(PKV_ERR_UNSUPPORTED, "decode: context too long (%d)", max_context_len);
  plan->seqs_per_launch = (int)sc;
  // waves of the largest launch: no more than kMaxGrid workgroups, and no more
  // than the tiles of the largest sequence chunk
  const int64_t tiles = (int64_t)sc * per_seq;
  int64_t grid = (tiles + kWaves - 1) / kWaves;
  if (grid > kMaxGrid) grid = kMaxGrid;
  if (grid < 1) grid = 1;
  plan->gc_max = gc_max;
  plan->D = D;
  layout_decode_workspace(plan, (int)grid * kWaves);
  return PKV_OK;
}

void layout_decode_workspace(DecodePlan* plan, int max_waves) {
  plan->max_waves = max_waves;
  // states: two slots per wave, gc heads each (whichever path runs)
  const size_t states = (size_t)plan->max_waves * 2 * plan->gc_max;
  plan->ws_ps_off = 0;
  plan->ws_rec_off = align_up(((size_t)plan->seqs_per_launch + 1) * sizeof(int32_t));
  plan->ws_ml_off = plan->ws_rec_off + align_up((size_t)plan->max_waves * sizeof(int4));
  plan->ws_acc_off = plan->ws_ml_off + align_up(states * 2 * sizeof(float));
  plan->workspace_bytes = plan->ws_acc_off + states * (size_t)plan->D * sizeof(float);
}

void attach_decode_workspace(DecodeArgs* a, const DecodePlan& plan, void* workspace) {
  char* ws = static_cast<char*>(workspace);
  a->ws_ps = reinterpret_cast<int32_t*>(ws + plan.ws_ps_off);
  a->ws_rec = reinterpret_cast<int4*>(ws + plan.ws_rec_off);
  a->ws_ml = reinterpret_cast<float*>(ws + plan.ws_ml_off);
  a->ws_acc = reinterpret_cast<float*>(ws + plan.ws_acc_off);
}

pkv_status launch_decode(int kv_dt, bool fp8, const DecodePlan& plan, DecodeArgs a,
                         hipStream_t stream, int* waves_only) {
  // (kv_dt: the dtype of q; the lane layout follows it, also over FP8 pools)
  const bool mf = kv_dt != DT_F32 && a.D == 128 && a.B >= 4 && plan.gc_mf > 0;
  a.gc = mf ? plan.gc_mf : plan.gc_vec;
  a.n_hchunks = (a.Hq / a.Hkv) / a.gc;
  a.rows_per_seq = a.Hkv * a.n_hchunks;
  int tile = 0, rpw = 0;
  tile_geometry(kv_dt, a.D, &tile, &rpw);
  const bool uni = a.B >= rpw;
  const int64_t nt_max = ((int64_t)a.max_ctx + tile - 1) / tile;
  const int S_total = a.S;
  const int ncu = device_cu_count();
  if (ncu <= 0) return fail(PKV_ERR_HIP, "decode: cannot query the current device");
  const int es = dt_bytes(kv_dt), oes = dt_bytes(a.out_dt);
  const int64_t row_bytes = (int64_t)a.Hkv * a.D * es;  // one token's K (or V) row, 16-bit pools
  if (a.new_k && (!mf || fp8)) {
    // decode step off the 16-bit matrix-core path: the cache write as a launch
    // of its own, then the plain decode over the written pools
    if (!waves_only) {
      const pkv_status st =
          launch_reshape_and_cache(a.new_k, a.new_v, const_cast<void*>(a.k_cache),
                                   const_cast<void*>(a.v_cache), a.slot_mapping, a.S, row_bytes,
                                   a.nslots, stream);
      if (st != PKV_OK) return st;
    }
    a.new_k = a.new_v = nullptr;
    a.slot_mapping = nullptr;
  }
  for (int s0 = 0; s0 < S_total; s0 += plan.seqs_per_launch) {
    DecodeArgs b = a;
    b.S = S_total - s0 < plan.seqs_per_launch ? S_total - s0 : plan.seqs_per_launch;
    b.q = static_cast<const char*>(a.q) + (int64_t)s0 * a.Hq * a.D * es;
    b.out = static_cast<char*>(a.out) + (int64_t)s0 * a.Hq * a.D * oes;
    b.block_tables = a.block_tables + (int64_t)s0 * a.max_nb;
    b.context_lens = a.context_lens + s0;
    if (a.seq_start) b.seq_start = a.seq_start + s0;
    if (a.lse) b.lse = a.lse + (int64_t)s0 * a.Hq;
    if (a.new_k) {
      b.new_k = static_cast<const char*>(a.new_k) + s0 * row_bytes;
      b.new_v = static_cast<const char*>(a.new_v) + s0 * row_bytes;
      b.slot_mapping = a.slot_mapping + s0;
    }
    // no more waves than the batch could ever use, nor than the workspace
    // has slots for (the launch also caps at one resident wave set)
    const int64_t max_tiles = (int64_t)b.S * a.rows_per_seq * nt_max;
    int64_t cap = (max_tiles + kWaves - 1) / kWaves;
    if (cap > plan.max_waves / kWaves) cap = plan.max_waves / kWaves;
    if (cap < 1) cap = 1;
    pkv_status st;
    if (fp8) {
      switch (kv_dt) {
        case DT_F16: st = launch_d<DT_F16, true>(b, (int)cap, ncu, uni, stream, waves_only); break;
        case DT_BF16: st = launch_d<DT_BF16, true>(b, (int)cap, ncu, uni, stream, waves_only); break;
        default: return fail(PKV_ERR_UNSUPPORTED, "decode_fp8: q dtype %d", kv_dt);
      }
    } else {
      switch (kv_dt) {
        case DT_F32: st = launch_d<DT_F32, false>(b, (int)cap, ncu, uni, stream, waves_only); break;
        case DT_F16: st = launch_d<DT_F16, false>(b, (int)cap, ncu, uni, stream, waves_only); break;
        case DT_BF16: st = launch_d<DT_BF16, false>(b, (int)cap, ncu, uni, stream, waves_only); break;
        default: return fail(PKV_ERR_UNSUPPORTED, "decode: kv dtype %d", kv_dt);
      }
    }
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

}  // namespace pkv
