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
// Design (gfx950, HBM-bound: every valid K/V row is read exactly once):
//  * One workgroup (4 waves) per (partition of P tokens, sequence, KV head,
//    chunk of GC query heads).  Long contexts are split into partitions whose
//    partial (max, sum, acc) states are merged by a second, tiny kernel.
//  * A token row of one KV head is D * elem bytes contiguous (256 B for bf16
//    D = 128).  LPR lanes cover one row with 16-byte loads, so one wave-load
//    instruction reads RPW = 64 / LPR complete rows, fully coalesced.  A tile
//    is 4 such loads (16 tokens for bf16 D = 128, i.e. exactly one block of
//    16): for blocks at least a tile long the whole tile sits in one physical
//    block and its table entry is a single scalar (SGPR) load per tile.
//  * Each K/V load serves all GC query heads of the group (GQA reuse in
//    registers).  q . k uses the packed dot2 instructions for 16-bit KV
//    (v_dot2c_f32_{bf16,f16}: exact products, fp32 accumulation), then a DPP
//    butterfly inside the LPR-lane row.  Every row of lanes keeps its own
//    online-softmax state; rows are merged with cross-lane shuffles and waves
//    through LDS once per workgroup.
//  * Loads of tile k + 4 (the wave's next tile) are issued before tile k is
//    computed, and the table entry of the tile after that is prefetched, so
//    each wave keeps a full tile of K and V (8 KiB for bf16) in flight.
//  * Summation order depends only on logical positions, so results are
//    bit-identical for any physical placement or aliasing of blocks.
//  * Rows past context_lens[s] and table entries past the last block are never
//    dereferenced (masked lanes load nothing), so stale or poisoned memory there
//    cannot reach the output.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLoadsPerTile = 4;

// DPP control words (row = 16 lanes).
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i within 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
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
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
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

// Partition kernel.  UNIFORM: the block size is a multiple of the tile, so a
// tile lies in one physical block and its table entry is wave-uniform.
template <int DT, int D, int GC, bool UNIFORM>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(const DecodeArgs a) {
  constexpr int ES = dt_bytes(DT);
  constexpr int EPL = 16 / ES;     // elements per lane per load
  constexpr int LPR = D * ES / 16; // lanes per token row
  constexpr int RPW = 64 / LPR;    // token rows per wave-load
  constexpr int NLD = kLoadsPerTile;
  constexpr int TILE = NLD * RPW;  // tokens per tile

  __shared__ float sm_acc[kWaves][GC][D];
  __shared__ float sm_m[kWaves][GC];
  __shared__ float sm_l[kWaves][GC];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane / LPR;
  const int col = lane % LPR;

  int idx = blockIdx.x;
  const int hc = idx % a.n_hchunks;
  idx /= a.n_hchunks;
  const int kvh = idx % a.Hkv;
  idx /= a.Hkv;
  const int s = idx % a.S;
  idx /= a.S;
  const int p = a.np_max - 1 - idx;  // longest work first: high partitions launch first

  const int L = min(a.context_lens[s], a.max_ctx);  // a larger value would overrun the table
  const int P = a.part_tokens;
  const int np = (L + P - 1) / P;
  const int G = a.Hq / a.Hkv;
  const int h0 = kvh * G + hc * GC;

  if (L <= 0) {  // empty context: defined as an all-zero output row
    if (p == 0) {
      for (int j = threadIdx.x; j < GC * D; j += kThreads)
        store_out(a.out, a.out_dt, ((int64_t)s * a.Hq + h0) * D + j, 0.f);
    }
    return;
  }
  if (p >= np) return;

  const int t0 = p * P;
  const int t1 = min(L, t0 + P);
  const int ntiles = (t1 - t0 + TILE - 1) / TILE;

  // this lane's slice of each query head (unscaled; the scale is applied to the score)
  uint4 qv[GC];
#pragma unroll
  for (int g = 0; g < GC; ++g)
    qv[g] = ld16(static_cast<const char*>(a.q) + (((int64_t)s * a.Hq + h0 + g) * D) * ES + col * 16);

  float m[GC], l[GC], acc[GC][EPL];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    m[g] = -__builtin_inff();
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  const int32_t* __restrict__ table = a.block_tables + (int64_t)s * a.max_nb;
  const int64_t row_stride = (int64_t)a.Hkv * D * ES;  // bytes between consecutive slots
  const int64_t blk_stride = row_stride * a.B;
  const char* kbase = static_cast<const char*>(a.k_cache) + (int64_t)kvh * D * ES;
  const char* vbase = static_cast<const char*>(a.v_cache) + (int64_t)kvh * D * ES;
  const int log2B = a.log2B;
  const int bmask = a.B - 1;

  // per-lane byte offset of load i inside a tile, relative to the tile's first slot
  int lane_off[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) lane_off[i] = (i * RPW + row) * (int)row_stride + col * 16;

  uint4 kb0[NLD], vb0[NLD], kb1[NLD], vb1[NLD];

  // Issue the K/V loads of tile k (k < ntiles).  `phys` is the tile's physical
  // block (UNIFORM only).
  auto issue = [&](int k, int phys, uint4 (&kb)[NLD], uint4 (&vb)[NLD]) {
    const int ts = t0 + k * TILE;
    if constexpr (UNIFORM) {
      const int64_t base = (int64_t)phys * blk_stride + (int64_t)(ts & bmask) * row_stride;
      const char* kp = kbase + base;
      const char* vp = vbase + base;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const bool valid = ts + i * RPW + row < t1;
        kb[i] = valid ? ld16(kp + lane_off[i]) : make_uint4(0, 0, 0, 0);
        vb[i] = valid ? ld16(vp + lane_off[i]) : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int tok = ts + i * RPW + row;
        if (tok < t1) {
          const int ph = table[tok >> log2B];
          const int64_t off = ((int64_t)ph * a.B + (tok & bmask)) * row_stride + col * 16;
          kb[i] = ld16(kbase + off);
          vb[i] = ld16(vbase + off);
        } else {
          kb[i] = make_uint4(0, 0, 0, 0);
          vb[i] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  auto compute = [&](int k, const uint4 (&kb)[NLD], const uint4 (&vb)[NLD]) {
    const int ts = t0 + k * TILE;
    float z[NLD][GC];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const bool valid = ts + i * RPW + row < t1;
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        const float part = dot16<DT>(kb[i], qv[g]);
        const float zz = row_sum<LPR>(part) * a.scale_log2;
        z[i][g] = valid ? zz : -__builtin_inff();
      }
    }
    float pr[NLD][GC];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      float tmax = z[0][g];
#pragma unroll
      for (int i = 1; i < NLD; ++i) tmax = fmaxf(tmax, z[i][g]);
      const float mn = fmaxf(m[g], tmax);
      const float mu = mn == -__builtin_inff() ? 0.f : mn;
      const float alpha = fast_exp2(m[g] - mu);
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        pr[i][g] = fast_exp2(z[i][g] - mu);
        ps += pr[i][g];
      }
      l[g] = fmaf(l[g], alpha, ps);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
      m[g] = mn;
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      float vf[EPL];
      widen16<DT>(vb[i], vf);
#pragma unroll
      for (int g = 0; g < GC; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(pr[i][g], vf[e], acc[g][e]);
    }
  };

  auto phys_of = [&](int k) -> int {
    if constexpr (UNIFORM) return table[(t0 + k * TILE) >> log2B];
    else return 0;
  };

  // Software pipeline over this wave's tiles wave, wave + 4, ...: loads of the
  // next tile are in flight while the current one is computed.
  int k = wave;
  if (k < ntiles) {
    issue(k, phys_of(k), kb0, vb0);
    int ph_next = (k + kWaves < ntiles) ? phys_of(k + kWaves) : 0;
    while (true) {
      const int k1 = k + kWaves;
      if (k1 < ntiles) {
        issue(k1, ph_next, kb1, vb1);
        ph_next = (k1 + kWaves < ntiles) ? phys_of(k1 + kWaves) : 0;
      }
      compute(k, kb0, vb0);
      if (k1 >= ntiles) break;
      const int k2 = k1 + kWaves;
      if (k2 < ntiles) {
        issue(k2, ph_next, kb0, vb0);
        ph_next = (k2 + kWaves < ntiles) ? phys_of(k2 + kWaves) : 0;
      }
      compute(k1, kb1, vb1);
      if (k2 >= ntiles) break;
      k = k2;
    }
  }

  // merge the RPW row states of this wave (rows differ in lane bits >= log2 LPR)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float mu = mn == -__builtin_inff() ? 0.f : mn;
      const float a1 = fast_exp2(m[g] - mu);
      const float a2 = fast_exp2(mo - mu);
      l[g] = l[g] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[g][e], off);
        acc[g][e] = acc[g][e] * a1 + ao * a2;
      }
      m[g] = mn;
    }
  }

  if (row == 0) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[wave][g][col * EPL + e] = acc[g][e];
      if (col == 0) {
        sm_m[wave][g] = m[g];
        sm_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();

  // merge the waves (fixed order) and write the partition result
  for (int j = threadIdx.x; j < GC * D; j += kThreads) {
    const int g = j / D;
    const int d = j % D;
    float M = sm_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][g]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = fast_exp2(sm_m[w][g] - M);
      num += sm_acc[w][g][d] * sc;
      den += sm_l[w][g] * sc;
    }
    const int h = h0 + g;
    if (np == 1) {
      store_out(a.out, a.out_dt, ((int64_t)s * a.Hq + h) * D + d, num / den);
    } else {
      const int64_t slot = ((int64_t)s * a.Hq + h) * a.np_max + p;
      a.ws_acc[slot * D + d] = num;
      if (d == 0) {
        a.ws_ml[2 * slot] = M;
        a.ws_ml[2 * slot + 1] = den;
      }
    }
  }
}

// Second pass for sequences split into several partitions:
// out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p   (m in log2 units).
template <int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(const DecodeArgs a) {
  const int s = blockIdx.x / a.Hq;
  const int h = blockIdx.x % a.Hq;
  const int L = min(a.context_lens[s], a.max_ctx);
  const int np = (L + a.part_tokens - 1) / a.part_tokens;
  if (np <= 1) return;  // written directly by the partition kernel
  const int d = threadIdx.x;
  const int64_t base = ((int64_t)s * a.Hq + h) * a.np_max;
  float M = -__builtin_inff();
  for (int p = 0; p < np; ++p) M = fmaxf(M, a.ws_ml[2 * (base + p)]);
  float num = 0.f, den = 0.f;
  for (int p = 0; p < np; ++p) {
    const float sc = fast_exp2(a.ws_ml[2 * (base + p)] - M);
    num += a.ws_acc[(base + p) * D + d] * sc;
    den += a.ws_ml[2 * (base + p) + 1] * sc;
  }
  store_out(a.out, a.out_dt, ((int64_t)s * a.Hq + h) * D + d, num / den);
}

template <int DT, int D, int GC>
pkv_status launch_typed(const DecodeArgs& a, hipStream_t stream) {
  constexpr int ES = dt_bytes(DT);
  constexpr int RPW = 64 / (D * ES / 16);
  constexpr int TILE = kLoadsPerTile * RPW;
  const int64_t grid = (int64_t)a.np_max * a.S * a.Hkv * a.n_hchunks;
  if (grid == 0) return PKV_OK;
  if (grid > 0x7fffffff) return fail(PKV_ERR_UNSUPPORTED, "decode grid too large (%lld)", (long long)grid);
  if (a.B >= TILE) {
    hipLaunchKernelGGL((decode_partition_kernel<DT, D, GC, true>), dim3((unsigned)grid),
                       dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_partition_kernel<DT, D, GC, false>), dim3((unsigned)grid),
                       dim3(kThreads), 0, stream, a);
  }
  pkv_status st = check_launch("paged_attention_decode (partition)");
  if (st != PKV_OK || a.np_max <= 1) return st;
  hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3(a.S * a.Hq), dim3(D), 0, stream, a);
  return check_launch("paged_attention_decode (reduce)");
}

template <int DT, int D>
pkv_status launch_gc(const DecodeArgs& a, hipStream_t stream) {
  switch (a.gc) {
    case 1: return launch_typed<DT, D, 1>(a, stream);
    case 2: return launch_typed<DT, D, 2>(a, stream);
    case 4: return launch_typed<DT, D, 4>(a, stream);
    case 8: return launch_typed<DT, D, 8>(a, stream);
    default: return fail(PKV_ERR_UNSUPPORTED, "decode: head chunk %d", a.gc);
  }
}

template <int DT>
pkv_status launch_d(const DecodeArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 64: return launch_gc<DT, 64>(a, stream);
    case 128: return launch_gc<DT, 128>(a, stream);
    default: return fail(PKV_ERR_UNSUPPORTED, "decode: head_dim %d", a.D);
  }
}

}  // namespace

pkv_status plan_decode(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t /*B*/,
                       int32_t max_context_len, DecodePlan* plan) {
  const int G = Hq / Hkv;
  int gc = 1;
  for (int c : {8, 4, 2}) {
    if (G % c == 0) {
      gc = c;
      break;
    }
  }
  plan->gc = gc;
  plan->part_tokens = 512;
  plan->np_max = max_context_len <= 0 ? 1 : (max_context_len + plan->part_tokens - 1) / plan->part_tokens;
  plan->workspace_bytes =
      plan->np_max <= 1 ? 0 : (size_t)S * Hq * plan->np_max * ((size_t)D + 2) * sizeof(float);
  return PKV_OK;
}

pkv_status launch_decode(int kv_dt, const DecodeArgs& a, hipStream_t stream) {
  switch (kv_dt) {
    case DT_F32: return launch_d<DT_F32>(a, stream);
    case DT_F16: return launch_d<DT_F16>(a, stream);
    case DT_BF16: return launch_d<DT_BF16>(a, stream);
    default: return fail(PKV_ERR_UNSUPPORTED, "decode: kv dtype %d", kv_dt);
  }
}

}  // namespace pkv
