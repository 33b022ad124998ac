// cache_ops.hip -- the data-movement kernels of the paged KV cache.
//
//  * reshape_and_cache: every new token's K row and V row (Hkv*D contiguous
//    elements each) is written to its absolute slot of the pool.  With the
//    [NB, B, Hkv, D] pool layout a slot's row is also Hkv*D contiguous
//    elements, so the "reshape" is a contiguous row copy to a computed address
//    ("LLM inference, part 3: single node", ch. 13 sec. 1: the GPU only does
//    kv_cache[slot_mapping[i]] = new_kv; CS349D lecture 3 sec. 3.2: one fused
//    kernel for split + reorder + block write).
//  * copy_blocks: all copy-on-write block copies of a step, for every layer,
//    in one launch (CS349D lecture 3 sec. 3.2 and sec. 4.1).
//  * swap_blocks: whole blocks between two sets of pools, one in device
//    memory and one in pinned host memory (or both on the device), for every
//    layer in one launch -- the swap-out / swap-in of a preempted sequence
//    (CS349D lecture 3 sec. 5.2: KV blocks copied to CPU memory and back; a
//    fixed cost per separate copy makes one batched launch pay off).  The
//    kernel reads and writes the pinned host pages directly over the host link.
//  * reshape_and_cache_fp8: the same scatter into an FP8 pool, each element
//    scaled by its KV head's scale and rounded into an OCP E4M3 code
//    ("LLM inference, part 3", ch. 10: scale and clip into 8 bits on write).
//
// All are copies (through HBM, or over the host link for swaps): 16-byte
// lanes, fully coalesced, one workgroup per row (or per block and layer), no
// LDS.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kTokensPerGroup = kCopyThreads / 64;  // reshape: one wave per token

// One wave per token, four tokens per workgroup; lane i copies the 16-byte
// chunks i, i + 64, ... of the token's K row and V row (a bf16 row of 8 heads
// x 128 is 128 chunks: two of K and two of V per lane, all four loads in
// flight together).  The row's first chunks are loaded without waiting for
// the slot (the loads do not depend on it); tokens whose slot lies outside
// [0, nslots) -- negative slots are padding -- store nothing.
__global__ __launch_bounds__(kCopyThreads) void reshape_and_cache_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int32_t T,
    int64_t nslots, int32_t row_chunks) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = (int64_t)blockIdx.x * kTokensPerGroup + wave;
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const int64_t slot = slot_mapping[t];
  const bool keep = slot >= 0 && slot < nslots;
  const uint4* ks = key + t * row_chunks;
  const uint4* vs = value + t * row_chunks;
  uint4* kd = k_cache + slot * row_chunks;
  uint4* vd = v_cache + slot * row_chunks;
  for (int i0 = 0; i0 < row_chunks; i0 += 128) {
    const int i1 = i0 + lane, i2 = i1 + 64;
    uint4 k1{}, v1{}, k2{}, v2{};
    if (i1 < row_chunks) {
      k1 = ks[i1];
      v1 = vs[i1];
    }
    if (i2 < row_chunks) {
      k2 = ks[i2];
      v2 = vs[i2];
    }
    if (keep) {
      if (i1 < row_chunks) {
        kd[i1] = k1;
        vd[i1] = v1;
      }
      if (i2 < row_chunks) {
        kd[i2] = k2;
        vd[i2] = v2;
      }
    }
  }
}

// fp32 -> OCP E4M3 code, written from the format: 4 exponent bits with bias 7,
// 3 mantissa bits, subnormals (steps of 2^-9 below 2^-6), largest finite
// value 448 = 1.75 * 2^8.  Round to nearest even; anything at or beyond 448
// (infinities too) clips to +-448; NaN gives the NaN code of its sign.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;  // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |x| >= 448: clip
  if (a < 0x3c800000u) {
    // |x| < 2^-6: code = |x| / 2^-9 rounded to an integer 0..8 (8 is the
    // smallest normal, 2^-6); the power-of-two product is exact
    return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  // normal: keep 3 of fp32's 23 mantissa bits, round to nearest even (a carry
  // into the exponent is the correct rounding), then rebias 127 -> 7
  const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
  return sign | (r - (120u << 3));
}

// the 8 elements e0 .. e0 + 7 of row as fp32 (e0 a multiple of 8; 16-byte
// aligned: one 16-byte load for 16-bit inputs, two for f32)
template <int IDT>
__device__ __forceinline__ void load8_f32(const void* row, int64_t e0, float (&x)[8]) {
  if constexpr (IDT == DT_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(row) + e0);
    const float4 a = p[0], b = p[1];
    x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w, x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(row) + e0);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (IDT == DT_BF16) {
        x[2 * j] = __uint_as_float(w[j] << 16);
        x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      } else {
        x[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] & 0xffffu));
        x[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] >> 16));
      }
    }
  }
}

// One wave per token, four tokens per workgroup; lane i quantizes the
// 8-element groups i, i + 64, ... of the token's K row and V row (one group =
// one 16-byte load of a 16-bit input, 8 code bytes, one 8-byte store; D is a
// multiple of 8, so a group lies in one KV head).  Slots as in the copy above.
template <int IDT>
__global__ __launch_bounds__(kCopyThreads) void reshape_and_cache_fp8_kernel(
    const void* __restrict__ key, const void* __restrict__ value, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int32_t T,
    int64_t nslots, const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    int32_t Hkv, int32_t D) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = (int64_t)blockIdx.x * kTokensPerGroup + wave;
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const int64_t slot = slot_mapping[t];
  const bool keep = slot >= 0 && slot < nslots;
  const int64_t row = (int64_t)Hkv * D;
  const int ngroups = (int)(row / 8);
  const char* krow = static_cast<const char*>(key) + t * row * dt_bytes(IDT);
  const char* vrow = static_cast<const char*>(value) + t * row * dt_bytes(IDT);
  for (int gi = lane; gi < ngroups; gi += 64) {
    const int64_t e0 = (int64_t)gi * 8;
    float kx[8], vx[8];
    load8_f32<IDT>(krow, e0, kx);
    load8_f32<IDT>(vrow, e0, vx);
    const int h = (int)(e0 / D);
    const float ks = k_scale[h], vs = v_scale[h];
    uint32_t kw[2] = {0u, 0u}, vw[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      kw[j >> 2] |= e4m3_code(kx[j] / ks) << (8 * (j & 3));
      vw[j >> 2] |= e4m3_code(vx[j] / vs) << (8 * (j & 3));
    }
    if (keep) {
      *reinterpret_cast<uint2*>(k_cache + slot * row + e0) = make_uint2(kw[0], kw[1]);
      *reinterpret_cast<uint2*>(v_cache + slot * row + e0) = make_uint2(vw[0], vw[1]);
    }
  }
}

constexpr int kMaxLayersPerLaunch = 64;

struct LayerPtrs {
  uint4* k[kMaxLayersPerLaunch];
  uint4* v[kMaxLayersPerLaunch];
};

// grid = (N pairs, layers in this launch, 2 = K/V).  Each workgroup copies one
// whole block of one pool of one layer.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    LayerPtrs ptrs, const int64_t* __restrict__ pairs, int64_t block_chunks) {
  const int64_t src = pairs[2 * (int64_t)blockIdx.x];
  const int64_t dst = pairs[2 * (int64_t)blockIdx.x + 1];
  uint4* pool = blockIdx.z == 0 ? ptrs.k[blockIdx.y] : ptrs.v[blockIdx.y];
  const uint4* s = pool + src * block_chunks;
  uint4* d = pool + dst * block_chunks;
  int64_t i = threadIdx.x;
  // 4 independent 16-byte loads in flight per thread before the stores
  for (; i + 3 * kCopyThreads < block_chunks; i += 4 * kCopyThreads) {
    const uint4 a = s[i], b = s[i + kCopyThreads], c = s[i + 2 * kCopyThreads],
                e = s[i + 3 * kCopyThreads];
    d[i] = a;
    d[i + kCopyThreads] = b;
    d[i + 2 * kCopyThreads] = c;
    d[i + 3 * kCopyThreads] = e;
  }
  for (; i < block_chunks; i += kCopyThreads) d[i] = s[i];
}

struct PoolPairPtrs {
  const uint4* src[kMaxLayersPerLaunch];
  uint4* dst[kMaxLayersPerLaunch];
};

// grid = (N pairs, pools in this launch).  Each workgroup copies block src of
// source pool y to block dst of destination pool y.
__global__ __launch_bounds__(kCopyThreads) void swap_blocks_kernel(
    PoolPairPtrs ptrs, const int64_t* __restrict__ pairs, int64_t block_chunks) {
  const int64_t src = pairs[2 * (int64_t)blockIdx.x];
  const int64_t dst = pairs[2 * (int64_t)blockIdx.x + 1];
  const uint4* s = ptrs.src[blockIdx.y] + src * block_chunks;
  uint4* d = ptrs.dst[blockIdx.y] + dst * block_chunks;
  int64_t i = threadIdx.x;
  for (; i + 3 * kCopyThreads < block_chunks; i += 4 * kCopyThreads) {
    const uint4 a = s[i], b = s[i + kCopyThreads], c = s[i + 2 * kCopyThreads],
                e = s[i + 3 * kCopyThreads];
    d[i] = a;
    d[i + kCopyThreads] = b;
    d[i + 2 * kCopyThreads] = c;
    d[i + 3 * kCopyThreads] = e;
  }
  for (; i < block_chunks; i += kCopyThreads) d[i] = s[i];
}

}  // namespace

pkv_status launch_swap_blocks(const void* const* src_pools, void* const* dst_pools,
                              int32_t num_pools, const int64_t* pairs, int32_t N,
                              int64_t block_bytes, hipStream_t stream) {
  if (N == 0 || num_pools == 0) return PKV_OK;
  for (int32_t p0 = 0; p0 < num_pools; p0 += kMaxLayersPerLaunch) {
    const int32_t np = num_pools - p0 < kMaxLayersPerLaunch ? num_pools - p0 : kMaxLayersPerLaunch;
    PoolPairPtrs ptrs{};
    for (int32_t i = 0; i < np; ++i) {
      ptrs.src[i] = static_cast<const uint4*>(src_pools[p0 + i]);
      ptrs.dst[i] = static_cast<uint4*>(dst_pools[p0 + i]);
    }
    hipLaunchKernelGGL(swap_blocks_kernel, dim3(N, np), dim3(kCopyThreads), 0, stream, ptrs, pairs,
                       block_bytes / 16);
    pkv_status st = check_launch("swap_blocks");
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

// workgroups of a reshape launch: one per kTokensPerGroup tokens
static unsigned reshape_grid(int32_t T) {
  return (unsigned)(((int64_t)T + kTokensPerGroup - 1) / kTokensPerGroup);
}

pkv_status launch_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slot_mapping, int32_t T,
                                    int64_t row_bytes, int64_t nslots, hipStream_t stream) {
  if (T == 0) return PKV_OK;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(reshape_grid(T)), dim3(kCopyThreads), 0, stream,
                     static_cast<const uint4*>(key), static_cast<const uint4*>(value),
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), slot_mapping, T,
                     nslots, (int32_t)(row_bytes / 16));
  return check_launch("reshape_and_cache");
}

pkv_status launch_reshape_and_cache_fp8(const void* key, const void* value, int in_dt,
                                        void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                        int32_t T, int32_t Hkv, int32_t D, int64_t nslots,
                                        const float* k_scale, const float* v_scale,
                                        hipStream_t stream) {
  if (T == 0) return PKV_OK;
  const dim3 grid(reshape_grid(T));
  uint8_t* kc = static_cast<uint8_t*>(k_cache);
  uint8_t* vc = static_cast<uint8_t*>(v_cache);
  switch (in_dt) {
    case DT_F32:
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<DT_F32>, grid, dim3(kCopyThreads), 0, stream,
                         key, value, kc, vc, slot_mapping, T, nslots, k_scale, v_scale, Hkv, D);
      break;
    case DT_F16:
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<DT_F16>, grid, dim3(kCopyThreads), 0, stream,
                         key, value, kc, vc, slot_mapping, T, nslots, k_scale, v_scale, Hkv, D);
      break;
    case DT_BF16:
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<DT_BF16>, grid, dim3(kCopyThreads), 0, stream,
                         key, value, kc, vc, slot_mapping, T, nslots, k_scale, v_scale, Hkv, D);
      break;
    default:
      return fail(PKV_ERR_UNSUPPORTED, "reshape_and_cache_fp8: input dtype %d", in_dt);
  }
  return check_launch("reshape_and_cache_fp8");
}

pkv_status launch_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                              const int64_t* pairs, int32_t N, int64_t block_bytes,
                              hipStream_t stream) {
  if (N == 0 || num_layers == 0) return PKV_OK;
  for (int32_t l0 = 0; l0 < num_layers; l0 += kMaxLayersPerLaunch) {
    const int32_t nl = num_layers - l0 < kMaxLayersPerLaunch ? num_layers - l0
                                                             : kMaxLayersPerLaunch;
    LayerPtrs ptrs{};
    for (int32_t l = 0; l < nl; ++l) {
      ptrs.k[l] = static_cast<uint4*>(k_caches[l0 + l]);
      ptrs.v[l] = static_cast<uint4*>(v_caches[l0 + l]);
    }
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(N, nl, 2), dim3(kCopyThreads), 0, stream, ptrs,
                       pairs, block_bytes / 16);
    pkv_status st = check_launch("copy_blocks");
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

}  // namespace pkv
