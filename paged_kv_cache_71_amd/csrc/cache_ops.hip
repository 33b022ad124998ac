// cache_ops.hip -- the two pure data-movement kernels of the paged KV cache.
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
//
// Both are HBM copies: 16-byte lanes, fully coalesced, one workgroup per row
// (or per block and layer), no LDS.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kCopyThreads = 256;

// One workgroup per token; thread i copies 16-byte chunks i, i+256, ... of the
// token's K row and V row.  Negative slots (padding) are skipped.
__global__ __launch_bounds__(kCopyThreads) void reshape_and_cache_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int64_t row_chunks) {
  const int64_t t = blockIdx.x;
  const int64_t slot = slot_mapping[t];
  if (slot < 0) return;
  const uint4* ks = key + t * row_chunks;
  const uint4* vs = value + t * row_chunks;
  uint4* kd = k_cache + slot * row_chunks;
  uint4* vd = v_cache + slot * row_chunks;
  for (int64_t i = threadIdx.x; i < row_chunks; i += kCopyThreads) {
    const uint4 kk = ks[i];
    const uint4 vv = vs[i];
    kd[i] = kk;
    vd[i] = vv;
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

}  // namespace

pkv_status launch_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slot_mapping, int32_t T,
                                    int64_t row_bytes, int32_t /*B*/, hipStream_t stream) {
  if (T == 0) return PKV_OK;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(T), dim3(kCopyThreads), 0, stream,
                     static_cast<const uint4*>(key), static_cast<const uint4*>(value),
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), slot_mapping,
                     row_bytes / 16);
  return check_launch("reshape_and_cache");
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
