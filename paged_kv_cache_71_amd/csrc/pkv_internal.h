// pkv_internal.h -- shared declarations of the HIP library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

// ---- error reporting (abi.hip) ------------------------------------------------
pkv_status fail(pkv_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pkv_status check_launch(const char* what);

// ---- dtype helpers --------------------------------------------------------------
enum : int { DT_F32 = PKV_F32, DT_F16 = PKV_F16, DT_BF16 = PKV_BF16 };

constexpr int dt_bytes(int dt) { return dt == DT_F32 ? 4 : 2; }

// Reinterpretation helpers usable on host and device.
__device__ __forceinline__ float bf16_lo_to_f32(uint32_t packed) {
  return __uint_as_float(packed << 16);
}
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t packed) {
  return __uint_as_float(packed & 0xffff0000u);
}
__device__ __forceinline__ float f16_lo_to_f32(uint32_t packed) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(packed & 0xffffu));
}
__device__ __forceinline__ float f16_hi_to_f32(uint32_t packed) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(packed >> 16));
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Store one fp32 result into an output tensor of dtype out_dt.
__device__ __forceinline__ void store_out(void* out, int out_dt, int64_t idx, float v) {
  if (out_dt == DT_F32) {
    static_cast<float*>(out)[idx] = v;
  } else if (out_dt == DT_BF16) {
    static_cast<uint16_t*>(out)[idx] = f32_to_bf16_bits(v);
  } else {
    static_cast<uint16_t*>(out)[idx] = f32_to_f16_bits(v);
  }
}

// ---- launchers (one per kernel family) -------------------------------------------
pkv_status launch_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slot_mapping, int32_t T,
                                    int64_t row_bytes, int32_t B, hipStream_t stream);

pkv_status launch_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                              const int64_t* pairs, int32_t N, int64_t block_bytes,
                              hipStream_t stream);

struct DecodePlan {
  int part_tokens;  // tokens per partition (multiple of 64)
  int np_max;       // partitions of the longest sequence
  int gc;           // query heads per workgroup (divides G)
  size_t workspace_bytes;
};
pkv_status plan_decode(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                       int32_t max_context_len, DecodePlan* plan);

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_acc;  // [S, Hq, np_max, D]
  float* ws_ml;   // [S, Hq, np_max, 2]  (running max in log2 units, sum)
  int32_t max_nb;
  int32_t S, Hq, Hkv, D, B, log2B;
  int32_t part_tokens, np_max, n_hchunks, gc;
  int32_t max_ctx;   // context lengths are clamped to this (<= max_nb * B)
  int32_t out_dt;
  float scale_log2;  // softmax scale * log2(e)
};
pkv_status launch_decode(int kv_dt, const DecodeArgs& a, hipStream_t stream);

struct PrefillArgs {
  void* out;
  const void* q;
  const int32_t* cu_seqlens_q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t max_nb;
  int32_t Tq, max_query_len, S, Hq, Hkv, D, B, log2B;
  int32_t max_ctx;   // context lengths are clamped to this (<= max_nb * B)
  int32_t out_dt;
  float scale_log2;
};
pkv_status launch_prefill(int kv_dt, const PrefillArgs& a, hipStream_t stream);

}  // namespace pkv
