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
enum : int { DT_F32 = PKV_F32, DT_F16 = PKV_F16, DT_BF16 = PKV_BF16, DT_FP8 = PKV_FP8_E4M3 };

constexpr int dt_bytes(int dt) { return dt == DT_F32 ? 4 : dt == DT_FP8 ? 1 : 2; }

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
  return __builtin_bit_cast(uint16_t, (__bf16)f);  // v_cvt_pk_bf16_f32: round to nearest even
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// 8 OCP E4M3 codes -> 8 elements of the 16-bit dtype DT, in order; every
// E4M3 value is exact in bf16 and in fp16 (unit scale).
template <int DT>
__device__ __forceinline__ uint4 fp8x8_to16(const uint2 v) {
  if constexpr (DT == DT_BF16) {
    return make_uint4(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.f, true)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.f, true)));
  } else {
    return make_uint4(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.x, 1.f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.x, 1.f, true)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.y, 1.f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.y, 1.f, true)));
  }
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

// Store N consecutive fp32 results (N = 4 or 8, idx a multiple of N) into an
// output tensor of dtype out_dt with 16- or 8-byte stores.
template <int N>
__device__ __forceinline__ void store_out_vec(void* out, int out_dt, int64_t idx, const float* v) {
  static_assert(N == 4 || N == 8, "vector width");
  if (out_dt == DT_F32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + idx);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) p[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  } else {
    uint32_t w[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const uint32_t lo = out_dt == DT_BF16 ? f32_to_bf16_bits(v[2 * i]) : f32_to_f16_bits(v[2 * i]);
      const uint32_t hi =
          out_dt == DT_BF16 ? f32_to_bf16_bits(v[2 * i + 1]) : f32_to_f16_bits(v[2 * i + 1]);
      w[i] = lo | (hi << 16);
    }
    uint16_t* base = static_cast<uint16_t*>(out) + idx;
    if constexpr (N == 8) *reinterpret_cast<uint4*>(base) = make_uint4(w[0], w[1], w[2], w[3]);
    else *reinterpret_cast<uint2*>(base) = make_uint2(w[0], w[1]);
  }
}

// ---- launchers (one per kernel family) -------------------------------------------
// nslots = NB * B: tokens with a slot outside [0, nslots) are skipped
pkv_status launch_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slot_mapping, int32_t T,
                                    int64_t row_bytes, int64_t nslots, hipStream_t stream);

pkv_status launch_reshape_and_cache_fp8(const void* key, const void* value, int in_dt,
                                        void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                        int32_t T, int32_t Hkv, int32_t D, int64_t nslots,
                                        const float* k_scale, const float* v_scale,
                                        hipStream_t stream);

pkv_status launch_swap_blocks(const void* const* src_pools, void* const* dst_pools,
                              int32_t num_pools, const int64_t* pairs, int32_t N,
                              int64_t block_bytes, hipStream_t stream);

pkv_status launch_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                              const int64_t* pairs, int32_t N, int64_t block_bytes,
                              hipStream_t stream);

struct DecodePlan {
  int gc_vec;           // query heads per row on the vector path (divides G)
  int gc_mf;            // ... on the matrix-core path (4, 8 or 16 dividing G; 0: none)
  int max_waves;        // waves of the largest split launch (sizes the workspace)
  int seqs_per_launch;  // sequences handled by one split + merge launch pair
  int gc_max, D;        // largest head chunk of either path; head dim (state sizes)
  size_t ws_ps_off, ws_rec_off, ws_ml_off, ws_acc_off;  // workspace layout (bytes)
  size_t workspace_bytes;
};
pkv_status plan_decode(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                       int32_t max_context_len, DecodePlan* plan);
// Lay the workspace out for at most max_waves waves per launch (plan_decode
// uses the argument-only bound; a launch never uses more than plan.max_waves).
void layout_decode_workspace(DecodePlan* plan, int max_waves);
struct DecodeArgs;
// point the workspace fields of a at the plan's layout inside ws
void attach_decode_workspace(DecodeArgs* a, const DecodePlan& plan, void* ws);

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t* ws_ps;   // [S + 1] prefix of tile counts (written by the split kernel)
  int4* ws_rec;     // [n_waves] rows cut at each wave's start: the merge's work list
  float* ws_ml;     // [2 * n_waves, gc, 2] partial (c * max, sum) in log2 units
  float* ws_acc;    // [2 * n_waves, gc, D] partial accumulators
  int32_t max_nb;
  int32_t S, Hq, Hkv, D, B, log2B;
  int32_t gc, n_hchunks, rows_per_seq, n_waves;  // (set by launch_decode)
  int32_t max_ctx;       // context lengths are clamped to this (<= max_nb * B)
  int32_t out_dt;
  float scale_log2;      // softmax scale * log2(e)
  const float* k_scale;  // FP8 pools: per-KV-head scales (device, [Hkv]); else unused
  const float* v_scale;
  // optional (null = off): first token attended per sequence (device [S],
  // 0 <= start <= context length; a multiple of B), and a log2-sum-exp output
  // per (sequence, head) (device [S, Hq]; -inf for an empty range)
  const int32_t* seq_start;
  float* lse;
  // optional (null = off): the decode step's new tokens, device [S, Hkv, D] of
  // the pools' 16-bit dtype.  Token context_lens[s] - 1 of sequence s is read
  // from new_k/new_v[s] instead of the pools, and those rows are stored at
  // slot_mapping[s] of the pools (int64 [S]; skipped outside [0, nslots)).
  const void* new_k = nullptr;
  const void* new_v = nullptr;
  const int64_t* slot_mapping = nullptr;
  int64_t nslots = 0;
};
// q_dt: dtype of q (and of the pools unless fp8); fp8: the pools hold E4M3 codes.
// waves_only != null: launch nothing, store the most waves any split launch of
// this call would run (on the current device) in *waves_only.
pkv_status launch_decode(int q_dt, bool fp8, const DecodePlan& plan, DecodeArgs a,
                         hipStream_t stream, int* waves_only = nullptr);

// Cascade decode (cascade.hip): groups of sequences sharing a prefix.
pkv_status cascade_workspace_size(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                  int32_t max_context_len, int32_t n_groups, int32_t max_group_size,
                                  int32_t max_prefix_len, int kv_dt, size_t* bytes);
pkv_status launch_decode_cascade(int kv_dt, bool fp8, const DecodeArgs& base, const int32_t* cu_group_seqs,
                                 const int32_t* group_prefix_lens, int32_t n_groups,
                                 int32_t max_group_size, int32_t max_prefix_len, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

struct PrefillArgs {
  void* out;
  const void* q;
  const int32_t* cu_seqlens_q;
  int32_t cu_base;   // subtracted from every cu_seqlens_q entry (mixed batches:
                     // the decode rows that come before the chunks)
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t max_nb;
  int32_t Tq, max_query_len, S, Hq, Hkv, D, B, log2B;
  int32_t max_ctx;   // context lengths are clamped to this (<= max_nb * B)
  int32_t out_dt;
  float scale_log2;
  // split of each workgroup's KV range (plan_prefill): n_split > 1 writes
  // partial results of rows whose range spans several splits to ws_o / ws_ml
  // and a merge kernel combines them
  int32_t n_split, tiles_per_split;
  float* ws_o;   // [n_split][Tq * Hq][D] unnormalised outputs
  float* ws_ml;  // [n_split][Tq * Hq][2] running max (log2 units) and weight sum
  // FP8 pools (launch_prefill with DT_FP8): q's 16-bit dtype and the per-KV-head
  // scales the codes are multiplied by
  int32_t q_dt;
  const float* k_scale;
  const float* v_scale;
};
// Split plan of a prefill launch: a deterministic function of the arguments
// (and of the device's CU count), so equal calls give equal bits.
struct PrefillPlan {
  int n_split;          // 1: no split
  int tiles_per_split;  // KV tiles (32 tokens) per split
  size_t workspace_bytes;
};
PrefillPlan plan_prefill(int kv_dt, int32_t S, int32_t Tq, int32_t max_query_len, int32_t Hq,
                         int32_t Hkv, int32_t D, int32_t B, int32_t max_ctx);
pkv_status launch_prefill(int kv_dt, const PrefillArgs& a, hipStream_t stream);
// Compute units of the current device (cached per device; 0 if unknown).
int device_cu_count();

// Mixed decode + prefill batch (mixed.hip): the decode part (dec.S sequences,
// plan for them) and the prefill part (pre: the whole batch's pointers, pre.S =
// number of prefill sequences after the num_decode decodes).
size_t mixed_workspace_size(const DecodePlan& plan, const PrefillPlan& pplan);
pkv_status launch_mixed(int kv_dt, bool fp8, const DecodePlan& plan, const PrefillPlan& pplan,
                        const DecodeArgs& dec, const PrefillArgs& pre, int32_t num_decode,
                        void* workspace, hipStream_t stream);

}  // namespace pkv
