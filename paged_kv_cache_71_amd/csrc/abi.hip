// abi.hip -- the C ABI of libpkv: host-side validation of every scalar argument,
// choice of kernel instantiation, launch on the caller's stream, and error
// reporting.  No device memory is allocated here.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <vector>

#include "pkv_internal.h"

namespace pkv {

namespace {
thread_local char g_last_error[512] = "";

bool supported_dtype(int dt) { return dt == PKV_F32 || dt == PKV_F16 || dt == PKV_BF16; }
bool supported_head_dim(int32_t D) { return D == 64 || D == 128; }
bool supported_block(int32_t B) {
  return B == 1 || B == 2 || B == 4 || B == 8 || B == 16 || B == 32;
}
// Tensor data is read and written with 16-byte vector accesses; index arrays
// and scales with accesses of their element size.
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
int ilog2(int32_t x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}
}  // namespace

pkv_status fail(pkv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

pkv_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace pkv

using namespace pkv;

#define PKV_REQUIRE(cond, status, ...) \
  do {                                 \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

namespace pkv {

// A cache write's arguments (both reshape entry points).
// fp8: the pools hold E4M3 codes and key/value (of in_dtype) are quantized
// with the per-head scales; else the pools and key/value are of in_dtype.
struct CacheWrite {
  const void* key;
  const void* value;
  const int64_t* slot_mapping;
  int32_t T;
  int64_t NB;
  pkv_dtype in_dtype;
  bool fp8;
  const float* k_scale;
  const float* v_scale;
};

static pkv_status check_cache_write(const char* who, const CacheWrite& cw, const void* k_cache,
                                    const void* v_cache, int32_t Hkv, int32_t D, int32_t B) {
  PKV_REQUIRE(cw.T >= 0, PKV_ERR_INVALID_ARG, "%s: T = %d", who, cw.T);
  PKV_REQUIRE(Hkv > 0 && D > 0 && B > 0 && cw.NB > 0, PKV_ERR_INVALID_ARG,
              "%s: Hkv=%d D=%d B=%d NB=%lld must be positive", who, Hkv, D, B, (long long)cw.NB);
  PKV_REQUIRE(supported_dtype(cw.in_dtype), PKV_ERR_UNSUPPORTED, "%s: dtype %d", who,
              (int)cw.in_dtype);
  PKV_REQUIRE(supported_head_dim(D), PKV_ERR_UNSUPPORTED, "%s: head_dim %d", who, D);
  PKV_REQUIRE(supported_block(B), PKV_ERR_UNSUPPORTED, "%s: block_size %d", who, B);
  PKV_REQUIRE(cw.NB <= INT64_MAX / B, PKV_ERR_INVALID_ARG, "%s: NB x B overflows", who);
  if (cw.T == 0) return PKV_OK;
  PKV_REQUIRE(cw.key && cw.value && k_cache && v_cache && cw.slot_mapping &&
                  (!cw.fp8 || (cw.k_scale && cw.v_scale)),
              PKV_ERR_INVALID_ARG, "%s: null pointer", who);
  PKV_REQUIRE(aligned(cw.key, 16) && aligned(cw.value, 16) && aligned(k_cache, 16) &&
                  aligned(v_cache, 16) && aligned(cw.slot_mapping, 8) && aligned(cw.k_scale, 4) &&
                  aligned(cw.v_scale, 4),
              PKV_ERR_INVALID_ARG,
              "%s: key, value and the pools must be 16-byte aligned, slot_mapping 8-byte, the "
              "scales 4-byte aligned", who);
  return PKV_OK;
}

// (checked arguments) the write's launch
static pkv_status launch_cache_write(const CacheWrite& cw, void* k_cache, void* v_cache,
                                     int32_t Hkv, int32_t D, int32_t B, hipStream_t stream) {
  const int64_t nslots = cw.NB * B;
  if (cw.fp8)
    return launch_reshape_and_cache_fp8(cw.key, cw.value, cw.in_dtype, k_cache, v_cache,
                                        cw.slot_mapping, cw.T, Hkv, D, nslots, cw.k_scale,
                                        cw.v_scale, stream);
  return launch_reshape_and_cache(cw.key, cw.value, k_cache, v_cache, cw.slot_mapping, cw.T,
                                  (int64_t)Hkv * D * dt_bytes(cw.in_dtype), nslots, stream);
}

}  // namespace pkv

extern "C" {

const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_OOM: return "PKV_ERR_OOM";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
  }
  return "PKV_ERR_UNKNOWN";
}

const char* pkv_last_error(void) { return g_last_error; }

const char* pkv_version(void) { return "pkv 0.1 gfx950"; }

pkv_status pkv_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                 const int64_t* slot_mapping, int32_t T, int32_t Hkv, int32_t D,
                                 int32_t B, int64_t NB, pkv_dtype kv_dtype, void* stream) {
  g_last_error[0] = 0;
  const pkv::CacheWrite cw{key, value, slot_mapping, T, NB, kv_dtype, false, nullptr, nullptr};
  const pkv_status st = pkv::check_cache_write("reshape_and_cache", cw, k_cache, v_cache, Hkv, D, B);
  if (st != PKV_OK) return st;
  return pkv::launch_cache_write(cw, k_cache, v_cache, Hkv, D, B, static_cast<hipStream_t>(stream));
}

pkv_status pkv_reshape_and_cache_fp8(const void* key, const void* value, pkv_dtype in_dtype,
                                     void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                     int32_t T, int32_t Hkv, int32_t D, int32_t B, int64_t NB,
                                     const float* k_scale, const float* v_scale, void* stream) {
  g_last_error[0] = 0;
  const pkv::CacheWrite cw{key, value, slot_mapping, T, NB, in_dtype, true, k_scale, v_scale};
  const pkv_status st =
      pkv::check_cache_write("reshape_and_cache_fp8", cw, k_cache, v_cache, Hkv, D, B);
  if (st != PKV_OK) return st;
  return pkv::launch_cache_write(cw, k_cache, v_cache, Hkv, D, B, static_cast<hipStream_t>(stream));
}

pkv_status pkv_decode_workspace_size(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                     int32_t max_context_len, size_t* bytes) {
  g_last_error[0] = 0;
  PKV_REQUIRE(bytes, PKV_ERR_INVALID_ARG, "decode_workspace_size: null output");
  PKV_REQUIRE(S >= 0 && Hq > 0 && Hkv > 0 && D > 0 && B > 0 && max_context_len >= 0,
              PKV_ERR_INVALID_ARG, "decode_workspace_size: bad sizes");
  PKV_REQUIRE(Hq % Hkv == 0, PKV_ERR_INVALID_ARG, "decode_workspace_size: Hq %% Hkv != 0");
  if (S == 0) {
    *bytes = 0;
    return PKV_OK;
  }
  DecodePlan plan;
  const pkv_status st = plan_decode(S, Hq, Hkv, D, B, max_context_len, &plan);
  if (st != PKV_OK) return st;
  *bytes = plan.workspace_bytes;
  return PKV_OK;
}

}  // extern "C"

// Both decode entry points: q_dtype is the dtype of q (and of the pools unless
// fp8, where the pools hold E4M3 codes with per-KV-head scales).
// Groups of sequences sharing a prefix (cascade decode), if on.
struct CascadeGroups {
  bool on = false;
  const int32_t* cu = nullptr;
  const int32_t* prefix_lens = nullptr;
  int32_t n_groups = 0, max_group_size = 0, max_prefix_len = 0;
};

// The allocation-free decode's scratch: a file-scope device array, one copy on
// every device the library runs on, held until the process ends.  Host code
// never uses its name as an address: scratch_address() gives the device's own
// address of it.  Every call on a device shares that device's copy.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

static std::atomic<void*> g_scratch_ptr[64];  // per device ordinal; null = not yet looked up

// Device address of this device's scratch (looked up once per device, with the
// device current; concurrent first calls store the same value).
static pkv_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PKV_ERR_HIP, "decode_noalloc: cannot query the current device");
  }
  if (dev < 0 || dev >= 64) return fail(PKV_ERR_UNSUPPORTED, "decode_noalloc: device %d", dev);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(PKV_ERR_HIP, "decode_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return PKV_OK;
}

// The decode step's new tokens (pkv_decode_step): one K and one V row per
// sequence and the slots they are written to.
struct StepTokens {
  const void* key = nullptr;
  const void* value = nullptr;
  const int64_t* slot_mapping = nullptr;
  int64_t NB = 0;
};

// use_scratch: the allocation-free variant; the workspace arguments are unused
// and the device's static scratch holds the partial states instead.
// step: a decode step (the new tokens written to the pools and attended).
static pkv_status decode_impl(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype kv_dtype,
                              bool fp8, const void* k_cache, const void* v_cache,
                              const float* k_scale, const float* v_scale,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t max_context_len, int32_t S,
                              int32_t Hq, int32_t Hkv, int32_t D, int32_t B, float scale,
                              void* workspace, size_t workspace_bytes, void* stream,
                              const CascadeGroups& cg = CascadeGroups(),
                              bool use_scratch = false, const StepTokens* step = nullptr) {
  g_last_error[0] = 0;
  const bool cascade = cg.on;
  PKV_REQUIRE(S >= 0 && Hq > 0 && Hkv > 0 && D > 0 && B > 0, PKV_ERR_INVALID_ARG,
              "decode: S=%d Hq=%d Hkv=%d D=%d B=%d", S, Hq, Hkv, D, B);
  PKV_REQUIRE(Hq % Hkv == 0, PKV_ERR_INVALID_ARG, "decode: Hq (%d) not a multiple of Hkv (%d)",
              Hq, Hkv);
  PKV_REQUIRE(max_context_len >= 0 && max_blocks_per_seq >= 0, PKV_ERR_INVALID_ARG,
              "decode: negative max_context_len or max_blocks_per_seq");
  PKV_REQUIRE(supported_dtype(kv_dtype) && supported_dtype(out_dtype), PKV_ERR_UNSUPPORTED,
              "decode: dtypes kv=%d out=%d", (int)kv_dtype, (int)out_dtype);
  PKV_REQUIRE(!fp8 || kv_dtype != PKV_F32, PKV_ERR_UNSUPPORTED,
              "decode_fp8: q must be f16 or bf16");
  PKV_REQUIRE(supported_head_dim(D), PKV_ERR_UNSUPPORTED, "decode: head_dim %d", D);
  PKV_REQUIRE(supported_block(B), PKV_ERR_UNSUPPORTED, "decode: block_size %d", B);
  PKV_REQUIRE((int64_t)max_context_len <= (int64_t)max_blocks_per_seq * B, PKV_ERR_INVALID_ARG,
              "decode: max_context_len %d exceeds table capacity %d x %d", max_context_len,
              max_blocks_per_seq, B);
  PKV_REQUIRE(scale == scale, PKV_ERR_INVALID_ARG, "decode: scale is NaN");
  PKV_REQUIRE((int64_t)B * Hkv * D * dt_bytes(fp8 ? (int)DT_FP8 : (int)kv_dtype) < ((int64_t)1 << 31),
              PKV_ERR_UNSUPPORTED,
              "decode: one block of one pool must be smaller than 2 GiB");
  if (cascade) {
    PKV_REQUIRE(cg.n_groups >= (S > 0 ? 1 : 0) && cg.n_groups <= S && cg.max_group_size >= 1 &&
                    cg.max_group_size <= S + (S == 0),
                PKV_ERR_INVALID_ARG, "decode_cascade: n_groups=%d max_group_size=%d for S=%d",
                cg.n_groups, cg.max_group_size, S);
    PKV_REQUIRE(cg.max_prefix_len >= 0, PKV_ERR_INVALID_ARG,
                "decode_cascade: negative max_prefix_len %d", cg.max_prefix_len);
  }
  if (step) {
    const pkv::CacheWrite cw{step->key, step->value, step->slot_mapping, S, step->NB,
                             kv_dtype, false, nullptr, nullptr};
    const pkv_status st = pkv::check_cache_write("decode_step", cw, k_cache, v_cache, Hkv, D, B);
    if (st != PKV_OK) return st;
    PKV_REQUIRE((int64_t)S * Hkv * D * dt_bytes(kv_dtype) / 16 < ((int64_t)1 << 31),
                PKV_ERR_UNSUPPORTED, "decode_step: %d new rows of %d x %d elements", S, Hkv, D);
  }
  if (S == 0) return PKV_OK;
  PKV_REQUIRE(out && q && k_cache && v_cache && block_tables && context_lens, PKV_ERR_INVALID_ARG,
              "decode: null pointer");
  PKV_REQUIRE(!fp8 || (k_scale && v_scale), PKV_ERR_INVALID_ARG, "decode_fp8: null scale array");
  PKV_REQUIRE(!cascade || (cg.cu && cg.prefix_lens), PKV_ERR_INVALID_ARG,
              "decode_cascade: null pointer");
  PKV_REQUIRE(aligned(out, 16) && aligned(q, 16) && aligned(k_cache, 16) && aligned(v_cache, 16) &&
                  aligned(workspace, 16),
              PKV_ERR_INVALID_ARG,
              "decode: out, q, the pools and the workspace must be 16-byte aligned");
  PKV_REQUIRE(aligned(block_tables, 4) && aligned(context_lens, 4) && aligned(k_scale, 4) &&
                  aligned(v_scale, 4) && aligned(cg.cu, 4) && aligned(cg.prefix_lens, 4),
              PKV_ERR_INVALID_ARG,
              "decode: index arrays and scales must be aligned to their element size");
  DecodePlan plan;
  const pkv_status pst = plan_decode(S, Hq, Hkv, D, B, max_context_len, &plan);
  if (pst != PKV_OK) return pst;
  if (!cascade && !use_scratch)
    PKV_REQUIRE(workspace_bytes >= plan.workspace_bytes && (plan.workspace_bytes == 0 || workspace),
                PKV_ERR_WORKSPACE, "decode: workspace of %zu bytes needed, %zu given",
                plan.workspace_bytes, workspace_bytes);
  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  attach_decode_workspace(&a, plan, workspace);
  a.max_nb = max_blocks_per_seq;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.B = B;
  a.log2B = ilog2(B);
  a.gc = a.n_hchunks = a.rows_per_seq = 0;  // chosen per path by launch_decode
  a.n_waves = 0;  // set per launch
  a.max_ctx = max_context_len;
  a.out_dt = out_dtype;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.seq_start = nullptr;
  a.lse = nullptr;
  if (step) {
    a.new_k = step->key;
    a.new_v = step->value;
    a.slot_mapping = step->slot_mapping;
    a.nslots = step->NB * B;
  }
  if (cascade)
    return launch_decode_cascade(kv_dtype, fp8, a, cg.cu, cg.prefix_lens, cg.n_groups,
                                 cg.max_group_size, cg.max_prefix_len, workspace, workspace_bytes,
                                 static_cast<hipStream_t>(stream));
  if (use_scratch) {
    // Size the states for the waves the launches will really run on this
    // device (the same grids as with a caller's workspace, hence the same
    // bits), then place them in the static scratch.
    void* ptr = nullptr;
    pkv_status st = scratch_address(&ptr);
    if (st != PKV_OK) return st;
    int waves = 0;
    st = launch_decode(kv_dtype, fp8, plan, a, static_cast<hipStream_t>(stream), &waves);
    if (st != PKV_OK) return st;
    if (waves < plan.max_waves) layout_decode_workspace(&plan, waves);
    PKV_REQUIRE(plan.workspace_bytes <= kNoAllocScratchBytes, PKV_ERR_WORKSPACE,
                "decode_noalloc: %zu bytes of partial states needed, the static scratch holds "
                "%zu (fewer sequences per call, or pkv_paged_attention_decode with a workspace)",
                plan.workspace_bytes, kNoAllocScratchBytes);
    attach_decode_workspace(&a, plan, ptr);
  }
  return launch_decode(kv_dtype, fp8, plan, a, static_cast<hipStream_t>(stream));
}

extern "C" {

pkv_status pkv_paged_attention_decode(void* out, pkv_dtype out_dtype, const void* q,
                                      const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t max_context_len,
                                      int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                      float scale, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  return decode_impl(out, out_dtype, q, kv_dtype, false, k_cache, v_cache, nullptr, nullptr,
                     block_tables, max_blocks_per_seq, context_lens, max_context_len, S, Hq, Hkv,
                     D, B, scale, workspace, workspace_bytes, stream);
}

pkv_status pkv_paged_attention_decode_noalloc(void* out, pkv_dtype out_dtype, const void* q,
                                              const void* k_cache, const void* v_cache,
                                              pkv_dtype kv_dtype, const int32_t* block_tables,
                                              int32_t max_blocks_per_seq,
                                              const int32_t* context_lens, int32_t max_context_len,
                                              int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                                              int32_t B, float scale, void* stream) {
  return decode_impl(out, out_dtype, q, kv_dtype, false, k_cache, v_cache, nullptr, nullptr,
                     block_tables, max_blocks_per_seq, context_lens, max_context_len, S, Hq, Hkv,
                     D, B, scale, nullptr, 0, stream, CascadeGroups(), true);
}

pkv_status pkv_decode_step(void* out, pkv_dtype out_dtype, const void* q, const void* key,
                           const void* value, const int64_t* slot_mapping, void* k_cache,
                           void* v_cache, int64_t NB, pkv_dtype kv_dtype,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t max_context_len, int32_t S,
                           int32_t Hq, int32_t Hkv, int32_t D, int32_t B, float scale,
                           void* workspace, size_t workspace_bytes, void* stream) {
  const StepTokens step{key, value, slot_mapping, NB};
  return decode_impl(out, out_dtype, q, kv_dtype, false, k_cache, v_cache, nullptr, nullptr,
                     block_tables, max_blocks_per_seq, context_lens, max_context_len, S, Hq, Hkv,
                     D, B, scale, workspace, workspace_bytes, stream, CascadeGroups(), false,
                     &step);
}

pkv_status pkv_decode_cascade_workspace_size(int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                                             int32_t B, int32_t max_context_len, int32_t n_groups,
                                             int32_t max_group_size, int32_t max_prefix_len,
                                             pkv_dtype kv_dtype, size_t* bytes) {
  g_last_error[0] = 0;
  PKV_REQUIRE(bytes, PKV_ERR_INVALID_ARG, "decode_cascade_workspace_size: null output");
  PKV_REQUIRE(S >= 0 && Hq > 0 && Hkv > 0 && D > 0 && B > 0 && max_context_len >= 0 &&
                  n_groups >= 0 && max_group_size >= 1 && max_prefix_len >= 0,
              PKV_ERR_INVALID_ARG, "decode_cascade_workspace_size: bad sizes");
  PKV_REQUIRE(Hq % Hkv == 0, PKV_ERR_INVALID_ARG, "decode_cascade_workspace_size: Hq %% Hkv != 0");
  PKV_REQUIRE(supported_dtype(kv_dtype), PKV_ERR_UNSUPPORTED,
              "decode_cascade_workspace_size: dtype %d", (int)kv_dtype);
  if (S == 0) {
    *bytes = 0;
    return PKV_OK;
  }
  return cascade_workspace_size(S, Hq, Hkv, D, B, max_context_len, n_groups, max_group_size,
                                max_prefix_len, kv_dtype, bytes);
}

pkv_status pkv_paged_attention_decode_cascade(
    void* out, pkv_dtype out_dtype, const void* q, const void* k_cache, const void* v_cache,
    pkv_dtype kv_dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t max_context_len, int32_t S, int32_t Hq, int32_t Hkv,
    int32_t D, int32_t B, float scale, const int32_t* cu_group_seqs,
    const int32_t* group_prefix_lens, int32_t n_groups, int32_t max_group_size,
    int32_t max_prefix_len, void* workspace, size_t workspace_bytes, void* stream) {
  CascadeGroups cg;
  cg.on = true;
  cg.cu = cu_group_seqs;
  cg.prefix_lens = group_prefix_lens;
  cg.n_groups = n_groups;
  cg.max_group_size = max_group_size;
  cg.max_prefix_len = max_prefix_len;
  return decode_impl(out, out_dtype, q, kv_dtype, false, k_cache, v_cache, nullptr, nullptr,
                     block_tables, max_blocks_per_seq, context_lens, max_context_len, S, Hq, Hkv,
                     D, B, scale, workspace, workspace_bytes, stream, cg);
}

pkv_status pkv_paged_attention_decode_cascade_fp8(
    void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype, const void* k_cache,
    const void* v_cache, const float* k_scale, const float* v_scale, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len, int32_t S,
    int32_t Hq, int32_t Hkv, int32_t D, int32_t B, float scale, const int32_t* cu_group_seqs,
    const int32_t* group_prefix_lens, int32_t n_groups, int32_t max_group_size,
    int32_t max_prefix_len, void* workspace, size_t workspace_bytes, void* stream) {
  CascadeGroups cg;
  cg.on = true;
  cg.cu = cu_group_seqs;
  cg.prefix_lens = group_prefix_lens;
  cg.n_groups = n_groups;
  cg.max_group_size = max_group_size;
  cg.max_prefix_len = max_prefix_len;
  return decode_impl(out, out_dtype, q, q_dtype, true, k_cache, v_cache, k_scale, v_scale,
                     block_tables, max_blocks_per_seq, context_lens, max_context_len, S, Hq, Hkv,
                     D, B, scale, workspace, workspace_bytes, stream, cg);
}

pkv_status pkv_paged_attention_decode_fp8(void* out, pkv_dtype out_dtype, const void* q,
                                          pkv_dtype q_dtype, const void* k_cache,
                                          const void* v_cache, const float* k_scale,
                                          const float* v_scale, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                                          int32_t max_context_len, int32_t S, int32_t Hq,
                                          int32_t Hkv, int32_t D, int32_t B, float scale,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, out_dtype, q, q_dtype, true, k_cache, v_cache, k_scale, v_scale,
                     block_tables, max_blocks_per_seq, context_lens, max_context_len, S, Hq, Hkv,
                     D, B, scale, workspace, workspace_bytes, stream);
}

}  // extern "C"

// Validates the prefill arguments and fills *a; *empty: nothing to compute.
// kv_dtype is q's dtype; fp8: the pools hold E4M3 codes with per-head scales.
static pkv_status prefill_args(void* out, pkv_dtype out_dtype, const void* q,
                               const int32_t* cu_seqlens_q, int32_t Tq, int32_t max_query_len,
                               const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                               bool fp8, const float* k_scale, const float* v_scale,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t max_context_len, int32_t S,
                               int32_t Hq, int32_t Hkv, int32_t D, int32_t B, float scale,
                               PrefillArgs* a, bool* empty) {
  *empty = true;
  PKV_REQUIRE(S >= 0 && Tq >= 0 && max_query_len >= 0 && Hq > 0 && Hkv > 0 && D > 0 && B > 0,
              PKV_ERR_INVALID_ARG, "prefill: S=%d Tq=%d max_query_len=%d Hq=%d Hkv=%d D=%d B=%d",
              S, Tq, max_query_len, Hq, Hkv, D, B);
  PKV_REQUIRE(Hq % Hkv == 0, PKV_ERR_INVALID_ARG, "prefill: Hq (%d) not a multiple of Hkv (%d)",
              Hq, Hkv);
  PKV_REQUIRE(max_query_len <= max_context_len || Tq == 0, PKV_ERR_INVALID_ARG,
              "prefill: max_query_len %d > max_context_len %d", max_query_len, max_context_len);
  PKV_REQUIRE(supported_dtype(kv_dtype) && supported_dtype(out_dtype), PKV_ERR_UNSUPPORTED,
              "prefill: dtypes kv=%d out=%d", (int)kv_dtype, (int)out_dtype);
  PKV_REQUIRE(supported_head_dim(D), PKV_ERR_UNSUPPORTED, "prefill: head_dim %d", D);
  PKV_REQUIRE(supported_block(B), PKV_ERR_UNSUPPORTED, "prefill: block_size %d", B);
  PKV_REQUIRE((int64_t)max_context_len <= (int64_t)max_blocks_per_seq * B, PKV_ERR_INVALID_ARG,
              "prefill: max_context_len %d exceeds table capacity %d x %d", max_context_len,
              max_blocks_per_seq, B);
  PKV_REQUIRE(scale == scale, PKV_ERR_INVALID_ARG, "prefill: scale is NaN");
  PKV_REQUIRE(!fp8 || kv_dtype != PKV_F32, PKV_ERR_UNSUPPORTED, "prefill_fp8: q must be f16 or bf16");
  PKV_REQUIRE((int64_t)B * Hkv * D * (fp8 ? 1 : dt_bytes(kv_dtype)) < ((int64_t)1 << 31),
              PKV_ERR_UNSUPPORTED, "prefill: one block of one pool must be smaller than 2 GiB");
  PKV_REQUIRE(!fp8 || (B >= 8 && Hq / Hkv <= 128), PKV_ERR_UNSUPPORTED,
              "prefill_fp8: needs block_size >= 8 and at most 128 query heads per KV head "
              "(B=%d, G=%d)", B, Hq / Hkv);
  if (S == 0 || Tq == 0) return PKV_OK;
  *empty = false;
  PKV_REQUIRE(out && q && cu_seqlens_q && k_cache && v_cache && block_tables && context_lens,
              PKV_ERR_INVALID_ARG, "prefill: null pointer");
  PKV_REQUIRE(!fp8 || (k_scale && v_scale), PKV_ERR_INVALID_ARG, "prefill_fp8: null scale array");
  PKV_REQUIRE(aligned(out, 16) && aligned(q, 16) && aligned(k_cache, 16) && aligned(v_cache, 16),
              PKV_ERR_INVALID_ARG, "prefill: out, q and the pools must be 16-byte aligned");
  PKV_REQUIRE(aligned(cu_seqlens_q, 4) && aligned(block_tables, 4) && aligned(context_lens, 4) &&
                  aligned(k_scale, 4) && aligned(v_scale, 4),
              PKV_ERR_INVALID_ARG,
              "prefill: index arrays and scales must be aligned to their element size");
  a->out = out;
  a->q = q;
  a->cu_seqlens_q = cu_seqlens_q;
  a->cu_base = 0;
  a->k_cache = k_cache;
  a->v_cache = v_cache;
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->max_nb = max_blocks_per_seq;
  a->Tq = Tq;
  a->max_query_len = max_query_len;
  a->S = S;
  a->Hq = Hq;
  a->Hkv = Hkv;
  a->D = D;
  a->B = B;
  a->log2B = ilog2(B);
  a->max_ctx = max_context_len;
  a->out_dt = out_dtype;
  a->scale_log2 = scale * 1.4426950408889634f;
  a->n_split = 1;
  a->tiles_per_split = 0;
  a->ws_o = nullptr;
  a->ws_ml = nullptr;
  a->q_dt = kv_dtype;
  a->k_scale = fp8 ? k_scale : nullptr;
  a->v_scale = fp8 ? v_scale : nullptr;
  return PKV_OK;
}

// Points a at its split plan and workspace (ws: plan.workspace_bytes bytes).
static void attach_prefill_plan(const PrefillPlan& plan, void* ws, PrefillArgs* a) {
  a->n_split = plan.n_split;
  a->tiles_per_split = plan.tiles_per_split;
  if (plan.n_split > 1) {
    a->ws_o = static_cast<float*>(ws);
    a->ws_ml = a->ws_o + (size_t)plan.n_split * a->Tq * a->Hq * a->D;
  }
}

extern "C" {

pkv_status pkv_prefill_workspace_size(int32_t S, int32_t Tq, int32_t max_query_len, int32_t Hq,
                                      int32_t Hkv, int32_t D, int32_t B, pkv_dtype kv_dtype,
                                      int32_t max_context_len, size_t* bytes) {
  g_last_error[0] = 0;
  PKV_REQUIRE(bytes, PKV_ERR_INVALID_ARG, "prefill_workspace_size: null output");
  PKV_REQUIRE(S >= 0 && Tq >= 0 && max_query_len >= 0 && Hq > 0 && Hkv > 0 && D > 0 && B > 0 &&
                  max_context_len >= 0 && Hq % Hkv == 0,
              PKV_ERR_INVALID_ARG, "prefill_workspace_size: bad sizes");
  *bytes = plan_prefill(kv_dtype, S, Tq, max_query_len, Hq, Hkv, D, B, max_context_len).workspace_bytes;
  return PKV_OK;
}

pkv_status pkv_paged_attention_prefill(void* out, pkv_dtype out_dtype, const void* q,
                                       const int32_t* cu_seqlens_q, int32_t Tq,
                                       int32_t max_query_len, const void* k_cache,
                                       const void* v_cache, pkv_dtype kv_dtype,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t max_context_len,
                                       int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                       float scale, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  g_last_error[0] = 0;
  PrefillArgs a;
  bool empty = true;
  const pkv_status st = prefill_args(out, out_dtype, q, cu_seqlens_q, Tq, max_query_len, k_cache,
                                     v_cache, kv_dtype, false, nullptr, nullptr, block_tables,
                                     max_blocks_per_seq, context_lens, max_context_len, S, Hq, Hkv,
                                     D, B, scale, &a, &empty);
  if (st != PKV_OK || empty) return st;
  const PrefillPlan plan = plan_prefill(kv_dtype, S, Tq, max_query_len, Hq, Hkv, D, B, max_context_len);
  PKV_REQUIRE(plan.workspace_bytes == 0 || (workspace && workspace_bytes >= plan.workspace_bytes),
              PKV_ERR_WORKSPACE, "prefill: workspace of %zu bytes needed, %zu given",
              plan.workspace_bytes, workspace ? workspace_bytes : (size_t)0);
  PKV_REQUIRE(aligned(workspace, 16), PKV_ERR_INVALID_ARG,
              "prefill: the workspace must be 16-byte aligned");
  attach_prefill_plan(plan, workspace, &a);
  return launch_prefill(kv_dtype, a, static_cast<hipStream_t>(stream));
}

pkv_status pkv_paged_attention_prefill_fp8(void* out, pkv_dtype out_dtype, const void* q,
                                           pkv_dtype q_dtype, const int32_t* cu_seqlens_q,
                                           int32_t Tq, int32_t max_query_len, const void* k_cache,
                                           const void* v_cache, const float* k_scale,
                                           const float* v_scale, const int32_t* block_tables,
                                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                                           int32_t max_context_len, int32_t S, int32_t Hq,
                                           int32_t Hkv, int32_t D, int32_t B, float scale,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  PrefillArgs a;
  bool empty = true;
  const pkv_status st = prefill_args(out, out_dtype, q, cu_seqlens_q, Tq, max_query_len, k_cache,
                                     v_cache, q_dtype, true, k_scale, v_scale, block_tables,
                                     max_blocks_per_seq, context_lens, max_context_len, S, Hq, Hkv,
                                     D, B, scale, &a, &empty);
  if (st != PKV_OK || empty) return st;
  const PrefillPlan plan = plan_prefill(DT_FP8, S, Tq, max_query_len, Hq, Hkv, D, B, max_context_len);
  PKV_REQUIRE(plan.workspace_bytes == 0 || (workspace && workspace_bytes >= plan.workspace_bytes),
              PKV_ERR_WORKSPACE, "prefill_fp8: workspace of %zu bytes needed, %zu given",
              plan.workspace_bytes, workspace ? workspace_bytes : (size_t)0);
  PKV_REQUIRE(aligned(workspace, 16), PKV_ERR_INVALID_ARG,
              "prefill_fp8: the workspace must be 16-byte aligned");
  attach_prefill_plan(plan, workspace, &a);
  return launch_prefill(DT_FP8, a, static_cast<hipStream_t>(stream));
}

pkv_status pkv_mixed_workspace_size(int32_t S, int32_t num_decode, int32_t Tq,
                                    int32_t max_query_len, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t B, pkv_dtype kv_dtype, int32_t max_context_len,
                                    size_t* bytes) {
  g_last_error[0] = 0;
  PKV_REQUIRE(bytes, PKV_ERR_INVALID_ARG, "mixed_workspace_size: null output");
  PKV_REQUIRE(S >= 0 && num_decode >= 0 && num_decode <= S && Tq >= num_decode &&
                  max_query_len >= 0 && Hq > 0 && Hkv > 0 && D > 0 && B > 0 &&
                  max_context_len >= 0 && Hq % Hkv == 0,
              PKV_ERR_INVALID_ARG, "mixed_workspace_size: bad sizes");
  DecodePlan plan{};
  if (num_decode > 0) {
    const pkv_status st = plan_decode(num_decode, Hq, Hkv, D, B, max_context_len, &plan);
    if (st != PKV_OK) return st;
  }
  const PrefillPlan pplan = plan_prefill(kv_dtype, S - num_decode, Tq - num_decode, max_query_len,
                                         Hq, Hkv, D, B, max_context_len);
  *bytes = mixed_workspace_size(plan, pplan);
  return PKV_OK;
}

}  // extern "C"

// Mixed batch; kv_dtype is q's dtype, fp8: E4M3 pools with per-head scales.
static pkv_status mixed_impl(void* out, pkv_dtype out_dtype, const void* q,
                             const int32_t* cu_seqlens_q, int32_t Tq, int32_t num_decode,
                             int32_t max_query_len, const void* k_cache, const void* v_cache,
                             pkv_dtype kv_dtype, bool fp8, const float* k_scale,
                             const float* v_scale, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t max_context_len, int32_t S, int32_t Hq, int32_t Hkv,
                             int32_t D, int32_t B, float scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  PKV_REQUIRE(num_decode >= 0 && num_decode <= S && num_decode <= Tq, PKV_ERR_INVALID_ARG,
              "mixed: num_decode %d outside [0, min(S=%d, Tq=%d)]", num_decode, S, Tq);
  PrefillArgs pa;
  bool empty = true;
  pkv_status st = prefill_args(out, out_dtype, q, cu_seqlens_q, Tq, max_query_len, k_cache,
                               v_cache, kv_dtype, fp8, k_scale, v_scale, block_tables,
                               max_blocks_per_seq, context_lens, max_context_len, S, Hq, Hkv, D, B,
                               scale, &pa, &empty);
  if (st != PKV_OK || empty) return st;
  DecodePlan plan{};
  if (num_decode > 0) {
    st = plan_decode(num_decode, Hq, Hkv, D, B, max_context_len, &plan);
    if (st != PKV_OK) return st;
  }
  const PrefillPlan pplan = plan_prefill(fp8 ? (int)DT_FP8 : (int)kv_dtype, S - num_decode,
                                         Tq - num_decode, max_query_len, Hq, Hkv, D, B,
                                         max_context_len);
  const size_t need = mixed_workspace_size(plan, pplan);
  PKV_REQUIRE(workspace && workspace_bytes >= need, PKV_ERR_WORKSPACE,
              "mixed: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  PKV_REQUIRE(aligned(workspace, 16), PKV_ERR_INVALID_ARG,
              "mixed: the workspace must be 16-byte aligned");
  DecodeArgs da{};
  da.out = out;
  da.q = q;
  da.k_cache = k_cache;
  da.v_cache = v_cache;
  da.block_tables = block_tables;
  da.context_lens = context_lens;
  attach_decode_workspace(&da, plan, workspace);
  da.max_nb = max_blocks_per_seq;
  da.S = num_decode;
  da.Hq = Hq;
  da.Hkv = Hkv;
  da.D = D;
  da.B = B;
  da.log2B = ilog2(B);
  da.max_ctx = max_context_len;
  da.out_dt = out_dtype;
  da.scale_log2 = scale * 1.4426950408889634f;
  da.k_scale = fp8 ? k_scale : nullptr;
  da.v_scale = fp8 ? v_scale : nullptr;
  pa.S = S - num_decode;
  return launch_mixed(kv_dtype, fp8, plan, pplan, da, pa, num_decode, workspace,
                      static_cast<hipStream_t>(stream));
}

extern "C" {

pkv_status pkv_paged_attention_mixed(void* out, pkv_dtype out_dtype, const void* q,
                                     const int32_t* cu_seqlens_q, int32_t Tq, int32_t num_decode,
                                     int32_t max_query_len, const void* k_cache,
                                     const void* v_cache, pkv_dtype kv_dtype,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, int32_t max_context_len,
                                     int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                     float scale, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  return mixed_impl(out, out_dtype, q, cu_seqlens_q, Tq, num_decode, max_query_len, k_cache,
                    v_cache, kv_dtype, false, nullptr, nullptr, block_tables, max_blocks_per_seq,
                    context_lens, max_context_len, S, Hq, Hkv, D, B, scale, workspace,
                    workspace_bytes, stream);
}

pkv_status pkv_paged_attention_mixed_fp8(void* out, pkv_dtype out_dtype, const void* q,
                                         pkv_dtype q_dtype, const int32_t* cu_seqlens_q,
                                         int32_t Tq, int32_t num_decode, int32_t max_query_len,
                                         const void* k_cache, const void* v_cache,
                                         const float* k_scale, const float* v_scale,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t max_context_len,
                                         int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                         float scale, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  return mixed_impl(out, out_dtype, q, cu_seqlens_q, Tq, num_decode, max_query_len, k_cache,
                    v_cache, q_dtype, true, k_scale, v_scale, block_tables, max_blocks_per_seq,
                    context_lens, max_context_len, S, Hq, Hkv, D, B, scale, workspace,
                    workspace_bytes, stream);
}


}  // extern "C"

// Address a kernel may use for p: device memory as is, pinned host memory
// through its device mapping.  Pageable host memory (or anything HIP does not
// know) is refused: a kernel touching it would fault.
static pkv_status device_view(const void* p, const void** out, const char* what) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PKV_ERR_INVALID_ARG, "%s: %p is neither device nor pinned host memory", what, p);
  }
  if (attr.type == hipMemoryTypeHost) {
    unsigned flags = 0;  // only page-locked (pinned) host memory has host flags
    if (!attr.devicePointer || hipHostGetFlags(&flags, const_cast<void*>(p)) != hipSuccess) {
      (void)hipGetLastError();
      return fail(PKV_ERR_INVALID_ARG, "%s: %p is neither device nor pinned host memory", what, p);
    }
    *out = attr.devicePointer;
  } else if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged ||
             attr.type == hipMemoryTypeUnified) {
    *out = p;
  } else {
    return fail(PKV_ERR_INVALID_ARG, "%s: %p is neither device nor pinned host memory", what, p);
  }
  return PKV_OK;
}

extern "C" {

pkv_status pkv_swap_blocks(const void* const* src_pools, void* const* dst_pools, int32_t num_pools,
                           const int64_t* block_pairs, int32_t N, int32_t B, int32_t Hkv,
                           int32_t D, pkv_dtype kv_dtype, void* stream) {
  g_last_error[0] = 0;
  PKV_REQUIRE(num_pools >= 0 && N >= 0 && B > 0 && Hkv > 0 && D > 0, PKV_ERR_INVALID_ARG,
              "swap_blocks: pools=%d N=%d B=%d Hkv=%d D=%d", num_pools, N, B, Hkv, D);
  PKV_REQUIRE(supported_dtype(kv_dtype) || kv_dtype == PKV_FP8_E4M3, PKV_ERR_UNSUPPORTED,
              "swap_blocks: dtype %d", (int)kv_dtype);
  PKV_REQUIRE(supported_head_dim(D), PKV_ERR_UNSUPPORTED, "swap_blocks: head_dim %d", D);
  PKV_REQUIRE(supported_block(B), PKV_ERR_UNSUPPORTED, "swap_blocks: block_size %d", B);
  if (N == 0 || num_pools == 0) return PKV_OK;
  PKV_REQUIRE(src_pools && dst_pools && block_pairs, PKV_ERR_INVALID_ARG, "swap_blocks: null pointer");
  PKV_REQUIRE(aligned(block_pairs, 8), PKV_ERR_INVALID_ARG,
              "swap_blocks: block_pairs must be 8-byte aligned");
  for (int32_t i = 0; i < num_pools; ++i) {
    PKV_REQUIRE(src_pools[i] && dst_pools[i], PKV_ERR_INVALID_ARG, "swap_blocks: null pool %d", i);
    PKV_REQUIRE(aligned(src_pools[i], 16) && aligned(dst_pools[i], 16), PKV_ERR_INVALID_ARG,
                "swap_blocks: pool %d is not 16-byte aligned", i);
  }
  std::vector<const void*> src(num_pools);
  std::vector<void*> dst(num_pools);
  for (int32_t i = 0; i < num_pools; ++i) {
    const void* d = nullptr;
    pkv_status st = device_view(src_pools[i], &src[i], "swap_blocks (source pool)");
    if (st != PKV_OK) return st;
    st = device_view(dst_pools[i], &d, "swap_blocks (destination pool)");
    if (st != PKV_OK) return st;
    dst[i] = const_cast<void*>(d);
  }
  const void* pairs = nullptr;
  const pkv_status st = device_view(block_pairs, &pairs, "swap_blocks (pairs)");
  if (st != PKV_OK) return st;
  const int64_t block_bytes = (int64_t)B * Hkv * D * dt_bytes(kv_dtype);
  return launch_swap_blocks(src.data(), dst.data(), num_pools, static_cast<const int64_t*>(pairs),
                            N, block_bytes, static_cast<hipStream_t>(stream));
}

pkv_status pkv_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                           const int64_t* block_pairs, int32_t N, int32_t B, int32_t Hkv,
                           int32_t D, pkv_dtype kv_dtype, void* stream) {
  g_last_error[0] = 0;
  PKV_REQUIRE(num_layers >= 0 && N >= 0 && B > 0 && Hkv > 0 && D > 0, PKV_ERR_INVALID_ARG,
              "copy_blocks: layers=%d N=%d B=%d Hkv=%d D=%d", num_layers, N, B, Hkv, D);
  PKV_REQUIRE(supported_dtype(kv_dtype) || kv_dtype == PKV_FP8_E4M3, PKV_ERR_UNSUPPORTED,
              "copy_blocks: dtype %d", (int)kv_dtype);
  PKV_REQUIRE(supported_head_dim(D), PKV_ERR_UNSUPPORTED, "copy_blocks: head_dim %d", D);
  PKV_REQUIRE(supported_block(B), PKV_ERR_UNSUPPORTED, "copy_blocks: block_size %d", B);
  if (N == 0 || num_layers == 0) return PKV_OK;
  PKV_REQUIRE(k_caches && v_caches && block_pairs, PKV_ERR_INVALID_ARG, "copy_blocks: null pointer");
  PKV_REQUIRE(aligned(block_pairs, 8), PKV_ERR_INVALID_ARG,
              "copy_blocks: block_pairs must be 8-byte aligned");
  for (int32_t l = 0; l < num_layers; ++l) {
    PKV_REQUIRE(k_caches[l] && v_caches[l], PKV_ERR_INVALID_ARG, "copy_blocks: null pool, layer %d",
                l);
    PKV_REQUIRE(aligned(k_caches[l], 16) && aligned(v_caches[l], 16), PKV_ERR_INVALID_ARG,
                "copy_blocks: pool of layer %d is not 16-byte aligned", l);
  }
  const int64_t block_bytes = (int64_t)B * Hkv * D * dt_bytes(kv_dtype);
  return launch_copy_blocks(k_caches, v_caches, num_layers, block_pairs, N, block_bytes,
                            static_cast<hipStream_t>(stream));
}

}  // extern "C"
