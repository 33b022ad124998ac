// mixed.hip -- one call for a batch that mixes decode requests and prefill
// chunks ("LLM inference, part 3: single node", ch. 13 sec. 1: one flattened
// token stream with cu_seqlens boundaries for requests of one token (decode)
// and of many (prefill); sec. 2: a chunk of a long prompt is packed with the
// running decodes in one batch, so the bandwidth-bound decodes and the
// compute-bound chunk fill the GPU together).
//
// Layout contract: the first num_decode sequences are decodes (one query row
// each, rows 0 .. num_decode - 1); the rest are prefill chunks.  Every output
// row is what paged_attention_decode / paged_attention_prefill give for it.
//
// Design: the two parts run concurrently.  The decode part (split + merge
// kernels, about one workgroup per CU on the matrix-core path, bound by HBM)
// goes on the caller's stream; the prefill part (tile kernel, bound by the
// matrix cores) on a library-owned stream of default priority, forked from
// and joined back into the caller's stream with events.  A CU holds a decode
// workgroup and a prefill workgroup at once, so the two share every CU.
#include <mutex>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kMaxDevices = 64;

struct AuxStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
AuxStream g_aux[kMaxDevices];
std::mutex g_aux_mutex;  // also orders the fork / launch / join of concurrent calls

pkv_status aux_for_current_device(AuxStream** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_HIP, "mixed: cannot query the current device");
  AuxStream& a = g_aux[dev];
  if (!a.s) {
    if (hipStreamCreateWithFlags(&a.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&a.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&a.join, hipEventDisableTiming) != hipSuccess)
      return fail(PKV_ERR_HIP, "mixed: cannot create the auxiliary stream");
  }
  *out = &a;
  return PKV_OK;
}

// cu_out[i] = cu[num_decode + i] - num_decode, i <= S_p (the prefill chunks'
// boundaries counted from their first row)
__global__ void rebase_cu_kernel(const int32_t* __restrict__ cu, int32_t num_decode, int32_t S_p,
                                 int32_t* __restrict__ cu_out) {
  for (int i = threadIdx.x; i <= S_p; i += blockDim.x) cu_out[i] = cu[num_decode + i] - num_decode;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t mixed_workspace_size(const DecodePlan& plan, int32_t S_prefill) {
  return align_up(plan.workspace_bytes) + ((size_t)S_prefill + 1) * sizeof(int32_t);
}

pkv_status launch_mixed(int kv_dt, const DecodePlan& plan, const DecodeArgs& dec,
                        const PrefillArgs& pre, int32_t num_decode, void* workspace,
                        hipStream_t stream) {
  const int32_t S_p = pre.S;
  char* ws = static_cast<char*>(workspace);
  int32_t* cu_p = reinterpret_cast<int32_t*>(ws + align_up(plan.workspace_bytes));
  if (S_p == 0) return dec.S ? launch_decode(kv_dt, false, plan, dec, stream) : PKV_OK;

  PrefillArgs p = pre;
  const int es = dt_bytes(kv_dt), oes = dt_bytes(pre.out_dt);
  p.q = static_cast<const char*>(pre.q) + (int64_t)num_decode * pre.Hq * pre.D * es;
  p.out = static_cast<char*>(pre.out) + (int64_t)num_decode * pre.Hq * pre.D * oes;
  p.cu_seqlens_q = cu_p;
  p.Tq = pre.Tq - num_decode;
  p.block_tables = pre.block_tables + (int64_t)num_decode * pre.max_nb;
  p.context_lens = pre.context_lens + num_decode;

  if (dec.S == 0) {
    hipLaunchKernelGGL(rebase_cu_kernel, dim3(1), dim3(256), 0, stream, pre.cu_seqlens_q, num_decode,
                       S_p, cu_p);
    const pkv_status st = check_launch("mixed (rebase)");
    return st != PKV_OK ? st : launch_prefill(kv_dt, p, stream);
  }

  std::lock_guard<std::mutex> lock(g_aux_mutex);
  AuxStream* aux = nullptr;
  pkv_status st = aux_for_current_device(&aux);
  if (st != PKV_OK) return st;
  // fork: the prefill part waits for everything queued on the caller's stream
  if (hipEventRecord(aux->fork, stream) != hipSuccess ||
      hipStreamWaitEvent(aux->s, aux->fork, 0) != hipSuccess)
    return fail(PKV_ERR_HIP, "mixed: fork failed");
  hipLaunchKernelGGL(rebase_cu_kernel, dim3(1), dim3(256), 0, aux->s, pre.cu_seqlens_q, num_decode,
                     S_p, cu_p);
  st = check_launch("mixed (rebase)");
  if (st == PKV_OK) st = launch_prefill(kv_dt, p, aux->s);
  const pkv_status sd = launch_decode(kv_dt, false, plan, dec, stream);
  // join: the caller's stream waits for the prefill part (also after a failed
  // launch, so nothing is left behind on the auxiliary stream unordered)
  if (hipEventRecord(aux->join, aux->s) != hipSuccess ||
      hipStreamWaitEvent(stream, aux->join, 0) != hipSuccess)
    return fail(PKV_ERR_HIP, "mixed: join failed");
  return st != PKV_OK ? st : sd;
}

}  // namespace pkv
