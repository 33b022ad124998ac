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
// Design: the two parts run one after the other on the caller's stream, the
// decode part (split + merge kernels, bound by HBM) and then the chunks
// (tile kernel on the matrix cores).  A chunk too small to fill the GPU by
// itself -- one long prompt's 512 tokens are 128 workgroups -- has its KV
// range split across the whole GPU (prefill's split plan), so neither part
// leaves CUs idle.  Running the two concurrently on two streams was measured
// slower (444 us against 425 us on 256 Llama-3-8B decodes + one 512-token
// chunk after 8192 tokens): the decode kernels need the same SIMD issue
// slots as the chunk's matrix-core work, and their fixed per-workgroup
// shares stretch when workgroups of the other kernel share their CUs.
#include "pkv_internal.h"

namespace pkv {
namespace {

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// Workspace: the decode part's, then the chunks' split partial results (when
// their plan splits).
size_t mixed_workspace_size(const DecodePlan& plan, const PrefillPlan& pplan) {
  return align_up(plan.workspace_bytes) + pplan.workspace_bytes;
}

pkv_status launch_mixed(int kv_dt, bool fp8, const DecodePlan& plan, const PrefillPlan& pplan,
                        const DecodeArgs& dec, const PrefillArgs& pre, int32_t num_decode,
                        void* workspace, hipStream_t stream) {
  const int32_t S_p = pre.S;
  char* ws_split = static_cast<char*>(workspace) + align_up(plan.workspace_bytes);
  if (S_p == 0) return dec.S ? launch_decode(kv_dt, fp8, plan, dec, stream) : PKV_OK;

  PrefillArgs p = pre;
  const int es = dt_bytes(kv_dt), oes = dt_bytes(pre.out_dt);
  p.q = static_cast<const char*>(pre.q) + (int64_t)num_decode * pre.Hq * pre.D * es;
  p.out = static_cast<char*>(pre.out) + (int64_t)num_decode * pre.Hq * pre.D * oes;
  // the chunks' boundaries, counted from their first row (row num_decode)
  p.cu_seqlens_q = pre.cu_seqlens_q + num_decode;
  p.cu_base = num_decode;
  p.Tq = pre.Tq - num_decode;
  p.block_tables = pre.block_tables + (int64_t)num_decode * pre.max_nb;
  p.context_lens = pre.context_lens + num_decode;
  p.n_split = pplan.n_split;
  p.tiles_per_split = pplan.tiles_per_split;
  if (pplan.n_split > 1) {
    p.ws_o = reinterpret_cast<float*>(ws_split);
    p.ws_ml = p.ws_o + (size_t)pplan.n_split * p.Tq * p.Hq * p.D;
  }

  if (dec.S > 0) {
    const pkv_status sd = launch_decode(kv_dt, fp8, plan, dec, stream);
    if (sd != PKV_OK) return sd;
  }
  return launch_prefill(fp8 ? (int)DT_FP8 : kv_dt, p, stream);
}

}  // namespace pkv
