// cascade.hip -- decode for groups of sequences that share a prefix of blocks.
//
// What is computed: exactly paged_attention_decode -- one softmax over every
// cached token of each sequence (CS349D lecture 3 sec. 3.2) -- for a batch
// whose sequences come in groups (the samples forked from one prompt) that
// alias the same leading blocks (CS349D lecture 3 sec. 4.1: fork shares the
// parent's blocks).  The S06 PagedAttention chapter ("in production" section)
// and CMU 11-868 lecture 24 (sec. 7.3 and further reading, cascade inference)
// describe the point: batch the shared prefix apart from the forked suffixes,
// so the prefix is read once per group instead of once per member, and merge
// the two partial softmaxes.
//
// Design (three steps on the caller's stream):
//  1. gather: per group, the members' queries laid out [kv head][member][query
//     head of the KV group], so that the group becomes one pseudo-sequence
//     with max_group_size * Hq query heads whose GQA mapping is the ordinary
//     one (head j -> KV head j / (max_group_size * G)); its table is the
//     first member's table truncated to the prefix.  Each member's suffix
//     starts at the prefix length.
//  2. two decode passes with the decode kernels: the pseudo-sequences over
//     their prefixes, and every sequence over its suffix (tokens from the
//     prefix length on); both write fp32 outputs and the log2-sum-exp of the
//     scaled scores per head.
//  3. combine: out = (o_p 2^lse_p + o_s 2^lse_s) / (2^lse_p + 2^lse_s) per
//     (sequence, head), the same merge as the decode partitions use; an empty
//     side has lse = -inf and weight 0.
// Members beyond a group's size are padded with copies of its last member
// (their results are never read).
#include "pkv_internal.h"

#include <math.h>

namespace pkv {
namespace {

constexpr int kThreads = 256;

struct CascadeLayout {
  size_t qg, ptab, plens, seq_start, seq_group, o_p, lse_p, o_s, lse_s, ws_p, ws_s, total;
  DecodePlan plan_p, plan_s;
  int max_pnb;
  int max_prefix_len;  // the host bound, cut to the longest context
};

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kGatherSplit = 8;  // workgroups per group for the query copy

// grid = (groups, kGatherSplit): workgroup (g, y) copies every kGatherSplit-th
// stretch of group g's query rows; y = 0 also writes the group's prefix
// length, its table and its members' suffix starts and group index.
__global__ __launch_bounds__(kThreads) void cascade_gather_kernel(
    const char* __restrict__ q, const int32_t* __restrict__ cu, const int32_t* __restrict__ plen,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ context_lens, int32_t max_nb,
    char* __restrict__ qg, int32_t* __restrict__ ptab, int32_t max_pnb,
    int32_t* __restrict__ plens, int32_t* __restrict__ seq_start, int32_t* __restrict__ seq_group,
    int32_t NM, int32_t Hq, int32_t Hkv, int32_t D, int32_t B, int32_t es, int32_t max_prefix) {
  const int g = blockIdx.x;
  const int s0 = cu[g];
  const int n = cu[g + 1] - s0;
  if (n <= 0) {  // empty group: nothing of it is ever read
    if (threadIdx.x == 0 && blockIdx.y == 0) plens[g] = 0;
    return;
  }
  const int G = Hq / Hkv;
  const int chunks = D * es / 16;  // 16-byte chunks per query row
  const int rows = Hkv * NM * G;
  for (int i = blockIdx.y * kThreads + threadIdx.x; i < rows * chunks; i += kGatherSplit * kThreads) {
    const int r = i / chunks, c = i - r * chunks;
    const int kvh = r / (NM * G);
    const int m = (r / G) % NM;
    const int gg = r % G;
    const int src_seq = s0 + min(m, n - 1);
    const uint4* src = reinterpret_cast<const uint4*>(
        q + (((int64_t)src_seq * Hq + kvh * G + gg) * D) * es);
    uint4* dst = reinterpret_cast<uint4*>(qg + (((int64_t)g * rows + r) * D) * es);
    dst[c] = src[c];
  }
  if (blockIdx.y != 0) return;
  // the prefix never exceeds any member's context nor the host bound
  int P = min(max(plen[g], 0), max_prefix);
  for (int m = 0; m < n; ++m) P = min(P, max(context_lens[s0 + m], 0));
  P = (P / B) * B;
  const int nb = P / B;
  for (int j = threadIdx.x; j < max_pnb; j += kThreads)
    ptab[(int64_t)g * max_pnb + j] = j < nb ? tables[(int64_t)s0 * max_nb + j] : -1;
  for (int m = threadIdx.x; m < n; m += kThreads) {
    seq_start[s0 + m] = P;
    seq_group[s0 + m] = g;
  }
  if (threadIdx.x == 0) plens[g] = P;
}

// One thread per (sequence, head, 4 consecutive elements).
__global__ __launch_bounds__(kThreads) void cascade_combine_kernel(
    void* __restrict__ out, int32_t out_dt, const float* __restrict__ o_p,
    const float* __restrict__ lse_p, const float* __restrict__ o_s, const float* __restrict__ lse_s,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ seq_group, int32_t S, int32_t NM,
    int32_t Hq, int32_t Hkv, int32_t D) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int per_row = D / 4;
  if (i >= (int64_t)S * Hq * per_row) return;
  const int c = (int)(i % per_row);
  const int64_t sh = i / per_row;  // s * Hq + h
  const int s = (int)(sh / Hq), h = (int)(sh % Hq);
  const int G = Hq / Hkv;
  const int g = seq_group[s];
  const int m = s - cu[g];
  const int64_t ph = (int64_t)g * NM * Hq + (int64_t)(h / G) * NM * G + m * G + h % G;
  const float lp = lse_p[ph], ls = lse_s[sh];
  const float M = fmaxf(lp, ls);
  const float wp = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(lp - M);
  const float ws = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(ls - M);
  const float den = wp + ws;
  const float4 a = reinterpret_cast<const float4*>(o_p + ph * D)[c];
  const float4 b = reinterpret_cast<const float4*>(o_s + sh * D)[c];
  float r[4] = {a.x * wp + b.x * ws, a.y * wp + b.y * ws, a.z * wp + b.z * ws, a.w * wp + b.w * ws};
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = den > 0.f ? r[k] / den : 0.f;
  store_out_vec<4>(out, out_dt, sh * D + 4 * c, r);
}

pkv_status cascade_layout(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                          int32_t max_context_len, int32_t n_groups, int32_t max_group_size,
                          int32_t max_prefix_len, int kv_dt, CascadeLayout* L) {
  if (max_prefix_len > max_context_len) max_prefix_len = max_context_len;  // a looser bound is harmless
  L->max_prefix_len = max_prefix_len;
  const int es = dt_bytes(kv_dt);
  const int NM = max_group_size;
  const int64_t Hq_p = (int64_t)NM * Hq;
  if (Hq_p > (1 << 20)) return fail(PKV_ERR_UNSUPPORTED, "decode_cascade: group too large");
  pkv_status st = plan_decode(n_groups, (int32_t)Hq_p, Hkv, D, B, max_prefix_len, &L->plan_p);
  if (st != PKV_OK) return st;
  st = plan_decode(S, Hq, Hkv, D, B, max_context_len, &L->plan_s);
  if (st != PKV_OK) return st;
  L->max_pnb = (max_prefix_len + B - 1) / B;
  if (L->max_pnb < 1) L->max_pnb = 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L->qg = take((size_t)n_groups * Hq_p * D * es);
  L->ptab = take((size_t)n_groups * L->max_pnb * sizeof(int32_t));
  L->plens = take((size_t)n_groups * sizeof(int32_t));
  L->seq_start = take((size_t)S * sizeof(int32_t));
  L->seq_group = take((size_t)S * sizeof(int32_t));
  L->o_p = take((size_t)n_groups * Hq_p * D * sizeof(float));
  L->lse_p = take((size_t)n_groups * Hq_p * sizeof(float));
  L->o_s = take((size_t)S * Hq * D * sizeof(float));
  L->lse_s = take((size_t)S * Hq * sizeof(float));
  L->ws_p = take(L->plan_p.workspace_bytes);
  L->ws_s = take(L->plan_s.workspace_bytes);
  L->total = off;
  return PKV_OK;
}

}  // namespace

pkv_status cascade_workspace_size(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                  int32_t max_context_len, int32_t n_groups, int32_t max_group_size,
                                  int32_t max_prefix_len, int kv_dt, size_t* bytes) {
  CascadeLayout L;
  const pkv_status st = cascade_layout(S, Hq, Hkv, D, B, max_context_len, n_groups,
                                       max_group_size, max_prefix_len, kv_dt, &L);
  if (st != PKV_OK) return st;
  *bytes = L.total;
  return PKV_OK;
}

pkv_status launch_decode_cascade(int kv_dt, bool fp8, const DecodeArgs& base, const int32_t* cu_group_seqs,
                                 const int32_t* group_prefix_lens, int32_t n_groups,
                                 int32_t max_group_size, int32_t max_prefix_len, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  CascadeLayout L;
  pkv_status st = cascade_layout(base.S, base.Hq, base.Hkv, base.D, base.B, base.max_ctx, n_groups,
                                 max_group_size, max_prefix_len, kv_dt, &L);
  if (st != PKV_OK) return st;
  if (workspace_bytes < L.total || !workspace)
    return fail(PKV_ERR_WORKSPACE, "decode_cascade: workspace of %zu bytes needed, %zu given",
                L.total, workspace_bytes);
  char* ws = static_cast<char*>(workspace);
  const int es = dt_bytes(kv_dt);
  const int NM = max_group_size;
  int32_t* seq_start = reinterpret_cast<int32_t*>(ws + L.seq_start);
  int32_t* seq_group = reinterpret_cast<int32_t*>(ws + L.seq_group);
  int32_t* ptab = reinterpret_cast<int32_t*>(ws + L.ptab);
  int32_t* plens = reinterpret_cast<int32_t*>(ws + L.plens);
  float* o_p = reinterpret_cast<float*>(ws + L.o_p);
  float* lse_p = reinterpret_cast<float*>(ws + L.lse_p);
  float* o_s = reinterpret_cast<float*>(ws + L.o_s);
  float* lse_s = reinterpret_cast<float*>(ws + L.lse_s);

  hipLaunchKernelGGL(cascade_gather_kernel, dim3(n_groups, kGatherSplit), dim3(kThreads), 0, stream,
                     static_cast<const char*>(base.q), cu_group_seqs, group_prefix_lens,
                     base.block_tables, base.context_lens, base.max_nb, ws + L.qg, ptab,
                     L.max_pnb, plens, seq_start, seq_group, NM, base.Hq, base.Hkv, base.D, base.B,
                     es, L.max_prefix_len);
  st = check_launch("decode_cascade (gather)");
  if (st != PKV_OK) return st;

  // prefixes: one pseudo-sequence per group
  DecodeArgs p = base;
  p.out = o_p;
  p.out_dt = DT_F32;
  p.q = ws + L.qg;
  p.block_tables = ptab;
  p.max_nb = L.max_pnb;
  p.context_lens = plens;
  p.S = n_groups;
  p.Hq = NM * base.Hq;
  p.max_ctx = L.max_prefix_len;
  attach_decode_workspace(&p, L.plan_p, ws + L.ws_p);
  p.seq_start = nullptr;
  p.lse = lse_p;
  if (n_groups > 0) {
    st = launch_decode(kv_dt, fp8, L.plan_p, p, stream);
    if (st != PKV_OK) return st;
  }

  // suffixes: every sequence from its group's prefix length on
  DecodeArgs sf = base;
  sf.out = o_s;
  sf.out_dt = DT_F32;
  attach_decode_workspace(&sf, L.plan_s, ws + L.ws_s);
  sf.seq_start = seq_start;
  sf.lse = lse_s;
  st = launch_decode(kv_dt, fp8, L.plan_s, sf, stream);
  if (st != PKV_OK) return st;

  const int64_t items = (int64_t)base.S * base.Hq * (base.D / 4);
  const int64_t blocks = (items + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(cascade_combine_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     base.out, base.out_dt, o_p, lse_p, o_s, lse_s, cu_group_seqs, seq_group,
                     base.S, NM, base.Hq, base.Hkv, base.D);
  return check_launch("decode_cascade (combine)");
}

}  // namespace pkv
