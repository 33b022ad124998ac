/*
 * pkv.h -- C ABI of the paged KV-cache attention library (libpkv.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * Plain C: only integers, floats and pointers cross this boundary.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Ownership: every pointer is owned by the caller.  Tensor pointers are
 *    DEVICE pointers (hipMalloc'd or torch CUDA tensors on the current device);
 *    the library allocates no device memory and keeps no state beyond a
 *    thread-local error string, the host block managers the caller creates,
 *    caches of the per-device CU count and of kernel occupancies, and the
 *    static scratch array of pkv_paged_attention_decode_noalloc.
 *  - Threads: the kernel calls may be made from several host threads at once
 *    (the caches are atomic); calls that overlap on one device need their own
 *    workspaces.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream).  Kernel calls are asynchronous on that stream.
 *  - Errors: scalar arguments are validated on the host before any launch; a
 *    failure returns a non-zero pkv_status and leaves all memory untouched.
 *    A failed launch returns PKV_ERR_HIP.  pkv_last_error() gives detail.
 *  - Alignment: tensor data (q, out, key, value, the pools, workspaces) is read
 *    and written with 16-byte vector accesses, so those pointers must be
 *    16-byte aligned; index arrays (tables, lengths, slots, pairs, cu arrays)
 *    and scales must be aligned to their element size.  Anything else is
 *    refused with PKV_ERR_INVALID_ARG before any launch.
 *  - Device-resident CONTENTS (block ids, slots, lengths, cu_seqlens) are the
 *    caller's contract and are not validated: out-of-range values are undefined
 *    behaviour.  The host block manager below only ever produces valid ones.
 *  - KV pool layout: K and V are separate pools of shape [NB, B, Hkv, D]
 *    (block, offset in block, kv head, head dim), elements of dtype kv_dtype,
 *    row-major.  (S06 PagedAttention chapter, "implementation" section: the
 *    pool is [num_blocks, block_size, n_kv_heads, head_dim].)
 *  - A slot is an absolute row index of a pool: slot = block * B + offset.
 *  - Supported instantiations: kv dtype {f32, f16, bf16}; D in {64, 128};
 *    B in {1, 2, 4, 8, 16, 32}; any Hkv >= 1 and Hq a multiple of Hkv.
 *    FP8 pools (PKV_FP8_E4M3) are written by pkv_reshape_and_cache_fp8, read
 *    by the _fp8 variants of decode, cascade decode, prefill and the mixed
 *    batch, and copied by pkv_copy_blocks and pkv_swap_blocks.
 *    Anything else returns PKV_ERR_UNSUPPORTED.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1, /* bad scalar argument or null pointer */
  PKV_ERR_UNSUPPORTED = 2, /* valid but not instantiated (dtype, D, B) */
  PKV_ERR_WORKSPACE = 3,   /* workspace too small or null */
  PKV_ERR_OOM = 4,         /* block manager: free list exhausted */
  PKV_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed */
} pkv_status;

/* PKV_FP8_E4M3: OCP 8-bit float E4M3 (sign, 4 exponent bits with bias 7, 3
 * mantissa bits, subnormals, no infinities, 0x7F/0xFF NaN, max 448); KV pools
 * only. */
typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_FP8_E4M3 = 3 } pkv_dtype;

/* Human-readable name of a status code (static storage). */
const char* pkv_status_string(pkv_status s);
/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* pkv_last_error(void);
/* Library version string, e.g. "pkv 0.1 gfx950". */
const char* pkv_version(void);

/* ------------------------------------------------------------------------
 * reshape_and_cache -- scatter new tokens' K/V rows into their slots.
 *
 * Defined by "LLM inference, part 3: single node", ch. 13 sec. 1 (the CPU
 * precomputes one absolute slot per new token and the GPU performs
 * kv_cache[slot_mapping[i]] = new_kv) and CS349D lecture 3 sec. 3.2 (the
 * split/reorder/block-write is one fused kernel).
 *
 *   key, value   : device, [T, Hkv, D] of kv_dtype (row-major)
 *   k_cache,
 *   v_cache      : device pools [NB, B, Hkv, D] of kv_dtype, written in place
 *   slot_mapping : device int64 [T]; slot < 0 means "skip this token"
 *                  (padding); a slot at or beyond NB * B is skipped too (no
 *                  write outside the pools), otherwise 0 <= slot < NB * B
 * Bytes are copied unchanged (bit-exact).  T == 0 is a no-op.
 * ------------------------------------------------------------------------ */
pkv_status pkv_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                 const int64_t* slot_mapping, int32_t T, int32_t Hkv, int32_t D,
                                 int32_t B, int64_t NB, pkv_dtype kv_dtype, void* stream);

/* ------------------------------------------------------------------------
 * paged_attention_decode -- one query token per sequence attends to its
 * whole paged context.
 *
 * Defined by CS349D lecture 3 sec. 3.2 (attention over the blocks of a block
 * table is mathematically identical to contiguous attention: one softmax over
 * every position of every block), CMU 11-868 lecture 24 sec. 3.2 (scores
 * within a block, blocks merged with an online softmax, no gather into a
 * contiguous buffer), "LLM inference, part 3" ch. 9 sec. 1 (GQA: query head h
 * uses KV head h / (Hq / Hkv)) and ch. 11 sec. 3 (block table tensor
 * [max_num_reqs, max_num_blocks_per_req], physical = table[req][logical]).
 *
 *   out            : device [S, Hq, D] of out_dtype (f32, f16 or bf16)
 *   q              : device [S, Hq, D] of kv_dtype
 *   k_cache,v_cache: device pools [NB, B, Hkv, D] of kv_dtype
 *   block_tables   : device int32 [S, max_blocks_per_seq]; entries past
 *                    ceil(context_lens[s] / B) are never read
 *   context_lens   : device int32 [S]; tokens cached for sequence s, the
 *                    current token included; rows past it are never read.
 *                    0 gives an all-zero output row.
 *   max_context_len: host bound >= every context_lens[s] (sizes the grid)
 *   scale          : softmax scale, usually 1/sqrt(D)
 *   workspace      : device scratch of at least pkv_decode_workspace_size()
 *                    bytes (a size that depends on the arguments only, not on
 *                    the device); contents on entry are ignored.  It holds the
 *                    partial softmax states of rows split between waves and
 *                    the list of those rows.
 * out[s, h, :] = sum_t softmax_t(scale * q[s,h,:] . K[s,t,:]) V[s,t,:],
 * computed in fp32.  The summation order depends only on logical positions,
 * so the result is bit-identical under any permutation of physical blocks and
 * when sequences alias shared blocks.
 * ------------------------------------------------------------------------ */
pkv_status pkv_decode_workspace_size(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                     int32_t max_context_len, size_t* bytes);

pkv_status pkv_paged_attention_decode(void* out, pkv_dtype out_dtype, const void* q,
                                      const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t max_context_len,
                                      int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                      float scale, void* workspace, size_t workspace_bytes,
                                      void* stream);

/* ------------------------------------------------------------------------
 * decode_step -- one decode step in one call: the new token of every
 * sequence is written to the pools and attended, as pkv_reshape_and_cache
 * (T = S) followed by pkv_paged_attention_decode.
 *
 * Defined by "LLM inference, part 3" ch. 13 sec. 1 (each step the new
 * tokens' K/V go to the slots the host computed, then attention reads the
 * cache through the block table) and CS349D lecture 3 sec. 3.2 (the block
 * write fused into the attention kernel's pass).
 *
 *   key, value   : device [S, Hkv, D] of kv_dtype; row s is the K (V) of the
 *                  newest token of sequence s, token context_lens[s] - 1
 *   slot_mapping : device int64 [S]; that token's slot (slots outside
 *                  [0, NB * B) are not written, as in pkv_reshape_and_cache)
 *   k_cache,
 *   v_cache      : device pools [NB, B, Hkv, D] of kv_dtype, written in place
 *   (the other arguments and the workspace as for pkv_paged_attention_decode;
 *   kv_dtype f32, f16 or bf16)
 * Precondition: for every s with context_lens[s] >= 1, slot_mapping[s] is the
 * slot the block table gives token context_lens[s] - 1 of sequence s, and no
 * other sequence reads that slot (the ordinary step of a block manager that
 * copies shared blocks before writing).  Then out and both pools are
 * bit-identical to the two calls made in order.  On the matrix-core path
 * (16-bit pools, D = 128, B >= 4, a multiple of 4 query heads per KV head) it is one
 * pass: the attention takes token context_lens[s] - 1 from key/value directly
 * while the same launch stores those rows in their slots; elsewhere the cache
 * write runs as its own launch first.  Errors as for both calls.
 * ------------------------------------------------------------------------ */
pkv_status pkv_decode_step(void* out, pkv_dtype out_dtype, const void* q, const void* key,
                           const void* value, const int64_t* slot_mapping, void* k_cache,
                           void* v_cache, int64_t NB, pkv_dtype kv_dtype,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t max_context_len, int32_t S,
                           int32_t Hq, int32_t Hkv, int32_t D, int32_t B, float scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * paged_attention_decode_noalloc -- pkv_paged_attention_decode without a
 * workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.
 *
 * Arguments, result and errors are those of pkv_paged_attention_decode (the
 * same kernels and launch shapes, so the same bits).  The partial softmax
 * states live in a static device array of 32 MiB inside the library, one per
 * device, held until the process ends; a call needs at most
 * (waves of its launch) x 2 x (query heads per row) x (D + 2) x 4 bytes of it,
 * about 4.3 MB for 32 query / 8 KV heads at D = 128 on a 256-CU device.  A
 * call needing more fails with PKV_ERR_WORKSPACE before any launch.  The call
 * allocates nothing (no hipMalloc, no hipFree).  Every call on a device shares
 * that device's array and nothing needs to start at zero; calls that overlap
 * on one device (two streams, two threads) race on it and give undefined
 * results: serialise them on one stream.
 * ------------------------------------------------------------------------ */
pkv_status pkv_paged_attention_decode_noalloc(void* out, pkv_dtype out_dtype, const void* q,
                                              const void* k_cache, const void* v_cache,
                                              pkv_dtype kv_dtype, const int32_t* block_tables,
                                              int32_t max_blocks_per_seq,
                                              const int32_t* context_lens, int32_t max_context_len,
                                              int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                                              int32_t B, float scale, void* stream);

/* ------------------------------------------------------------------------
 * paged_attention_decode_cascade -- decode for a batch whose sequences come
 * in groups that share a prefix of blocks (the samples forked from one
 * prompt), reading each group's prefix once instead of once per member.
 *
 * Defined by the S06 PagedAttention chapter ("in production" section: a
 * cascade path batches the shared prefix apart from the forked suffixes),
 * CMU 11-868 lecture 24 sec. 7.3 and further reading (cascade attention /
 * cascade inference for shared-prefix batch decode) and CS349D lecture 3 sec.
 * 4.1 (forked sequences share the parent's blocks).  The result is that of
 * pkv_paged_attention_decode on the same arguments (one softmax over every
 * cached token of each sequence); only the summation order differs: the
 * prefix and the suffix are attended separately and their two softmax states
 * merged (log-sum-exp), so the output agrees with the plain decode to fp32
 * rounding, not bit for bit.
 *
 *   (arguments as for pkv_paged_attention_decode, 16- or 32-bit pools)
 *   cu_group_seqs     : device int32 [n_groups + 1]; group g is sequences
 *                       cu[g] .. cu[g+1]-1 (consecutive, every sequence in
 *                       exactly one group: cu[0] = 0, cu[n_groups] = S)
 *   group_prefix_lens : device int32 [n_groups]; tokens every member of the
 *                       group holds in the same physical blocks (a multiple
 *                       of B; longer values are cut to the shortest member and
 *                       to max_prefix_len, then rounded down to a multiple of
 *                       B); 0 for a group that shares nothing
 *   n_groups          : host, >= 1 when S > 0
 *   max_group_size    : host bound >= every group's size
 *   max_prefix_len    : host bound >= every prefix length used (values above
 *                       max_context_len act as max_context_len)
 *   workspace         : device scratch of pkv_decode_cascade_workspace_size()
 *                       bytes (depends on the arguments only)
 * ------------------------------------------------------------------------ */
pkv_status pkv_decode_cascade_workspace_size(int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                                             int32_t B, int32_t max_context_len, int32_t n_groups,
                                             int32_t max_group_size, int32_t max_prefix_len,
                                             pkv_dtype kv_dtype, size_t* bytes);

pkv_status pkv_paged_attention_decode_cascade(
    void* out, pkv_dtype out_dtype, const void* q, const void* k_cache, const void* v_cache,
    pkv_dtype kv_dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t max_context_len, int32_t S, int32_t Hq, int32_t Hkv,
    int32_t D, int32_t B, float scale, const int32_t* cu_group_seqs,
    const int32_t* group_prefix_lens, int32_t n_groups, int32_t max_group_size,
    int32_t max_prefix_len, void* workspace, size_t workspace_bytes, void* stream);

/* Cascade decode over FP8 (E4M3) pools with per-KV-head scales: the
 * arguments of pkv_paged_attention_decode_cascade with q in q_dtype (f16 or
 * bf16) and k_scale / v_scale as for pkv_paged_attention_decode_fp8; the
 * workspace is pkv_decode_cascade_workspace_size(..., q_dtype, ...).  Same
 * result, within the FP8 decode's tolerance, as pkv_paged_attention_decode_fp8
 * on the same pools ("LLM inference, part 3" ch. 10 for the cache format). */
pkv_status pkv_paged_attention_decode_cascade_fp8(
    void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype, const void* k_cache,
    const void* v_cache, const float* k_scale, const float* v_scale, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len, int32_t S,
    int32_t Hq, int32_t Hkv, int32_t D, int32_t B, float scale, const int32_t* cu_group_seqs,
    const int32_t* group_prefix_lens, int32_t n_groups, int32_t max_group_size,
    int32_t max_prefix_len, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * FP8 KV cache -- the pools hold OCP E4M3 codes, one byte per element, with
 * one fp32 scale per KV head for K and one for V.
 *
 * Defined by "LLM inference, part 3: single node", ch. 10 (KV-cache
 * quantization: on write each 16-bit K/V value is scaled and clipped into 8
 * bits, halving the bytes that decode must read; on read it is scaled back;
 * FP8 keeps sign, exponent and mantissa, i.e. it is still a float).
 *
 * pkv_reshape_and_cache_fp8: as pkv_reshape_and_cache, but element (h, d) of
 * token t is stored as the E4M3 code nearest to fp32(x) / scale[h] (fp32
 * division, round to nearest even; |x / scale| >= 448 and infinities clip to
 * +-448; NaN stays NaN).
 *   key, value       : device [T, Hkv, D] of in_dtype (f32, f16 or bf16)
 *   k_cache, v_cache : device pools [NB, B, Hkv, D] of E4M3 codes (uint8)
 *   k_scale, v_scale : device fp32 [Hkv]; positive and finite (caller's
 *                      contract, like the other device contents)
 *
 * pkv_paged_attention_decode_fp8: as pkv_paged_attention_decode, with q of
 * q_dtype (f16 or bf16) and every cached element read as code * scale of its
 * KV head:  out[s,h,:] = sum_t softmax_t(scale * q . K_t) V_t with
 * K_t = k_code * k_scale[h / G], V_t = v_code * v_scale[h / G].  The codes
 * are widened exactly; the K scale is folded into the score scale and the V
 * scale into the result (fp32).  The workspace is the same as for
 * pkv_paged_attention_decode (pkv_decode_workspace_size).
 * ------------------------------------------------------------------------ */
pkv_status pkv_reshape_and_cache_fp8(const void* key, const void* value, pkv_dtype in_dtype,
                                     void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                     int32_t T, int32_t Hkv, int32_t D, int32_t B, int64_t NB,
                                     const float* k_scale, const float* v_scale, void* stream);

pkv_status pkv_paged_attention_decode_fp8(void* out, pkv_dtype out_dtype, const void* q,
                                          pkv_dtype q_dtype, const void* k_cache,
                                          const void* v_cache, const float* k_scale,
                                          const float* v_scale, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                                          int32_t max_context_len, int32_t S, int32_t Hq,
                                          int32_t Hkv, int32_t D, int32_t B, float scale,
                                          void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * paged_attention_prefill -- a causal query chunk per sequence over its
 * paged context (earlier prompt + the chunk itself).
 *
 * Defined by "LLM inference, part 3" ch. 13 sec. 1 (flattened varlen batch
 * with cu_seqlens boundaries; the block table locates earlier KV) and sec. 2
 * (chunked prefill: each chunk reads the earlier prompt's KV through the block
 * table) and CS349D lecture 3 sec. 7.2 (a token's K/V depend only on earlier
 * tokens, so the mask is causal).
 *
 *   out            : device [Tq, Hq, D] of out_dtype
 *   q              : device [Tq, Hq, D] of kv_dtype (rows of all chunks
 *                    concatenated)
 *   cu_seqlens_q   : device int32 [S + 1]; chunk of sequence s is rows
 *                    cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1; cu_seqlens_q[S]==Tq
 *   max_query_len  : host bound >= every chunk length
 *   context_lens   : device int32 [S]; prior context + chunk, the chunk's K/V
 *                    already written to the cache (pkv_reshape_and_cache)
 *   workspace      : device scratch of pkv_prefill_workspace_size() bytes
 *                    (may be NULL when that size is 0)
 * Row i of sequence s sits at position context_lens[s] - Q_s + i and attends
 * to positions 0 .. context_lens[s] - Q_s + i.  kv_dtype f16/bf16 use the
 * matrix cores (16-bit operands, fp32 accumulation; the softmax weights enter
 * the PV product as kv_dtype values, split into two parts for bf16); f32 uses
 * fp32 vector math.  A call with too few (sequence, KV head, query tile)
 * units to fill the GPU -- few sequences with long contexts -- splits each
 * unit's KV range and merges the partial softmax results (log-sum-exp); the
 * split is a function of the arguments and the device's CU count only, so
 * equal calls give equal bits.  A workspace smaller than the size query's
 * answer fails with PKV_ERR_WORKSPACE and launches nothing.
 * ------------------------------------------------------------------------ */
pkv_status pkv_prefill_workspace_size(int32_t S, int32_t Tq, int32_t max_query_len, int32_t Hq,
                                      int32_t Hkv, int32_t D, int32_t B, pkv_dtype kv_dtype,
                                      int32_t max_context_len, size_t* bytes);

pkv_status pkv_paged_attention_prefill(void* out, pkv_dtype out_dtype, const void* q,
                                       const int32_t* cu_seqlens_q, int32_t Tq,
                                       int32_t max_query_len, const void* k_cache,
                                       const void* v_cache, pkv_dtype kv_dtype,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t max_context_len,
                                       int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                       float scale, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* ------------------------------------------------------------------------
 * paged_attention_prefill_fp8 -- pkv_paged_attention_prefill over pools of
 * OCP FP8 E4M3 codes, one fp32 scale per KV head for K and one for V (the
 * pools of pkv_reshape_and_cache_fp8; "LLM inference, part 3" ch. 10: KV
 * cache quantization), so chunked prefill can run over a quantized cache.
 *
 *   q, out             : as for pkv_paged_attention_prefill, q in q_dtype
 *                        (f16 or bf16)
 *   k_cache, v_cache   : device uint8 [NB, B, Hkv, D]
 *   k_scale, v_scale   : device float [Hkv]
 *   workspace          : pkv_prefill_workspace_size(..., PKV_FP8_E4M3, ...)
 * Every cached element is read as code * scale of its KV head (exact in
 * fp32); the codes are widened to q_dtype exactly and the products run on the
 * matrix cores as in the 16-bit prefill.  Needs block_size >= 8 and at most
 * 128 query heads per KV head (PKV_ERR_UNSUPPORTED otherwise).
 * ------------------------------------------------------------------------ */
pkv_status pkv_paged_attention_prefill_fp8(void* out, pkv_dtype out_dtype, const void* q,
                                           pkv_dtype q_dtype, const int32_t* cu_seqlens_q,
                                           int32_t Tq, int32_t max_query_len, const void* k_cache,
                                           const void* v_cache, const float* k_scale,
                                           const float* v_scale, const int32_t* block_tables,
                                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                                           int32_t max_context_len, int32_t S, int32_t Hq,
                                           int32_t Hkv, int32_t D, int32_t B, float scale,
                                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * paged_attention_mixed -- one call for a batch mixing decode requests and
 * prefill chunks.
 *
 * Defined by "LLM inference, part 3: single node", ch. 13 sec. 1 (one
 * flattened token stream; cu_seqlens separates requests of one token (decode)
 * and of many (prefill)) and sec. 2 (a chunk of a long prompt is packed with
 * the running decodes into one batch, so the bandwidth-bound decodes and the
 * compute-bound chunk use the GPU together).
 *
 *   (arguments as for pkv_paged_attention_prefill, over the whole batch)
 *   num_decode : host; sequences 0 .. num_decode - 1 are decodes with one
 *                query row each (rows 0 .. num_decode - 1, so
 *                cu_seqlens_q[i] == i for i <= num_decode); the others are
 *                prefill chunks
 *   workspace  : device scratch of pkv_mixed_workspace_size() bytes
 * Every output row equals what pkv_paged_attention_decode (decode rows) or
 * pkv_paged_attention_prefill (chunk rows) give for it, bit for bit: the
 * decode part and then the chunks, on `stream`; chunks too few to fill the
 * GPU have their KV ranges split as in pkv_paged_attention_prefill.
 * ------------------------------------------------------------------------ */
pkv_status pkv_mixed_workspace_size(int32_t S, int32_t num_decode, int32_t Tq,
                                    int32_t max_query_len, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t B, pkv_dtype kv_dtype, int32_t max_context_len,
                                    size_t* bytes);

pkv_status pkv_paged_attention_mixed(void* out, pkv_dtype out_dtype, const void* q,
                                     const int32_t* cu_seqlens_q, int32_t Tq, int32_t num_decode,
                                     int32_t max_query_len, const void* k_cache,
                                     const void* v_cache, pkv_dtype kv_dtype,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, int32_t max_context_len,
                                     int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                     float scale, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* Mixed batch over FP8 (E4M3) pools with per-KV-head scales: the arguments of
 * pkv_paged_attention_mixed with q in q_dtype (f16 or bf16) and k_scale /
 * v_scale as for pkv_paged_attention_decode_fp8; the workspace is
 * pkv_mixed_workspace_size(..., PKV_FP8_E4M3, ...).  Every row equals what
 * pkv_paged_attention_decode_fp8 / pkv_paged_attention_prefill_fp8 give for
 * it, bit for bit; the chunks need block_size >= 8. */
pkv_status pkv_paged_attention_mixed_fp8(void* out, pkv_dtype out_dtype, const void* q,
                                         pkv_dtype q_dtype, const int32_t* cu_seqlens_q,
                                         int32_t Tq, int32_t num_decode, int32_t max_query_len,
                                         const void* k_cache, const void* v_cache,
                                         const float* k_scale, const float* v_scale,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t max_context_len,
                                         int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                         float scale, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* ------------------------------------------------------------------------
 * copy_blocks -- batched whole-block copies for copy-on-write.
 *
 * Defined by CS349D lecture 3 sec. 4.1 (writing into a block whose refcount is
 * above one first copies it to a fresh block) and sec. 3.2 (the many small CoW
 * copies are merged into one kernel launch).
 *
 *   k_caches, v_caches : HOST arrays of num_layers DEVICE pointers, each a
 *                        pool [NB, B, Hkv, D] of kv_dtype
 *   block_pairs        : DEVICE int64 [N, 2] of (src, dst) physical blocks
 * For every layer and pair, block dst of the K pool and of the V pool becomes
 * a bit copy of block src.  Destinations must be distinct and no destination
 * may also be a source in the same call (copy-on-write targets are freshly
 * allocated blocks); then every pair reads the pre-call contents.  N == 0 or
 * num_layers == 0 is a no-op.
 * ------------------------------------------------------------------------ */
pkv_status pkv_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                           const int64_t* block_pairs, int32_t N, int32_t B, int32_t Hkv,
                           int32_t D, pkv_dtype kv_dtype, void* stream);

/* ------------------------------------------------------------------------
 * swap_blocks -- batched whole-block copies between two sets of pools, for
 * swapping a preempted sequence's KV blocks out to host memory and back.
 *
 * Defined by CS349D lecture 3 sec. 5.2 (recovery by swapping: the blocks are
 * copied to CPU memory, from a CPU block allocator, and copied back on
 * resume; each separate copy has a fixed cost, so many small copies are worth
 * batching) and "LLM inference, part 3" ch. 14 (swap-out / swap-in over the
 * host link as the alternative to recomputation).
 *
 *   src_pools, dst_pools : HOST arrays of num_pools pointers; pool i of src
 *                          pairs with pool i of dst (e.g. the K and V pools of
 *                          every layer).  Each pointer is device memory or
 *                          pinned host memory (hipHostMalloc, torch
 *                          pin_memory); pageable host memory is refused with
 *                          PKV_ERR_INVALID_ARG.  Pools are [NB_x, B, Hkv, D] of
 *                          kv_dtype (PKV_FP8_E4M3 allowed); the two sides may
 *                          have different block counts.
 *   block_pairs          : device or pinned host int64 [N, 2] of (source block,
 *                          destination block)
 * For every pool and pair, destination block dst becomes a bit copy of source
 * block src.  Destinations must be distinct and the two sides must not
 * overlap.  One kernel launch (per 64 pools) on `stream` does all copies; it
 * reads and writes the host side directly.  N == 0 or num_pools == 0 is a
 * no-op.
 * ------------------------------------------------------------------------ */
pkv_status pkv_swap_blocks(const void* const* src_pools, void* const* dst_pools, int32_t num_pools,
                           const int64_t* block_pairs, int32_t N, int32_t B, int32_t Hkv,
                           int32_t D, pkv_dtype kv_dtype, void* stream);

/* ------------------------------------------------------------------------
 * Host block manager (CPU only; builds block tables, slots and CoW pairs).
 *
 * Defined by the S06 PagedAttention chapter ("block manager" listing: a free
 * list; a request gets ceil(n / B) blocks, any free block will do; out of
 * blocks -> the allocator fails; "reference counts must be exact" section: the
 * number of tables holding a block equals its refcount), the kwkr.cn
 * PagedAttention post (KV-cache manager: blocks taken from the front of the free
 * list, a new block only once the last one is full, OOM on exhaustion) and
 * CS349D lecture 3 sec. 4.1 (fork copies the parent's table and raises every
 * refcount; the first write into a shared partly-filled last block copies it;
 * freeing decrements refcounts and returns blocks that reach zero).
 *
 * Sequences are identified by small non-negative ids assigned by the manager.
 * Every call returns PKV_OK or an error and leaves the state unchanged on
 * error.  Not thread-safe: one manager per thread.
 * ------------------------------------------------------------------------ */
typedef struct pkv_block_manager pkv_block_manager;

/* free_order: host int32 [num_blocks] permutation of 0..num_blocks-1 giving the
 * order blocks are handed out (NULL = 0, 1, 2, ...).  Freed blocks go to the
 * back of the free list. */
pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                         pkv_block_manager** out);
void pkv_bm_destroy(pkv_block_manager* bm);
/* New sequence holding n_tokens tokens (ceil(n_tokens / B) fresh blocks). */
pkv_status pkv_bm_add_seq(pkv_block_manager* bm, int32_t n_tokens, int32_t* seq_id);
/* Grow sequence by one token.  *slot receives the new token's slot.  If the
 * last block was shared and partly filled, it is replaced by a fresh private
 * copy: *cow_src / *cow_dst receive (old, new) block ids, which the caller must
 * copy (pkv_copy_blocks) before writing the slot; otherwise both are -1. */
pkv_status pkv_bm_append_token(pkv_block_manager* bm, int32_t seq_id, int64_t* slot,
                               int32_t* cow_src, int32_t* cow_dst);
/* New sequence sharing every block of parent (refcounts + 1). */
pkv_status pkv_bm_fork(pkv_block_manager* bm, int32_t parent, int32_t* child);
/* Drop a sequence: refcounts - 1, blocks reaching zero return to the free list. */
pkv_status pkv_bm_free_seq(pkv_block_manager* bm, int32_t seq_id);
/* Copy the sequence's table into out[0..cap); *n receives its length. */
pkv_status pkv_bm_table(const pkv_block_manager* bm, int32_t seq_id, int32_t* out, int32_t cap,
                        int32_t* n);
pkv_status pkv_bm_seq_len(const pkv_block_manager* bm, int32_t seq_id, int32_t* n_tokens);
/* Slots of positions [start, start + count) of the sequence (all < seq_len). */
pkv_status pkv_bm_slots(const pkv_block_manager* bm, int32_t seq_id, int32_t start,
                        int32_t count, int64_t* out);
pkv_status pkv_bm_refcount(const pkv_block_manager* bm, int32_t block, int32_t* refcount);
pkv_status pkv_bm_num_free(const pkv_block_manager* bm, int32_t* n);
/* Verify every invariant: refcount(b) == number of live tables holding b, free
 * blocks have refcount 0 and appear once, every table has ceil(len / B)
 * entries.  Returns PKV_OK or PKV_ERR_INVALID_ARG with detail. */
pkv_status pkv_bm_check(const pkv_block_manager* bm);

/* Swapping (CS349D lecture 3 sec. 5.2): a CPU pool of num_cpu_blocks blocks
 * (resets the CPU free list; refused while a sequence is swapped out). */
pkv_status pkv_bm_set_cpu_blocks(pkv_block_manager* bm, int32_t num_cpu_blocks);
pkv_status pkv_bm_num_free_cpu(const pkv_block_manager* bm, int32_t* n);
/* Swap a resident sequence out: every block of its table gets a CPU block;
 * pairs (host int64 [cap, 2]) receives (GPU block, CPU block) in table order,
 * *n their number; the GPU blocks are released (freed unless another sequence
 * holds them).  The copies must be issued (pkv_swap_blocks) before anything
 * writes into the released blocks.  While swapped out, the sequence has no
 * table or slots and cannot grow or fork; free_seq returns its CPU blocks.
 * PKV_ERR_OOM if the CPU pool is short (nothing changes). */
pkv_status pkv_bm_swap_out(pkv_block_manager* bm, int32_t seq_id, int64_t* pairs, int32_t cap,
                           int32_t* n);
/* Swap a sequence back in: fresh GPU blocks for its CPU blocks, pairs =
 * (CPU block, GPU block) in table order; the CPU blocks return to the CPU
 * free list (issue the copies before reusing them).  PKV_ERR_OOM if the GPU
 * pool is short (nothing changes). */
pkv_status pkv_bm_swap_in(pkv_block_manager* bm, int32_t seq_id, int64_t* pairs, int32_t cap,
                          int32_t* n);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
