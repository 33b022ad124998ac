/*
 * pkv_oracle.c -- reference oracle for paged KV-cache attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this file.  The product
 * library never links it, and it shares no code, header, table or helper with
 * the HIP kernels: dtype decoding, gathering and attention are written out here
 * on their own.
 *
 * What it computes, and from where:
 *
 *  - Paged attention is ordinary softmax attention over the logical sequence of
 *    keys and values; the block table only changes where each row is read from.
 *    (CS349D lecture 3 notes, "PagedAttention", sec. 3.2: the block-wise form is
 *    mathematically identical to contiguous attention; sec. 3.1: a per-sequence
 *    block table maps logical block i to any physical block.)
 *
 *  - The oracle therefore does the plainest thing: it GATHERS each sequence's
 *    rows through the table into a contiguous buffer, then runs textbook
 *    max-subtracted softmax attention on it.  The gather follows the KV-cache
 *    manager of the kwkr.cn PagedAttention/RadixAttention post ("code"
 *    section: concatenate the table's physical blocks, then truncate to the
 *    sequence length) and the pool layout of the S06 PagedAttention chapter
 *    ("implementation" section: pool [num_blocks, block_size, n_kv_heads,
 *    head_dim]; only the written rows of the last block are used).
 *
 *  - GQA: query head h reads KV head h / G with G = Hq / Hkv (consecutive
 *    grouping; "LLM inference, part 3: single node", ch. 9 sec. 1, groups of
 *    query heads share one K/V head).
 *
 *  - Prefill: query row i of a chunk of Q rows in a sequence whose context
 *    (chunk included) has L tokens sits at absolute position L - Q + i and
 *    attends to positions 0..L-Q+i (causal).  ("LLM inference, part 3", ch. 13
 *    sec. 2, chunked prefill reads the earlier prompt's KV through the block
 *    table; CS349D lecture 3 sec. 7.2, a token's K/V depend only on the tokens
 *    before it.)
 *
 *  - reshape_and_cache writes new K/V rows to absolute slots
 *    kv_cache[slot_mapping[i]] = new_kv ("LLM inference, part 3", ch. 13 sec. 1,
 *    slot_mapping); slot = block * block_size + offset; a negative slot means
 *    "skip this token".
 *
 *  - copy_blocks copies whole physical blocks (K and V, every layer given) for
 *    copy-on-write (CS349D lecture 3 sec. 3.2 and sec. 4.1: many small CoW
 *    copies are merged into one launch; the copy is made before the write).
 *
 *  - swap_blocks copies whole blocks between two sets of pools (device and
 *    host) for swapping a preempted sequence out and back in (CS349D lecture
 *    3 sec. 5.2): destination block := source block in every pool.
 *
 *  - FP8 KV cache ("LLM inference, part 3: single node", ch. 10: on write a
 *    16-bit K/V value is scaled and clipped into 8 bits; on read it is scaled
 *    back).  Format: OCP FP8 E4M3 (1 sign bit, 4 exponent bits with bias 7, 3
 *    mantissa bits; subnormals; no infinities; 0x7F / 0xFF are NaN; largest
 *    finite value 448).  Reading of the pages: one fp32 scale per KV head for
 *    K and one for V; stored code = nearest finite E4M3 value to
 *    fp32(x) / scale (ties to the even code, so anything beyond 448 clips to
 *    448); the attended value is code * scale.  The division is done in fp32
 *    because it decides an integer code.
 *
 * Precision: every floating-point operation is IEEE binary64, compiled without
 * fast-math and with FP contraction off.  Stored elements are widened exactly
 * (fp32 directly; fp16 by its IEEE definition including subnormals; bf16 as the
 * upper half of an fp32 word).
 *
 * Parity pins: every function here is pinned by tests that do not reuse this
 * file's arithmetic (worked values printed on the pages, torch's fp64 SDPA,
 * brute-force Python loops, closed forms and invariants).  No function is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define PKVO_F32 0
#define PKVO_F16 1
#define PKVO_BF16 2
#define PKVO_FP8 3 /* OCP E4M3 codes */

#define PKVO_OK 0
#define PKVO_EINVAL -1
#define PKVO_ENOMEM -2
#define PKVO_ERANGE -3 /* a block id, slot or length outside its valid range */

static int elem_bytes(int dtype) {
  switch (dtype) {
    case PKVO_F32: return 4;
    case PKVO_F16: return 2;
    case PKVO_BF16: return 2;
    case PKVO_FP8: return 1;
    default: return 0;
  }
}

/* IEEE binary16 -> binary64, exact. */
static double f16_bits_to_f64(uint16_t h) {
  int sign = h >> 15;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* zero or subnormal: m * 2^-24 */
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexp((double)(m | 0x400), e - 25); /* (1 + m/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* bfloat16 -> binary64, exact: bf16 is the high 16 bits of an fp32 word. */
static double bf16_bits_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP FP8 E4M3 code -> binary64, exact.  Exponent field e, mantissa m:
 * e == 0: m * 2^-9 (zero or subnormal); otherwise (8 + m) * 2^(e - 10), i.e.
 * (1 + m/8) * 2^(e - 7); e == 15 with m == 7 is NaN. */
double pkvo_e4m3_to_f64(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xf;
  int m = code & 0x7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp((double)(8 + m), e - 10);
  return sign ? -v : v;
}

/* binary32 -> OCP FP8 E4M3 code: the finite E4M3 value nearest to x, ties
 * to the code with an even mantissa (IEEE round-to-nearest-even over the
 * finite values only, so |x| beyond 448 -- infinities included -- clips to
 * 448); NaN gives the NaN code of x's sign.  Plain search over all 127
 * non-negative finite codes. */
uint8_t pkvo_e4m3_from_f32(float x) {
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(sign | 0x7f);
  if (isinf(x)) return (uint8_t)(sign | 0x7e);
  const double a = fabs((double)x);
  int best = 0;
  double best_d = a; /* distance to +0 (code 0) */
  for (int c = 1; c <= 0x7e; ++c) {
    const double d = fabs(pkvo_e4m3_to_f64((uint8_t)c) - a);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return (uint8_t)(sign | best);
}

/* Widen element idx of a stored array of the given dtype to binary64. */
double pkvo_load_elem(const void* base, int dtype, int64_t idx) {
  switch (dtype) {
    case PKVO_F32: {
      float f;
      memcpy(&f, (const char*)base + 4 * idx, 4);
      return (double)f;
    }
    case PKVO_F16: {
      uint16_t h;
      memcpy(&h, (const char*)base + 2 * idx, 2);
      return f16_bits_to_f64(h);
    }
    case PKVO_BF16: {
      uint16_t b;
      memcpy(&b, (const char*)base + 2 * idx, 2);
      return bf16_bits_to_f64(b);
    }
    case PKVO_FP8:
      return pkvo_e4m3_to_f64(((const uint8_t*)base)[idx]);
    default:
      return NAN;
  }
}

/*
 * Gather one sequence's rows for KV head kv_head into a contiguous buffer.
 *   dst   : [L, D] binary64, row t = logical token t
 *   cache : pool [NB, B, Hkv, D] of the given dtype
 *   table : this sequence's block table row (logical block -> physical block)
 * Row t lives in physical block table[t / B] at offset t % B.
 */
int pkvo_gather(double* dst, const void* cache, int dtype, const int32_t* table, int32_t L,
                int64_t NB, int32_t Hkv, int32_t D, int32_t B, int32_t kv_head) {
  if (!elem_bytes(dtype) || L < 0 || Hkv <= 0 || D <= 0 || B <= 0 || kv_head < 0 ||
      kv_head >= Hkv)
    return PKVO_EINVAL;
  for (int32_t t = 0; t < L; ++t) {
    int64_t blk = table[t / B];
    int64_t off = t % B;
    if (blk < 0 || blk >= NB) return PKVO_ERANGE;
    int64_t row = ((blk * B + off) * Hkv + kv_head) * (int64_t)D;
    for (int32_t d = 0; d < D; ++d) dst[(int64_t)t * D + d] = pkvo_load_elem(cache, dtype, row + d);
  }
  return PKVO_OK;
}

/*
 * Textbook softmax attention of one query row over n contiguous rows:
 *   z_t = scale * sum_d q[d] K[t][d];  p_t = exp(z_t - max z) / sum_u exp(z_u - max z)
 *   out[d] = sum_t p_t V[t][d]
 * n == 0 gives out = 0 (an empty context attends to nothing).
 */
int pkvo_attend(double* out, const double* q, const double* K, const double* V, int32_t n,
                int32_t D, double scale) {
  if (n < 0 || D <= 0) return PKVO_EINVAL;
  for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
  if (n == 0) return PKVO_OK;
  double* z = (double*)malloc(sizeof(double) * (size_t)n);
  if (!z) return PKVO_ENOMEM;
  double zmax = -INFINITY;
  for (int32_t t = 0; t < n; ++t) {
    double acc = 0.0;
    for (int32_t d = 0; d < D; ++d) acc += q[d] * K[(int64_t)t * D + d];
    z[t] = scale * acc;
    if (z[t] > zmax) zmax = z[t];
  }
  double denom = 0.0;
  for (int32_t t = 0; t < n; ++t) {
    z[t] = exp(z[t] - zmax);
    denom += z[t];
  }
  for (int32_t t = 0; t < n; ++t) {
    double p = z[t] / denom;
    for (int32_t d = 0; d < D; ++d) out[d] += p * V[(int64_t)t * D + d];
  }
  free(z);
  return PKVO_OK;
}

static int check_shapes(int dtype, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                        int32_t max_nb) {
  if (!elem_bytes(dtype) || S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || B <= 0 || max_nb < 0)
    return PKVO_EINVAL;
  if (Hq % Hkv != 0) return PKVO_EINVAL;
  return PKVO_OK;
}

/*
 * Decode: one query token per sequence attends to all context_lens[s] cached
 * tokens of that sequence (the current token's K/V included).
 *   out  : [S, Hq, D] binary64
 *   q    : [S, Hq, D] in dtype
 *   block_tables : [S, max_nb] int32, context_lens : [S] int32
 */
int pkvo_decode(double* out, const void* q, const void* k_cache, const void* v_cache, int dtype,
                const int32_t* block_tables, int32_t max_nb, const int32_t* context_lens,
                int64_t NB, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                double scale) {
  int rc = check_shapes(dtype, S, Hq, Hkv, D, B, max_nb);
  if (rc) return rc;
  const int32_t G = Hq / Hkv;
  int32_t maxL = 0;
  for (int32_t s = 0; s < S; ++s) {
    int32_t L = context_lens[s];
    if (L < 0 || (int64_t)L > (int64_t)max_nb * B) return PKVO_ERANGE;
    if (L > maxL) maxL = L;
  }
  double* K = (double*)malloc(sizeof(double) * ((size_t)maxL * D + 1));
  double* V = (double*)malloc(sizeof(double) * ((size_t)maxL * D + 1));
  double* qd = (double*)malloc(sizeof(double) * (size_t)D);
  if (!K || !V || !qd) {
    free(K); free(V); free(qd);
    return PKVO_ENOMEM;
  }
  for (int32_t s = 0; s < S && rc == PKVO_OK; ++s) {
    const int32_t L = context_lens[s];
    const int32_t* table = block_tables + (int64_t)s * max_nb;
    for (int32_t g = 0; g < Hkv && rc == PKVO_OK; ++g) {
      rc = pkvo_gather(K, k_cache, dtype, table, L, NB, Hkv, D, B, g);
      if (rc == PKVO_OK) rc = pkvo_gather(V, v_cache, dtype, table, L, NB, Hkv, D, B, g);
      for (int32_t j = 0; j < G && rc == PKVO_OK; ++j) {
        const int32_t h = g * G + j;
        const int64_t base = ((int64_t)s * Hq + h) * D;
        for (int32_t d = 0; d < D; ++d) qd[d] = pkvo_load_elem(q, dtype, base + d);
        rc = pkvo_attend(out + base, qd, K, V, L, D, scale);
      }
    }
  }
  free(K); free(V); free(qd);
  return rc;
}

/*
 * Prefill over a flattened varlen batch (rows of all sequences concatenated):
 *   cu_seqlens_q : [S + 1] prefix sums of per-sequence query-chunk lengths
 *   context_lens : [S] tokens cached per sequence, chunk included
 *   q, out       : [Tq, Hq, D], Tq = cu_seqlens_q[S]
 * Only the query tokens listed in rows[0..n_rows) are computed (rows == NULL
 * means all Tq of them); the other rows of out are left untouched.  Query row
 * i of sequence s is at absolute position L_s - Q_s + i and sees positions
 * 0..L_s - Q_s + i.
 */
static int prefill_rows_impl(double* out, const void* q, int q_dtype,
                             const int32_t* cu_seqlens_q, int32_t Tq, const void* k_cache,
                             const void* v_cache, int kv_dtype, const float* k_scale,
                             const float* v_scale, const int32_t* block_tables, int32_t max_nb,
                             const int32_t* context_lens, int64_t NB, int32_t S, int32_t Hq,
                             int32_t Hkv, int32_t D, int32_t B, double scale, const int32_t* rows,
                             int32_t n_rows) {
  if (q_dtype == PKVO_FP8) return PKVO_EINVAL;
  int rc = check_shapes(q_dtype, S, Hq, Hkv, D, B, max_nb);
  if (rc) return rc;
  if (!elem_bytes(kv_dtype)) return PKVO_EINVAL;
  if (cu_seqlens_q[0] != 0 || cu_seqlens_q[S] != Tq) return PKVO_EINVAL;
  const int32_t G = Hq / Hkv;
  int32_t maxL = 0;
  for (int32_t s = 0; s < S; ++s) {
    int32_t Qs = cu_seqlens_q[s + 1] - cu_seqlens_q[s];
    int32_t L = context_lens[s];
    if (Qs < 0 || L < Qs || (int64_t)L > (int64_t)max_nb * B) return PKVO_ERANGE;
    if (L > maxL) maxL = L;
  }
  if (rows == NULL) n_rows = Tq;
  /* mark which query rows are wanted */
  unsigned char* want = (unsigned char*)calloc((size_t)Tq + 1, 1);
  double* K = (double*)malloc(sizeof(double) * ((size_t)maxL * D + 1));
  double* V = (double*)malloc(sizeof(double) * ((size_t)maxL * D + 1));
  double* qd = (double*)malloc(sizeof(double) * (size_t)D);
  if (!want || !K || !V || !qd) {
    free(want); free(K); free(V); free(qd);
    return PKVO_ENOMEM;
  }
  for (int32_t r = 0; r < n_rows; ++r) {
    int32_t row = rows ? rows[r] : r;
    if (row < 0 || row >= Tq) {
      rc = PKVO_ERANGE;
      break;
    }
    want[row] = 1;
  }
  for (int32_t s = 0; s < S && rc == PKVO_OK; ++s) {
    const int32_t r0 = cu_seqlens_q[s], Qs = cu_seqlens_q[s + 1] - r0, L = context_lens[s];
    int any = 0;
    for (int32_t i = 0; i < Qs; ++i) any |= want[r0 + i];
    if (!any) continue;
    const int32_t* table = block_tables + (int64_t)s * max_nb;
    for (int32_t g = 0; g < Hkv && rc == PKVO_OK; ++g) {
      rc = pkvo_gather(K, k_cache, kv_dtype, table, L, NB, Hkv, D, B, g);
      if (rc == PKVO_OK) rc = pkvo_gather(V, v_cache, kv_dtype, table, L, NB, Hkv, D, B, g);
      if (k_scale && v_scale) {
        for (int64_t e = 0; e < (int64_t)L * D; ++e) {
          K[e] *= (double)k_scale[g];
          V[e] *= (double)v_scale[g];
        }
      }
      for (int32_t i = 0; i < Qs && rc == PKVO_OK; ++i) {
        if (!want[r0 + i]) continue;
        const int32_t visible = L - Qs + i + 1; /* positions 0 .. L-Qs+i */
        for (int32_t j = 0; j < G && rc == PKVO_OK; ++j) {
          const int32_t h = g * G + j;
          const int64_t base = ((int64_t)(r0 + i) * Hq + h) * D;
          for (int32_t d = 0; d < D; ++d) qd[d] = pkvo_load_elem(q, q_dtype, base + d);
          rc = pkvo_attend(out + base, qd, K, V, visible, D, scale);
        }
      }
    }
  }
  free(want); free(K); free(V); free(qd);
  return rc;
}

int pkvo_prefill_rows(double* out, const void* q, const int32_t* cu_seqlens_q, int32_t Tq,
                      const void* k_cache, const void* v_cache, int dtype,
                      const int32_t* block_tables, int32_t max_nb, const int32_t* context_lens,
                      int64_t NB, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                      double scale, const int32_t* rows, int32_t n_rows) {
  return prefill_rows_impl(out, q, dtype, cu_seqlens_q, Tq, k_cache, v_cache, dtype, NULL, NULL,
                           block_tables, max_nb, context_lens, NB, S, Hq, Hkv, D, B, scale, rows,
                           n_rows);
}

/*
 * Prefill over FP8 pools: as pkvo_prefill_rows, with q in q_dtype and every
 * cached element read as code * scale of its KV head (the same reading of an
 * FP8 pool as pkvo_decode_fp8).
 */
int pkvo_prefill_fp8_rows(double* out, const void* q, int q_dtype, const int32_t* cu_seqlens_q,
                          int32_t Tq, const uint8_t* k_cache, const uint8_t* v_cache,
                          const float* k_scale, const float* v_scale, const int32_t* block_tables,
                          int32_t max_nb, const int32_t* context_lens, int64_t NB, int32_t S,
                          int32_t Hq, int32_t Hkv, int32_t D, int32_t B, double scale,
                          const int32_t* rows, int32_t n_rows) {
  if (!k_scale || !v_scale) return PKVO_EINVAL;
  return prefill_rows_impl(out, q, q_dtype, cu_seqlens_q, Tq, k_cache, v_cache, PKVO_FP8, k_scale,
                           v_scale, block_tables, max_nb, context_lens, NB, S, Hq, Hkv, D, B,
                           scale, rows, n_rows);
}

int pkvo_prefill(double* out, const void* q, const int32_t* cu_seqlens_q, int32_t Tq,
                 const void* k_cache, const void* v_cache, int dtype,
                 const int32_t* block_tables, int32_t max_nb, const int32_t* context_lens,
                 int64_t NB, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                 double scale) {
  return pkvo_prefill_rows(out, q, cu_seqlens_q, Tq, k_cache, v_cache, dtype, block_tables,
                           max_nb, context_lens, NB, S, Hq, Hkv, D, B, scale, NULL, 0);
}

/*
 * reshape_and_cache: token t's K row [Hkv, D] (and V row) goes to slot
 * slot_mapping[t] = blk * B + off of the pool [NB, B, Hkv, D]; slots < 0 are
 * skipped.  Bytes are copied unchanged.
 */
int pkvo_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                           const int64_t* slot_mapping, int32_t T, int32_t Hkv, int32_t D,
                           int32_t B, int64_t NB, int dtype) {
  const int eb = elem_bytes(dtype);
  if (!eb || T < 0 || Hkv <= 0 || D <= 0 || B <= 0 || NB <= 0) return PKVO_EINVAL;
  const size_t row_bytes = (size_t)Hkv * D * eb;
  for (int32_t t = 0; t < T; ++t) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    if (slot >= NB * B) return PKVO_ERANGE;
    const int64_t blk = slot / B, off = slot % B;
    const size_t dst = (size_t)(blk * B + off) * row_bytes;
    memcpy((char*)k_cache + dst, (const char*)key + (size_t)t * row_bytes, row_bytes);
    memcpy((char*)v_cache + dst, (const char*)value + (size_t)t * row_bytes, row_bytes);
  }
  return PKVO_OK;
}

/*
 * copy_blocks: for every layer and every (src, dst) pair, block dst of the K
 * pool and of the V pool becomes a copy of block src.  All pairs read the
 * state from before the call (sources are snapshotted first).
 */
int pkvo_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                     const int64_t* pairs, int32_t N, int32_t B, int32_t Hkv, int32_t D,
                     int64_t NB, int dtype) {
  const int eb = elem_bytes(dtype);
  if (!eb || num_layers < 0 || N < 0 || B <= 0 || Hkv <= 0 || D <= 0) return PKVO_EINVAL;
  for (int32_t i = 0; i < N; ++i)
    if (pairs[2 * i] < 0 || pairs[2 * i] >= NB || pairs[2 * i + 1] < 0 || pairs[2 * i + 1] >= NB)
      return PKVO_ERANGE;
  const size_t blk_bytes = (size_t)B * Hkv * D * eb;
  char* snap = (char*)malloc(blk_bytes * (size_t)(N > 0 ? N : 1) * 2);
  if (!snap) return PKVO_ENOMEM;
  for (int32_t l = 0; l < num_layers; ++l) {
    char* kc = (char*)k_caches[l];
    char* vc = (char*)v_caches[l];
    for (int32_t i = 0; i < N; ++i) {
      memcpy(snap + (size_t)(2 * i) * blk_bytes, kc + (size_t)pairs[2 * i] * blk_bytes, blk_bytes);
      memcpy(snap + (size_t)(2 * i + 1) * blk_bytes, vc + (size_t)pairs[2 * i] * blk_bytes,
             blk_bytes);
    }
    for (int32_t i = 0; i < N; ++i) {
      memcpy(kc + (size_t)pairs[2 * i + 1] * blk_bytes, snap + (size_t)(2 * i) * blk_bytes,
             blk_bytes);
      memcpy(vc + (size_t)pairs[2 * i + 1] * blk_bytes, snap + (size_t)(2 * i + 1) * blk_bytes,
             blk_bytes);
    }
  }
  free(snap);
  return PKVO_OK;
}

/* Exact binary32 value of element idx of a 16- or 32-bit stored array (every
 * fp16 and bf16 value is exactly representable in binary32). */
static float load_f32(const void* base, int dtype, int64_t idx) {
  return (float)pkvo_load_elem(base, dtype, idx);
}

/*
 * Quantizing reshape_and_cache for an FP8 pool: token t's K row [Hkv, D] (in
 * in_dtype) goes to slot slot_mapping[t] of the pool [NB, B, Hkv, D] of E4M3
 * codes, element (h, d) stored as e4m3(fp32(key) / k_scale[h]); V likewise
 * with v_scale.  Slots < 0 are skipped.
 */
int pkvo_reshape_and_cache_fp8(const void* key, const void* value, int in_dtype, uint8_t* k_cache,
                               uint8_t* v_cache, const int64_t* slot_mapping, int32_t T,
                               int32_t Hkv, int32_t D, int32_t B, int64_t NB,
                               const float* k_scale, const float* v_scale) {
  if (in_dtype == PKVO_FP8 || !elem_bytes(in_dtype) || T < 0 || Hkv <= 0 || D <= 0 || B <= 0 ||
      NB <= 0)
    return PKVO_EINVAL;
  for (int32_t t = 0; t < T; ++t) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    if (slot >= NB * B) return PKVO_ERANGE;
    for (int32_t h = 0; h < Hkv; ++h) {
      for (int32_t d = 0; d < D; ++d) {
        const int64_t src = ((int64_t)t * Hkv + h) * D + d;
        const int64_t dst = (slot * Hkv + h) * D + d;
        const float kq = load_f32(key, in_dtype, src) / k_scale[h];
        const float vq = load_f32(value, in_dtype, src) / v_scale[h];
        k_cache[dst] = pkvo_e4m3_from_f32(kq);
        v_cache[dst] = pkvo_e4m3_from_f32(vq);
      }
    }
  }
  return PKVO_OK;
}

/*
 * Decode over an FP8 pool: as pkvo_decode, with q in q_dtype and every cached
 * element read as code * scale of its KV head (k_scale for K, v_scale for V;
 * the products are exact in binary64).
 */
int pkvo_decode_fp8(double* out, const void* q, int q_dtype, const uint8_t* k_cache,
                    const uint8_t* v_cache, const float* k_scale, const float* v_scale,
                    const int32_t* block_tables, int32_t max_nb, const int32_t* context_lens,
                    int64_t NB, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                    double scale) {
  if (q_dtype == PKVO_FP8) return PKVO_EINVAL;
  int rc = check_shapes(q_dtype, S, Hq, Hkv, D, B, max_nb);
  if (rc) return rc;
  const int32_t G = Hq / Hkv;
  int32_t maxL = 0;
  for (int32_t s = 0; s < S; ++s) {
    int32_t L = context_lens[s];
    if (L < 0 || (int64_t)L > (int64_t)max_nb * B) return PKVO_ERANGE;
    if (L > maxL) maxL = L;
  }
  double* K = (double*)malloc(sizeof(double) * ((size_t)maxL * D + 1));
  double* V = (double*)malloc(sizeof(double) * ((size_t)maxL * D + 1));
  double* qd = (double*)malloc(sizeof(double) * (size_t)D);
  if (!K || !V || !qd) {
    free(K); free(V); free(qd);
    return PKVO_ENOMEM;
  }
  for (int32_t s = 0; s < S && rc == PKVO_OK; ++s) {
    const int32_t L = context_lens[s];
    const int32_t* table = block_tables + (int64_t)s * max_nb;
    for (int32_t g = 0; g < Hkv && rc == PKVO_OK; ++g) {
      rc = pkvo_gather(K, k_cache, PKVO_FP8, table, L, NB, Hkv, D, B, g);
      if (rc == PKVO_OK) rc = pkvo_gather(V, v_cache, PKVO_FP8, table, L, NB, Hkv, D, B, g);
      for (int64_t i = 0; i < (int64_t)L * D; ++i) {
        K[i] *= (double)k_scale[g];
        V[i] *= (double)v_scale[g];
      }
      for (int32_t j = 0; j < G && rc == PKVO_OK; ++j) {
        const int32_t h = g * G + j;
        const int64_t base = ((int64_t)s * Hq + h) * D;
        for (int32_t d = 0; d < D; ++d) qd[d] = pkvo_load_elem(q, q_dtype, base + d);
        rc = pkvo_attend(out + base, qd, K, V, L, D, scale);
      }
    }
  }
  free(K); free(V); free(qd);
  return rc;
}

/*
 * swap_blocks: for every pool p and pair i, block pairs[2i+1] of dst_pools[p]
 * becomes a copy of block pairs[2i] of src_pools[p] (block_bytes each; the
 * sources have NB_src blocks, the destinations NB_dst).
 */
int pkvo_swap_blocks(void* const* src_pools, void* const* dst_pools, int32_t num_pools,
                     const int64_t* pairs, int32_t N, int64_t block_bytes, int64_t NB_src,
                     int64_t NB_dst) {
  if (num_pools < 0 || N < 0 || block_bytes <= 0) return PKVO_EINVAL;
  for (int32_t i = 0; i < N; ++i)
    if (pairs[2 * i] < 0 || pairs[2 * i] >= NB_src || pairs[2 * i + 1] < 0 ||
        pairs[2 * i + 1] >= NB_dst)
      return PKVO_ERANGE;
  for (int32_t p = 0; p < num_pools; ++p)
    for (int32_t i = 0; i < N; ++i)
      memcpy((char*)dst_pools[p] + (size_t)pairs[2 * i + 1] * (size_t)block_bytes,
             (const char*)src_pools[p] + (size_t)pairs[2 * i] * (size_t)block_bytes,
             (size_t)block_bytes);
  return PKVO_OK;
}
