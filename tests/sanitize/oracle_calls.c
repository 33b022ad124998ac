/* The fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every
 * exported function on small seeded inputs, including empty contexts, one-row
 * contexts, ragged last blocks, negative slots and every E4M3 code.  Exit
 * status 0 = clean. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double pkvo_load_elem(const void* base, int dtype, int64_t idx);
double pkvo_e4m3_to_f64(uint8_t code);
uint8_t pkvo_e4m3_from_f32(float x);
int pkvo_decode(double* out, const void* q, const void* k, const void* v, int dtype,
                const int32_t* tables, int32_t max_nb, const int32_t* lens, int64_t NB, int32_t S,
                int32_t Hq, int32_t Hkv, int32_t D, int32_t B, double scale);
int pkvo_prefill(double* out, const void* q, const int32_t* cu, int32_t Tq, const void* k,
                 const void* v, int dtype, const int32_t* tables, int32_t max_nb,
                 const int32_t* lens, int64_t NB, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                 int32_t B, double scale);
int pkvo_prefill_fp8_rows(double* out, const void* q, int q_dtype, const int32_t* cu, int32_t Tq,
                          const uint8_t* k, const uint8_t* v, const float* ks, const float* vs,
                          const int32_t* tables, int32_t max_nb, const int32_t* lens, int64_t NB,
                          int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B, double scale,
                          const int32_t* rows, int32_t n_rows);
int pkvo_reshape_and_cache(const void* key, const void* value, void* k, void* v,
                           const int64_t* slots, int32_t T, int32_t Hkv, int32_t D, int32_t B,
                           int64_t NB, int dtype);
int pkvo_reshape_and_cache_fp8(const void* key, const void* value, int in_dtype, uint8_t* k,
                               uint8_t* v, const int64_t* slots, int32_t T, int32_t Hkv, int32_t D,
                               int32_t B, int64_t NB, const float* ks, const float* vs);
int pkvo_decode_fp8(double* out, const void* q, int q_dtype, const uint8_t* k, const uint8_t* v,
                    const float* ks, const float* vs, const int32_t* tables, int32_t max_nb,
                    const int32_t* lens, int64_t NB, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                    int32_t B, double scale);
int pkvo_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                     const int64_t* pairs, int32_t N, int32_t B, int32_t Hkv, int32_t D, int64_t NB,
                     int dtype);
int pkvo_swap_blocks(void* const* src, void* const* dst, int32_t num_pools, const int64_t* pairs,
                     int32_t N, int64_t block_bytes, int64_t src_nb, int64_t dst_nb);

#define CHECK(x)                                                       \
  do {                                                                 \
    if (!(x)) {                                                        \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #x);     \
      return 1;                                                        \
    }                                                                  \
  } while (0)

static uint32_t rng_state = 12345u;
static uint16_t rnd16(void) { /* xorshift32, finite bf16/f16 patterns */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 17;
  rng_state ^= rng_state << 5;
  return (uint16_t)((rng_state & 0x3fffu) | ((rng_state >> 16) & 0x8000u));
}

int main(void) {
  enum { S = 4, Hq = 4, Hkv = 2, D = 8, B = 4, NB = 16, MAXNB = 4 };
  const int32_t lens[S] = {0, 1, 7, 16};
  int32_t tables[S * MAXNB];
  for (int i = 0; i < S * MAXNB; ++i) tables[i] = (i * 7) % NB;
  for (int dt = 0; dt < 3; ++dt) {
    const size_t es = dt == 0 ? 4 : 2, pool = (size_t)NB * B * Hkv * D;
    unsigned char* k = malloc(pool * es);
    unsigned char* v = malloc(pool * es);
    unsigned char* q = malloc((size_t)S * Hq * D * es);
    for (size_t i = 0; i < pool; ++i) {
      if (es == 4) {
        float a = (float)((int)rnd16() % 200 - 100) / 50.f, b = (float)((int)rnd16() % 200 - 100) / 50.f;
        memcpy(k + 4 * i, &a, 4);
        memcpy(v + 4 * i, &b, 4);
      } else {
        uint16_t a = rnd16(), b = rnd16();
        memcpy(k + 2 * i, &a, 2);
        memcpy(v + 2 * i, &b, 2);
      }
    }
    for (size_t i = 0; i < (size_t)S * Hq * D; ++i) {
      uint16_t a = rnd16();
      if (es == 4) {
        float f = (float)(a % 100) / 40.f;
        memcpy(q + 4 * i, &f, 4);
      } else {
        memcpy(q + 2 * i, &a, 2);
      }
    }
    double out[S * Hq * D];
    CHECK(pkvo_decode(out, q, k, v, dt, tables, MAXNB, lens, NB, S, Hq, Hkv, D, B, 0.3) == 0);
    for (int i = 0; i < Hq * D; ++i) CHECK(out[i] == 0.0); /* empty context */
    const int32_t cu[S + 1] = {0, 0, 1, 4, 9};
    CHECK(pkvo_prefill(out, q, cu, S, k, v, dt, tables, MAXNB, lens, NB, S, Hq, Hkv, D, B, 0.3) !=
          0); /* cu[S] != Tq */
    const int32_t cu2[S + 1] = {0, 0, 1, 3, 4};
    CHECK(pkvo_prefill(out, q, cu2, 4, k, v, dt, tables, MAXNB, lens, NB, S, Hq, Hkv, D, B, 0.3) == 0);
    int64_t slots[3] = {5, -1, NB * B - 1};
    CHECK(pkvo_reshape_and_cache(q, q, k, v, slots, 3, Hkv, D, B, NB, dt) == 0);
    int64_t bad[1] = {NB * B};
    CHECK(pkvo_reshape_and_cache(q, q, k, v, bad, 1, Hkv, D, B, NB, dt) != 0);
    void* kp[2] = {k, k};
    void* vp[2] = {v, v};
    int64_t pairs[4] = {1, 9, 2, 10};
    CHECK(pkvo_copy_blocks(kp, vp, 1, pairs, 2, B, Hkv, D, NB, dt) == 0);
    void* src[1] = {k};
    void* dst[1] = {v};
    CHECK(pkvo_swap_blocks(src, dst, 1, pairs, 2, (int64_t)B * Hkv * D * es, NB, NB) == 0);
    (void)pkvo_load_elem(k, dt, (int64_t)pool - 1);
    free(k);
    free(v);
    free(q);
  }
  /* FP8: every code both ways, quantizing reshape, decode and prefill */
  for (int c = 0; c < 256; ++c) {
    const double x = pkvo_e4m3_to_f64((uint8_t)c);
    if (!isnan(x)) CHECK(pkvo_e4m3_from_f32((float)x) == (uint8_t)c || x == 0.0);
  }
  {
    const size_t pool = (size_t)NB * B * Hkv * D;
    uint8_t* k = malloc(pool);
    uint8_t* v = malloc(pool);
    uint16_t* q = malloc(sizeof(uint16_t) * S * Hq * D);
    for (size_t i = 0; i < pool; ++i) {
      k[i] = (uint8_t)(rnd16() & 0x7e);
      v[i] = (uint8_t)(rnd16() & 0xfe) & 0xf7;
    }
    for (int i = 0; i < S * Hq * D; ++i) q[i] = rnd16();
    const float ks[Hkv] = {0.01f, 0.02f}, vs[Hkv] = {0.005f, 0.03f};
    double out[S * Hq * D];
    CHECK(pkvo_decode_fp8(out, q, 2, k, v, ks, vs, tables, MAXNB, lens, NB, S, Hq, Hkv, D, B, 0.2) == 0);
    const int32_t cu[S + 1] = {0, 0, 1, 3, 4}, rows[2] = {1, 3};
    CHECK(pkvo_prefill_fp8_rows(out, q, 1, cu, 4, k, v, ks, vs, tables, MAXNB, lens, NB, S, Hq,
                                Hkv, D, B, 0.2, rows, 2) == 0);
    int64_t slots[2] = {3, -7};
    CHECK(pkvo_reshape_and_cache_fp8(q, q, 2, k, v, slots, 2, Hkv, D, B, NB, ks, vs) == 0);
    free(k);
    free(v);
    free(q);
  }
  puts("oracle_calls clean");
  return 0;
}
