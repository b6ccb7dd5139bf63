/* Calls every function of the CPU oracle (oracle/oracle.h) on small pools:
 * codecs over every input, scatter with skipped and out-of-range slots, block
 * copies, decode and split decode with windows and empty contexts, prefill.
 * Built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py; the run aborts on any invalid access or undefined
 * behaviour. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);         \
      abort();                                                                \
    }                                                                         \
  } while (0)

static uint32_t rng_state = 12345u;
static uint32_t next_u32(void) {
  rng_state = rng_state * 1664525u + 1013904223u;
  return rng_state >> 8;
}
/* a binary16 bit pattern of a finite value in about [-4, 4] */
static uint16_t small_f16(void) { return (uint16_t)(((next_u32() & 1u) << 15) | (0x3000u + next_u32() % 0x1400u)); }

static void run(int elem_bytes, int fp8_format, int bs, int Hkv, int D, int window) {
  const int nb = 24, S = 5, g = 2, Hq = Hkv * g, max_blocks = 6;
  const size_t pool_elems = (size_t)nb * bs * Hkv * D;
  void* k = calloc(pool_elems, (size_t)elem_bytes);
  void* v = calloc(pool_elems, (size_t)elem_bytes);
  double khs[4] = {0.5, 1.0, 2.0, 0.25}, vhs[4] = {1.0, 0.125, 4.0, 2.0};
  orc_pool p = {k, v, nb, 0, bs, Hkv, D, elem_bytes, fp8_format, 0.03, 0.02,
                elem_bytes == 1 && Hkv <= 4 ? khs : NULL, elem_bytes == 1 && Hkv <= 4 ? vhs : NULL,
                window};
  /* tables: a permutation of the pool's blocks */
  int32_t bt[5 * 6], lens[5] = {0, 1, bs + 3, 3 * bs, max_blocks * bs};
  for (int i = 0; i < S * max_blocks; ++i) bt[i] = i % nb;
  /* write every position of every sequence, plus skipped slots */
  const int T = max_blocks * bs * S + 3;
  uint16_t* kn = malloc(sizeof(uint16_t) * (size_t)T * Hkv * D);
  uint16_t* vn = malloc(sizeof(uint16_t) * (size_t)T * Hkv * D);
  int64_t* slots = malloc(sizeof(int64_t) * (size_t)T);
  for (size_t i = 0; i < (size_t)T * Hkv * D; ++i) { kn[i] = small_f16(); vn[i] = small_f16(); }
  for (int t = 0; t < T - 3; ++t) slots[t] = (int64_t)(t % (nb * bs));
  slots[T - 3] = -1;
  slots[T - 2] = (int64_t)nb * bs;           /* past the pool: skipped */
  slots[T - 1] = -7;
  orc_scatter(&p, kn, vn, slots, T, 2);
  int64_t pairs[4] = {1, 20, 2, 21};
  orc_copy_blocks(&p, pairs, 2);
  uint16_t* q = malloc(sizeof(uint16_t) * (size_t)S * Hq * D);
  for (int i = 0; i < S * Hq * D; ++i) q[i] = small_f16();
  double* out = malloc(sizeof(double) * (size_t)S * Hq * D);
  double* out2 = malloc(sizeof(double) * (size_t)S * Hq * D);
  orc_decode(&p, q, S, Hq, bt, max_blocks, lens, 0.125f, NULL, 0, out, 2);
  orc_decode_split(&p, q, S, Hq, bt, max_blocks, lens, 0.125f, 16, NULL, 0, out2, 2);
  for (int i = 0; i < S * Hq * D; ++i) {
    CHECK(isfinite(out[i]));
    CHECK(fabs(out[i] - out2[i]) <= 1e-12 * (1.0 + fabs(out[i])));
  }
  int32_t units[4] = {2, 0, 4, Hkv - 1};
  orc_decode(&p, q, S, Hq, bt, max_blocks, lens, 0.125f, units, 2, out, 1);
  double* Kc = malloc(sizeof(double) * (size_t)max_blocks * bs * D);
  double* Vc = malloc(sizeof(double) * (size_t)max_blocks * bs * D);
  orc_gather_head(&p, bt, lens[4], Hkv - 1, Kc, Vc);
  double qd[256], o[256];
  for (int d = 0; d < D; ++d) qd[d] = (double)(d % 7) - 3.0;
  orc_attend(qd, Kc, Vc, lens[4], D, 0.1, o);
  orc_attend(qd, Kc, Vc, 0, D, 0.1, o);
  /* prefill: every sequence's last q_len positions are new */
  int32_t qs[6] = {0, 0, 1, 1 + bs + 3, 1 + bs + 3 + 7, 1 + bs + 3 + 7 + 2 * bs};
  const int total_q = qs[5];
  uint16_t* qp = malloc(sizeof(uint16_t) * (size_t)total_q * Hq * D);
  for (int i = 0; i < total_q * Hq * D; ++i) qp[i] = small_f16();
  double* op = malloc(sizeof(double) * (size_t)total_q * Hq * D);
  orc_prefill(&p, qp, qs, S, Hq, bt, max_blocks, lens, 0.125f, NULL, 0, op, 2);
  int32_t rows[6] = {3, 0, 6, 4, Hkv - 1, 0};
  orc_prefill(&p, qp, qs, S, Hq, bt, max_blocks, lens, 0.125f, rows, 2, op, 1);
  for (int i = 0; i < total_q * Hq * D; ++i) CHECK(isfinite(op[i]));
  free(k); free(v); free(kn); free(vn); free(slots); free(q); free(out); free(out2);
  free(Kc); free(Vc); free(qp); free(op);
}

int main(void) {
  /* codecs over every input */
  for (uint32_t b = 0; b < 65536; ++b) (void)orc_f16_value((uint16_t)b);
  for (uint32_t b = 0; b < 256; ++b) {
    (void)orc_e4m3fn_value((uint8_t)b);
    (void)orc_e5m2_value((uint8_t)b);
  }
  for (uint32_t i = 0; i < 200000; ++i) {
    uint32_t bits = next_u32() * 2654435761u;
    float x;
    memcpy(&x, &bits, 4);
    (void)orc_e4m3fn_encode(x);
    (void)orc_e5m2_encode(x);
  }
  CHECK(orc_e4m3fn_encode(INFINITY) == 0x7E && orc_e4m3fn_encode(NAN) == 0x7F);
  const int shapes[][5] = {{2, 0, 16, 2, 64}, {2, 0, 8, 4, 128}, {1, 0, 16, 2, 64},
                           {1, 1, 32, 4, 128}, {1, 0, 8, 1, 256}, {2, 0, 32, 1, 256}};
  for (int i = 0; i < 6; ++i)
    for (int w = 0; w < 3; ++w)
      run(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], shapes[i][4],
          w == 0 ? 0 : (w == 1 ? 1 : 2 * shapes[i][2] + 5));
  printf("oracle_stress ok\n");
  return 0;
}
