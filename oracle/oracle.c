/*
 * oracle.c -- plain CPU reference for paged-attention decode, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Every routine is the plain
 * definition: gather the context through the block table into contiguous rows,
 * then evaluate softmax(scale * q.K^T) V with the max subtracted, in double
 * precision.  No blocking, fusion or reordering beyond that.
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- codecs */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent 0 holds zero and subnormals (fraction * 2^-24); 31 holds inf/NaN. */
double orc_f16_value(uint16_t bits) {
  int sign = bits >> 15;
  int e = (bits >> 10) & 0x1F;
  int f = bits & 0x3FF;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + f), e - 25);
  }
  return sign ? -v : v;
}

/* OCP e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent 0 holds zero and subnormals (m * 2^-9).  There are no infinities;
 * exponent 15 with mantissa 7 is NaN, so the largest finite value is
 * 1.75 * 2^8 = 448. */
double orc_e4m3fn_value(uint8_t byte) {
  int sign = byte >> 7;
  int e = (byte >> 3) & 0xF;
  int m = byte & 0x7;
  double v;
  if (e == 15 && m == 7) {
    v = NAN;
  } else if (e == 0) {
    v = ldexp((double)m, -9);
  } else {
    v = ldexp((double)(8 + m), e - 10); /* 2^(e-7) * (1 + m/8) */
  }
  return sign ? -v : v;
}

/* Round a non-negative double to the nearest integer, ties to the even one. */
static double round_half_even(double n) {
  double fl = floor(n);
  double frac = n - fl;
  if (frac > 0.5) return fl + 1.0;
  if (frac < 0.5) return fl;
  return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* fp32 -> e4m3fn.  Steps: NaN stays NaN (sign kept, S.1111.111); magnitudes at
 * or beyond the largest finite value saturate to 448 (values in (448, 464)
 * would round to 448 anyway, and 464 is a tie that rounds to the even
 * mantissa 448); otherwise find the binade, count quanta of that binade and
 * round the count to nearest even.  Below 2^-6 the quantum is the subnormal
 * step 2^-9. */
uint8_t orc_e4m3fn_encode(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(sign | 0x7F);
  double a = fabs((double)x);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  if (a == 0.0) return sign;
  int ex;
  (void)frexp(a, &ex);           /* a = fr * 2^ex, fr in [0.5, 1) */
  int E = ex - 1;                /* a = 2^E * (1.f)                 */
  if (E < -6) {
    double n = round_half_even(a * 512.0);   /* quanta of 2^-9: 0..8 */
    return (uint8_t)(sign | (uint8_t)n);     /* 8 is the smallest normal, 0x08 */
  }
  double quantum = ldexp(1.0, E - 3);
  double n = round_half_even(a / quantum);   /* 8..16 */
  if (n == 16.0) {
    E += 1;
    n = 8.0;
  }
  int code = ((E + 7) << 3) | ((int)n - 8);
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)(sign | code);
}

/* OCP e5m2: 1 sign bit, 5 exponent bits (bias 15), 2 mantissa bits.
 * Exponent 0 holds zero and subnormals (m * 2^-16); exponent 31 holds the
 * infinities (m = 0) and NaN (m != 0), so the largest finite value is
 * 1.75 * 2^15 = 57344. */
double orc_e5m2_value(uint8_t byte) {
  int sign = byte >> 7;
  int e = (byte >> 2) & 0x1F;
  int m = byte & 0x3;
  double v;
  if (e == 31) {
    v = m ? NAN : INFINITY;
  } else if (e == 0) {
    v = ldexp((double)m, -16);
  } else {
    v = ldexp((double)(4 + m), e - 17); /* 2^(e-15) * (1 + m/4) */
  }
  return sign ? -v : v;
}

/* fp32 -> e5m2, the same steps as for e4m3fn with this format's constants:
 * NaN stays NaN (sign kept, S.11111.11); magnitudes at or beyond the largest
 * finite value, infinities included, saturate to 57344 (S.11110.11); otherwise
 * count quanta of the binade (2^(E-2)) and round the count to nearest even.
 * Below 2^-14 the quantum is the subnormal step 2^-16. */
uint8_t orc_e5m2_encode(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(sign | 0x7F);
  double a = fabs((double)x);
  if (a >= 57344.0) return (uint8_t)(sign | 0x7B);
  if (a == 0.0) return sign;
  int ex;
  (void)frexp(a, &ex);           /* a = fr * 2^ex, fr in [0.5, 1) */
  int E = ex - 1;                /* a = 2^E * (1.f)                 */
  if (E < -14) {
    double n = round_half_even(a * 65536.0);  /* quanta of 2^-16: 0..4 */
    return (uint8_t)(sign | (uint8_t)n);      /* 4 is the smallest normal, 0x04 */
  }
  double quantum = ldexp(1.0, E - 2);
  double n = round_half_even(a / quantum);    /* 4..8 */
  if (n == 8.0) {
    E += 1;
    n = 4.0;
  }
  int code = ((E + 15) << 2) | ((int)n - 4);
  if (code > 0x7B) code = 0x7B;
  return (uint8_t)(sign | code);
}

void orc_e5m2_values(const uint8_t* bytes, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e5m2_value(bytes[i]);
}

void orc_e5m2_encode_n(const float* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e5m2_encode(x[i]);
}

void orc_f16_values(const uint16_t* bits, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_value(bits[i]);
}

void orc_e4m3fn_values(const uint8_t* bytes, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3fn_value(bytes[i]);
}

void orc_e4m3fn_encode_n(const float* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3fn_encode(x[i]);
}

/* ------------------------------------------------------------ pool access */

static int64_t block_stride_of(const orc_pool* p) {
  if (p->block_stride) return p->block_stride;
  return (int64_t)p->block_size * p->num_kv_heads * p->head_dim * p->elem_bytes;
}

/* Byte offset of element (block, offset-in-block, kv head, dim). */
static int64_t elem_offset(const orc_pool* p, int64_t blk, int32_t off, int32_t kh, int32_t d) {
  int64_t in_block = (((int64_t)off * p->num_kv_heads + kh) * p->head_dim + d) * p->elem_bytes;
  return blk * block_stride_of(p) + in_block;
}

static double read_elem(const orc_pool* p, const void* base, int64_t byte_off, double scale) {
  const uint8_t* b = (const uint8_t*)base + byte_off;
  if (p->elem_bytes == 2) {
    uint16_t bits;
    memcpy(&bits, b, 2);
    return orc_f16_value(bits);
  }
  return (p->fp8_format == ORC_FP8_E5M2 ? orc_e5m2_value(*b) : orc_e4m3fn_value(*b)) * scale;
}

static int nthreads_or_default(int n) { return n > 0 ? n : omp_get_max_threads(); }

/* The dequantisation scale of KV head kh: per head when given, else per tensor. */
static double k_scale_of(const orc_pool* p, int32_t kh) {
  return p->k_head_scales ? p->k_head_scales[kh] : p->k_scale;
}
static double v_scale_of(const orc_pool* p, int32_t kh) {
  return p->v_head_scales ? p->v_head_scales[kh] : p->v_scale;
}

/* ---------------------------------------------------------------- writes */

static int slot_ok(const orc_pool* p, int64_t slot) {
  return slot >= 0 && slot < p->num_blocks * p->block_size;
}

/* Per-block scales: runs of consecutive tokens in one block, taken one after
 * another (the rule is spelled out in oracle.h). */
static void scatter_per_block(const orc_pool* p, const uint16_t* k_new, const uint16_t* v_new,
                              const int64_t* slots, int64_t T) {
  const int32_t Hkv = p->num_kv_heads, D = p->head_dim, bs = p->block_size;
  const int e5m2 = p->fp8_format == ORC_FP8_E5M2;
  const float fmax_fmt = e5m2 ? 57344.0f : 448.0f;
  char* written = (char*)malloc((size_t)bs);
  int64_t i = 0;
  while (i < T) {
    if (!slot_ok(p, slots[i])) {
      ++i;
      continue;
    }
    const int64_t blk = slots[i] / bs;
    int64_t j = i + 1;
    while (j < T && slot_ok(p, slots[j]) && slots[j] / bs == blk) ++j;
    memset(written, 0, (size_t)bs);
    for (int64_t t = i; t < j; ++t) written[slots[t] % bs] = 1;
    const int fresh = written[0];
    for (int which = 0; which < 2; ++which) {
      uint8_t* pool = (uint8_t*)(which ? p->v : p->k);
      const uint16_t* src = which ? v_new : k_new;
      float* scales = which ? p->v_block_scales : p->k_block_scales;
      for (int32_t kh = 0; kh < Hkv; ++kh) {
        float amax = 0.0f;
        for (int64_t t = i; t < j; ++t)
          for (int32_t d = 0; d < D; ++d) {
            const float x = (float)orc_f16_value(src[(t * Hkv + kh) * D + d]);
            if (isfinite(x)) amax = fmaxf(amax, fabsf(x));
          }
        const float c = fmaxf(amax / fmax_fmt, FLT_MIN);
        const float old = scales[blk * Hkv + kh];
        const float nw = fresh ? c : fmaxf(old, c);
        if (!fresh && nw > old) {
          for (int32_t o = 0; o < bs; ++o) {
            if (written[o]) continue;
            for (int32_t d = 0; d < D; ++d) {
              uint8_t* b = pool + elem_offset(p, blk, o, kh, d);
              const float v = (float)(e5m2 ? orc_e5m2_value(*b) : orc_e4m3fn_value(*b));
              const float y = (v * old) / nw;
              *b = e5m2 ? orc_e5m2_encode(y) : orc_e4m3fn_encode(y);
            }
          }
        }
        for (int64_t t = i; t < j; ++t) {
          const int32_t off = (int32_t)(slots[t] % bs);
          for (int32_t d = 0; d < D; ++d) {
            const float x = (float)orc_f16_value(src[(t * Hkv + kh) * D + d]);
            pool[elem_offset(p, blk, off, kh, d)] =
                e5m2 ? orc_e5m2_encode(x / nw) : orc_e4m3fn_encode(x / nw);
          }
        }
        scales[blk * Hkv + kh] = nw;
      }
    }
    i = j;
  }
  free(written);
}

void orc_scatter(const orc_pool* p, const uint16_t* k_new, const uint16_t* v_new,
                 const int64_t* slots, int64_t T, int nthreads) {
  const int32_t Hkv = p->num_kv_heads, D = p->head_dim;
  if (p->elem_bytes == 1 && p->k_block_scales) {
    scatter_per_block(p, k_new, v_new, slots, T);
    return;
  }
#pragma omp parallel for schedule(static) num_threads(nthreads_or_default(nthreads))
  for (int64_t i = 0; i < T; ++i) {
    int64_t slot = slots[i];
    /* padding (negative) and slots outside the pool write nothing */
    if (slot < 0 || slot >= p->num_blocks * p->block_size) continue;
    int64_t blk = slot / p->block_size;
    int32_t off = (int32_t)(slot % p->block_size);
    for (int32_t kh = 0; kh < Hkv; ++kh) {
      const float ks = (float)k_scale_of(p, kh), vs = (float)v_scale_of(p, kh);
      for (int32_t d = 0; d < D; ++d) {
        int64_t src = ((int64_t)i * Hkv + kh) * D + d;
        int64_t dst = elem_offset(p, blk, off, kh, d);
        if (p->elem_bytes == 2) {
          memcpy((uint8_t*)p->k + dst, &k_new[src], 2);
          memcpy((uint8_t*)p->v + dst, &v_new[src], 2);
        } else {
          float kx = (float)orc_f16_value(k_new[src]);
          float vx = (float)orc_f16_value(v_new[src]);
          if (p->fp8_format == ORC_FP8_E5M2) {
            ((uint8_t*)p->k)[dst] = orc_e5m2_encode(kx / ks);
            ((uint8_t*)p->v)[dst] = orc_e5m2_encode(vx / vs);
          } else {
            ((uint8_t*)p->k)[dst] = orc_e4m3fn_encode(kx / ks);
            ((uint8_t*)p->v)[dst] = orc_e4m3fn_encode(vx / vs);
          }
        }
      }
    }
  }
}

void orc_copy_blocks(const orc_pool* p, const int64_t* pairs, int64_t n) {
  const int64_t stride = block_stride_of(p);
  const int64_t bytes = (int64_t)p->block_size * p->num_kv_heads * p->head_dim * p->elem_bytes;
  for (int64_t i = 0; i < n; ++i) {
    int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || src >= p->num_blocks || dst < 0 || dst >= p->num_blocks) continue;
    memmove((uint8_t*)p->k + dst * stride, (const uint8_t*)p->k + src * stride, (size_t)bytes);
    memmove((uint8_t*)p->v + dst * stride, (const uint8_t*)p->v + src * stride, (size_t)bytes);
    if (p->k_block_scales) {
      const int32_t H = p->num_kv_heads;
      memmove(p->k_block_scales + dst * H, p->k_block_scales + src * H, (size_t)H * sizeof(float));
      memmove(p->v_block_scales + dst * H, p->v_block_scales + src * H, (size_t)H * sizeof(float));
    }
  }
}

/* ------------------------------------------------------------------ reads */

void orc_gather_head(const orc_pool* p, const int32_t* bt_row, int32_t len, int32_t kh,
                     double* Kc, double* Vc) {
  const int32_t D = p->head_dim;
  for (int32_t t = 0; t < len; ++t) {
    int64_t blk = bt_row[t / p->block_size];
    int32_t off = t % p->block_size;
    /* the row's dequantisation scales: per block when the pool keeps them */
    const double ks = p->k_block_scales && p->elem_bytes == 1
                          ? (double)p->k_block_scales[blk * p->num_kv_heads + kh]
                          : k_scale_of(p, kh);
    const double vs = p->v_block_scales && p->elem_bytes == 1
                          ? (double)p->v_block_scales[blk * p->num_kv_heads + kh]
                          : v_scale_of(p, kh);
    for (int32_t d = 0; d < D; ++d) {
      int64_t o = elem_offset(p, blk, off, kh, d);
      Kc[(int64_t)t * D + d] = read_elem(p, p->k, o, ks);
      Vc[(int64_t)t * D + d] = read_elem(p, p->v, o, vs);
    }
  }
}

void orc_attend(const double* q, const double* Kc, const double* Vc, int32_t len,
                int32_t D, double scale, double* out) {
  for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
  if (len <= 0) return;
  double* x = (double*)malloc(sizeof(double) * (size_t)len);
  double m = -INFINITY;
  for (int32_t t = 0; t < len; ++t) {
    double dot = 0.0;
    for (int32_t d = 0; d < D; ++d) dot += q[d] * Kc[(int64_t)t * D + d];
    x[t] = scale * dot;
    if (x[t] > m) m = x[t];
  }
  double denom = 0.0;
  for (int32_t t = 0; t < len; ++t) {
    double w = exp(x[t] - m);
    denom += w;
    for (int32_t d = 0; d < D; ++d) out[d] += w * Vc[(int64_t)t * D + d];
  }
  for (int32_t d = 0; d < D; ++d) out[d] /= denom;
  free(x);
}

/* First position a query sees when n positions (0 .. n - 1) precede and include it. */
static int32_t window_start(const orc_pool* p, int32_t n) {
  return (p->sliding_window > 0 && n > p->sliding_window) ? n - p->sliding_window : 0;
}

/* One (sequence, KV head) unit of work, evaluated for each of its query heads. */
typedef void (*head_fn)(const double* q, const double* Kc, const double* Vc, int32_t len,
                        int32_t D, double scale, int32_t psz, double* out);

static void attend_adapter(const double* q, const double* Kc, const double* Vc, int32_t len,
                           int32_t D, double scale, int32_t psz, double* out) {
  (void)psz;
  orc_attend(q, Kc, Vc, len, D, scale, out);
}

/* Partitioned evaluation: per partition, m_p = max score, l_p = sum exp(x - m_p),
 * o_p = sum exp(x - m_p) v / l_p; then M = max m_p and
 * out = sum_p exp(m_p - M) l_p o_p / sum_p exp(m_p - M) l_p. */
static void attend_split(const double* q, const double* Kc, const double* Vc, int32_t len,
                         int32_t D, double scale, int32_t psz, double* out) {
  for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
  if (len <= 0) return;
  int32_t np = (len + psz - 1) / psz;
  double* m = (double*)malloc(sizeof(double) * (size_t)np);
  double* l = (double*)malloc(sizeof(double) * (size_t)np);
  double* o = (double*)calloc((size_t)np * (size_t)D, sizeof(double));
  for (int32_t pi = 0; pi < np; ++pi) {
    int32_t t0 = pi * psz, t1 = t0 + psz < len ? t0 + psz : len;
    double mp = -INFINITY;
    for (int32_t t = t0; t < t1; ++t) {
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d) dot += q[d] * Kc[(int64_t)t * D + d];
      double xt = scale * dot;
      if (xt > mp) mp = xt;
    }
    double lp = 0.0;
    for (int32_t t = t0; t < t1; ++t) {
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d) dot += q[d] * Kc[(int64_t)t * D + d];
      double w = exp(scale * dot - mp);
      lp += w;
      for (int32_t d = 0; d < D; ++d) o[(int64_t)pi * D + d] += w * Vc[(int64_t)t * D + d];
    }
    for (int32_t d = 0; d < D; ++d) o[(int64_t)pi * D + d] /= lp;
    m[pi] = mp;
    l[pi] = lp;
  }
  double M = -INFINITY;
  for (int32_t pi = 0; pi < np; ++pi)
    if (m[pi] > M) M = m[pi];
  double W = 0.0;
  for (int32_t pi = 0; pi < np; ++pi) {
    double w = exp(m[pi] - M) * l[pi];
    W += w;
    for (int32_t d = 0; d < D; ++d) out[d] += w * o[(int64_t)pi * D + d];
  }
  for (int32_t d = 0; d < D; ++d) out[d] /= W;
  free(m);
  free(l);
  free(o);
}

static void decode_units(const orc_pool* p, const uint16_t* qbits, int32_t S, int32_t Hq,
                         const int32_t* bt, int32_t max_blocks, const int32_t* lens,
                         float scale, int32_t psz, const int32_t* units, int64_t n_units,
                         double* out, int nthreads, head_fn fn) {
  const int32_t Hkv = p->num_kv_heads, D = p->head_dim, g = Hq / Hkv;
  const int64_t total = units ? n_units : (int64_t)S * Hkv;
  const double sc = (double)scale;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads_or_default(nthreads))
  for (int64_t u = 0; u < total; ++u) {
    int32_t s = units ? units[2 * u] : (int32_t)(u / Hkv);
    int32_t kh = units ? units[2 * u + 1] : (int32_t)(u % Hkv);
    int32_t len = lens[s];
    size_t rows = (size_t)(len > 0 ? len : 1) * (size_t)D;
    double* Kc = (double*)malloc(sizeof(double) * rows);
    double* Vc = (double*)malloc(sizeof(double) * rows);
    double* qd = (double*)malloc(sizeof(double) * (size_t)D);
    orc_gather_head(p, bt + (int64_t)s * max_blocks, len, kh, Kc, Vc);
    /* the query (position len - 1) sees the last sliding_window positions */
    const int32_t w0 = window_start(p, len);
    for (int32_t h = kh * g; h < (kh + 1) * g; ++h) {
      const uint16_t* qh = qbits + ((int64_t)s * Hq + h) * D;
      for (int32_t d = 0; d < D; ++d) qd[d] = orc_f16_value(qh[d]);
      fn(qd, Kc + (int64_t)w0 * D, Vc + (int64_t)w0 * D, len - w0, D, sc, psz,
         out + ((int64_t)s * Hq + h) * D);
    }
    free(Kc);
    free(Vc);
    free(qd);
  }
}

void orc_decode(const orc_pool* p, const uint16_t* q, int32_t S, int32_t Hq,
                const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                float scale, const int32_t* units, int64_t n_units, double* out, int nthreads) {
  decode_units(p, q, S, Hq, block_tables, max_blocks, seq_lens, scale, 0, units, n_units, out,
               nthreads, attend_adapter);
}

void orc_decode_split(const orc_pool* p, const uint16_t* q, int32_t S, int32_t Hq,
                      const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                      float scale, int32_t partition_size, const int32_t* units,
                      int64_t n_units, double* out, int nthreads) {
  decode_units(p, q, S, Hq, block_tables, max_blocks, seq_lens, scale, partition_size, units,
               n_units, out, nthreads, attend_split);
}

/* ---------------------------------------------------------------- prefill */

void orc_prefill(const orc_pool* p, const uint16_t* qbits, const int32_t* q_start, int32_t S,
                 int32_t Hq, const int32_t* bt, int32_t max_blocks, const int32_t* lens,
                 float scale, const int32_t* rows, int64_t n_rows, double* out, int nthreads) {
  const int32_t Hkv = p->num_kv_heads, D = p->head_dim, g = Hq / Hkv;
  const double sc = (double)scale;
  /* with rows == NULL, enumerate (s, kh, i) in order */
  int64_t total = n_rows;
  int32_t* all = NULL;
  if (!rows) {
    total = 0;
    for (int32_t s = 0; s < S; ++s) total += (int64_t)(q_start[s + 1] - q_start[s]) * Hkv;
    all = (int32_t*)malloc(sizeof(int32_t) * 3 * (size_t)(total > 0 ? total : 1));
    int64_t u = 0;
    for (int32_t s = 0; s < S; ++s)
      for (int32_t kh = 0; kh < Hkv; ++kh)
        for (int32_t i = 0; i < q_start[s + 1] - q_start[s]; ++i) {
          all[3 * u] = s;
          all[3 * u + 1] = kh;
          all[3 * u + 2] = i;
          ++u;
        }
    rows = all;
  }
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads_or_default(nthreads))
  for (int64_t u = 0; u < total; ++u) {
    const int32_t s = rows[3 * u], kh = rows[3 * u + 1], i = rows[3 * u + 2];
    const int32_t q_len = q_start[s + 1] - q_start[s];
    const int32_t pos = lens[s] - q_len + i;      /* this query's position */
    const int32_t n = pos + 1;                    /* keys it sees: 0..pos */
    double* Kc = (double*)malloc(sizeof(double) * (size_t)n * (size_t)D);
    double* Vc = (double*)malloc(sizeof(double) * (size_t)n * (size_t)D);
    double* qd = (double*)malloc(sizeof(double) * (size_t)D);
    orc_gather_head(p, bt + (int64_t)s * max_blocks, n, kh, Kc, Vc);
    const int64_t row = (int64_t)q_start[s] + i;
    const int32_t w0 = window_start(p, n);
    for (int32_t h = kh * g; h < (kh + 1) * g; ++h) {
      const uint16_t* qh = qbits + (row * Hq + h) * D;
      for (int32_t d = 0; d < D; ++d) qd[d] = orc_f16_value(qh[d]);
      orc_attend(qd, Kc + (int64_t)w0 * D, Vc + (int64_t)w0 * D, n - w0, D, sc,
                 out + (row * Hq + h) * D);
    }
    free(Kc);
    free(Vc);
    free(qd);
  }
  free(all);
}
