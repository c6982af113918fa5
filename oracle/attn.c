/*
 * Oracle for the paged decode path: append, whole-block copy and decode
 * attention in plain C, float64 arithmetic.
 *
 * TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py load this library.  It shares no code, header
 * or table with the HIP library: the pool layout below is restated here from
 * its definition, not included.
 *
 * What it computes:
 *
 *  - Attention of one decode step: the new token's query is dotted with the
 *    key of every cached token, scaled by 1/sqrt(d_h), passed through a
 *    softmax over all of the sequence's tokens, and the weights average the
 *    cached values [KV Cache 与 PagedAttention, "注意力机制的计算";
 *    PagedAttention：大模型KV Cache内存管理革新 §3.2 (its per-page softmax
 *    is not followed: the softmax spans the whole context)].  The step attends
 *    over the 1 x i row of step i [KV Cache 工程学 §15.1].
 *  - Paging only changes where a token's K/V live: token j of a sequence
 *    sits in slot j % 16 of the physical block named by entry j / 16 of the
 *    sequence's block table [KV Cache 工程学 §15.5; 新一代 KV Cache 管理
 *    §8.1].  The result therefore equals attention over the contiguous
 *    per-sequence cache [KV Cache 工程学 §15.2].
 *  - Grouped-query heads: query head h reads kv head h / (h_q / h_kv)
 *    (contiguous groups; the pages only say h_kv < h_q [§15.2, §15.7]).
 *
 * Pool layout (a choice of this build; the pages only say "flat pool"):
 *    X = 16 / element size (8 for bf16, 4 for f32)
 *    K element (blk, g, t, d) at (((blk*Hkv + g)*(D/X) + d/X)*16 + t)*X + d%X
 *    V element (blk, g, t, d) at  ((blk*Hkv + g)*D + d)*16 + t
 *
 * Element types: 0 = float32, 1 = bfloat16 (raw uint16 bits), 2 = int8 with
 * a float32 scale per (token, kv head) [KV Cache 工程学 §15.7 "KV Cache 量化":
 * FP16 -> INT8 halves the cache], 3 = FP8 E4M3 with the same scales (the
 * other one-byte format the section names).  Every element is widened
 * exactly to double before use; an int8 or FP8 element stands for
 * value(code) * scale.
 *
 * int8 pools (a choice of this build): a (block, kv head) tile is
 * 16 * D int8 codes followed by 16 float32 scales (one per token slot),
 * 16 * D + 64 bytes:
 *    K code (blk, g, t, d) at byte ((blk*Hkv + g)*TB + ((d/16)*16 + p(t))*16 + d%16)
 *    where p(t) exchanges bits 2 and 3 of t (slots 0-3, 8-11, 4-7, 12-15 in
 *    that order along each 256-byte row of 16-byte units)
 *    V code (blk, g, t, d) at byte ((blk*Hkv + g)*TB + d*16 + t)
 *    scale of slot t at byte ((blk*Hkv + g)*TB + 16*D + 4*t), in each pool
 * Queries and the rows handed to append are bfloat16.  Quantisation of a
 * token's row x[0..D) of one kv head, in float32 as the kernels do it:
 *    amax = max |x_d|, scale = amax / 127, code_d = rint(x_d / scale)
 *    clamped to [-127, 127] (round half to even; all zero when amax = 0).
 * FP8 pools have the same tiles; the codes are FP8 E4M3 as the OCP 8-bit
 * floating point format defines it (sign, 4 exponent bits with bias 7, 3
 * mantissa bits; exponent 0 holds the subnormals m/8 * 2^-6; no
 * infinities; 448 is the largest finite value, S.1111.111 is NaN):
 *    amax = max |x_d|, scale = amax / 448, code_d = the E4M3 value nearest to
 *    x_d / scale (ties to the even mantissa), saturated at 448, the sign kept
 *    (so -0 codes as 0x80); all zero when amax = 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define BLOCK 16

static double elem(const void *base, size_t i, int dtype) {
  if (dtype == 0) return (double)((const float *)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static size_t esize(int dtype) { return dtype == 0 ? 4 : dtype == 1 ? 2 : 1; }

/* One-byte codes with a float32 scale per (token, kv head): int8 or FP8. */
static int is_q8(int dtype) { return dtype == 2 || dtype == 3; }

/* Element type of queries and of the rows given to append. */
static int row_type(int dtype) { return is_q8(dtype) ? 1 : dtype; }

/* Value of an FP8 E4M3 code (the OCP definition). */
static double e4m3_value(unsigned char c) {
  int e = (c >> 3) & 15, m = c & 7;
  double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);
  return (c & 0x80) ? -v : v;
}

/* The E4M3 code of the value nearest to y (ties to the even mantissa),
 * saturated at 448; y is finite. */
static unsigned char e4m3_code(float y) {
  unsigned char s = signbit(y) ? 0x80 : 0;
  double a = fabs((double)y);
  if (a >= 448.0) return s | 0x7E;
  if (a < ldexp(1.0, -6)) return s | (unsigned char)nearbyint(a * 512.0); /* multiples of 2^-9; 8 is 2^-6 */
  int e;
  double f = frexp(a, &e); /* a = (2f) * 2^(e-1), 2f in [1, 2) */
  double q = nearbyint((2.0 * f - 1.0) * 8.0);
  int E = e - 1 + 7;
  if (q == 8.0) {
    q = 0.0;
    E += 1;
  }
  return s | (unsigned char)(E << 3) | (unsigned char)q;
}

/* Bytes of one (block, kv head) tile of an int8 pool. */
static size_t tile_bytes_i8(int D) { return (size_t)16 * D + 64; }

/* Place of token slot t among the 16-byte units of a row of a one-byte K
 * tile: t with its bits 2 and 3 exchanged. */
static size_t k8_pos(int t) { return (size_t)((t & 3) | ((t & 4) << 1) | ((t & 8) >> 1)); }

static size_t k_at(int64_t blk, int g, int t, int d, int Hkv, int D, int dtype) {
  int X = (int)(16 / esize(dtype));
  return ((((size_t)blk * Hkv + g) * (size_t)(D / X) + (size_t)(d / X)) * BLOCK + (size_t)t) * X + (size_t)(d % X);
}

static size_t v_at(int64_t blk, int g, int t, int d, int Hkv, int D) {
  return (((size_t)blk * Hkv + g) * (size_t)D + (size_t)d) * BLOCK + (size_t)t;
}

/* Value of the int8 or FP8 code of K or V element (blk, g, t, d) times the
 * scale of slot t. */
static double i8_value(const void *pool, int64_t blk, int g, int t, int d, int Hkv, int D, int is_v, int dtype) {
  const unsigned char *tile = (const unsigned char *)pool + ((size_t)blk * Hkv + g) * tile_bytes_i8(D);
  size_t at = is_v ? (size_t)d * BLOCK + t : ((size_t)(d / 16) * BLOCK + k8_pos(t)) * 16 + d % 16;
  float sc;
  memcpy(&sc, tile + (size_t)16 * D + 4 * (size_t)t, sizeof sc);
  double v = dtype == 3 ? e4m3_value(tile[at]) : (double)(signed char)tile[at];
  return v * (double)sc;
}

/* Value of K element (blk, g, t, d) of a pool, widened to double. */
static double kval(const void *pool, int64_t blk, int g, int t, int d, int Hkv, int D, int dtype) {
  if (is_q8(dtype)) return i8_value(pool, blk, g, t, d, Hkv, D, 0, dtype);
  return elem(pool, k_at(blk, g, t, d, Hkv, D, dtype), dtype);
}
static double vval(const void *pool, int64_t blk, int g, int t, int d, int Hkv, int D, int dtype) {
  if (is_q8(dtype)) return i8_value(pool, blk, g, t, d, Hkv, D, 1, dtype);
  return elem(pool, v_at(blk, g, t, d, Hkv, D), dtype);
}

/* Quantise one row x[0..D) (bfloat16) into int8 or FP8 codes at code(d) and
 * its scale, in float32. */
static void quantise_row(const uint16_t *x, int D, unsigned char *tile, int t, int is_v, int dtype) {
  float amax = 0.0f;
  for (int d = 0; d < D; ++d) {
    float v = (float)elem(x, (size_t)d, 1);
    float a = fabsf(v);
    if (a > amax) amax = a;
  }
  float scale = amax / (dtype == 3 ? 448.0f : 127.0f);
  for (int d = 0; d < D; ++d) {
    float v = (float)elem(x, (size_t)d, 1);
    unsigned char code = 0;
    if (amax > 0.0f && dtype == 3) {
      code = e4m3_code(v / scale);
    } else if (amax > 0.0f) {
      float r = rintf(v / scale);
      int q = r > 127.0f ? 127 : r < -127.0f ? -127 : (int)r;
      code = (unsigned char)(signed char)q;
    }
    size_t at = is_v ? (size_t)d * BLOCK + t : ((size_t)(d / 16) * BLOCK + k8_pos(t)) * 16 + d % 16;
    tile[at] = code;
  }
  memcpy(tile + (size_t)16 * D + 4 * (size_t)t, &scale, sizeof scale);
}

static void copy_elem(void *dst, size_t di, const void *src, size_t si, int dtype) {
  size_t s = esize(dtype);
  memcpy((char *)dst + di * s, (const char *)src + si * s, s);
}

/* Write token t's K and V (rows of k_new/v_new [T][Hkv][D]) into slot
 * slots[t] = block*16 + offset.  Negative slots are skipped.  Bits are
 * copied unchanged. */
void orc_append(int dtype, int Hkv, int D, void *kpool, void *vpool, const void *k_new,
                const void *v_new, const int64_t *slots, int64_t T) {
  for (int64_t t = 0; t < T; ++t) {
    int64_t s = slots[t];
    if (s < 0) continue;
    int64_t blk = s / BLOCK;
    int off = (int)(s % BLOCK);
    if (is_q8(dtype)) {
      for (int g = 0; g < Hkv; ++g) {
        size_t row = ((size_t)t * Hkv + g) * D;
        size_t tile = ((size_t)blk * Hkv + g) * tile_bytes_i8(D);
        quantise_row((const uint16_t *)k_new + row, D, (unsigned char *)kpool + tile, off, 0, dtype);
        quantise_row((const uint16_t *)v_new + row, D, (unsigned char *)vpool + tile, off, 1, dtype);
      }
      continue;
    }
    for (int g = 0; g < Hkv; ++g)
      for (int d = 0; d < D; ++d) {
        size_t src = ((size_t)t * Hkv + g) * D + d;
        copy_elem(kpool, k_at(blk, g, off, d, Hkv, D, dtype), k_new, src, dtype);
        copy_elem(vpool, v_at(blk, g, off, d, Hkv, D), v_new, src, dtype);
      }
  }
}

/* Copy-on-write support: copy every slot, head and element of block
 * pairs[2i] into block pairs[2i+1], for K and V. */
void orc_copy_blocks(int dtype, int Hkv, int D, void *kpool, void *vpool, const int32_t *pairs,
                     int n) {
  for (int i = 0; i < n; ++i) {
    int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (is_q8(dtype)) {
      size_t tb = (size_t)Hkv * tile_bytes_i8(D);
      memcpy((char *)kpool + dst * tb, (const char *)kpool + src * tb, tb);
      memcpy((char *)vpool + dst * tb, (const char *)vpool + src * tb, tb);
      continue;
    }
    for (int g = 0; g < Hkv; ++g)
      for (int t = 0; t < BLOCK; ++t)
        for (int d = 0; d < D; ++d) {
          copy_elem(kpool, k_at(dst, g, t, d, Hkv, D, dtype), kpool, k_at(src, g, t, d, Hkv, D, dtype), dtype);
          copy_elem(vpool, v_at(dst, g, t, d, Hkv, D), vpool, v_at(src, g, t, d, Hkv, D), dtype);
        }
  }
}

/* Decode attention over the paged pool.  q [B][Hq][D], tables [B][max_blocks],
 * ctx [B], out [B][Hq][D] (double).  A sequence with ctx 0 gets output 0. */
void orc_paged_attention(int dtype, int Hq, int Hkv, int D, const void *q, const void *kpool,
                         const void *vpool, const int32_t *tables, int max_blocks,
                         const int32_t *ctx, int B, double scale, double *out) {
  int G = Hq / Hkv, qt = row_type(dtype);
#pragma omp parallel for schedule(dynamic)
  for (int64_t bh = 0; bh < (int64_t)B * Hq; ++bh) {
    int b = (int)(bh / Hq), h = (int)(bh % Hq), g = h / G;
    int n = ctx[b];
    double *o = out + (size_t)bh * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (n <= 0) continue;
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
      int64_t blk = tables[(size_t)b * max_blocks + j / BLOCK];
      double acc = 0.0;
      for (int d = 0; d < D; ++d)
        acc += elem(q, (size_t)bh * D + d, qt) * kval(kpool, blk, g, j % BLOCK, d, Hkv, D, dtype);
      s[j] = scale * acc;
      if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int j = 0; j < n; ++j) {
      int64_t blk = tables[(size_t)b * max_blocks + j / BLOCK];
      double w = exp(s[j] - m);
      l += w;
      for (int d = 0; d < D; ++d) o[d] += w * vval(vpool, blk, g, j % BLOCK, d, Hkv, D, dtype);
    }
    for (int d = 0; d < D; ++d) o[d] /= l;
    free(s);
  }
}

/* The same attention for one sequence whose cache is contiguous:
 * q [Hq][D], k and v [n][Hkv][D], out [Hq][D]. */
void orc_contiguous_attention(int dtype, int Hq, int Hkv, int D, const void *q, const void *k,
                              const void *v, int n, double scale, double *out) {
  int G = Hq / Hkv;
  for (int h = 0; h < Hq; ++h) {
    int g = h / G;
    double *o = out + (size_t)h * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (n <= 0) continue;
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
      double acc = 0.0;
      for (int d = 0; d < D; ++d)
        acc += elem(q, (size_t)h * D + d, dtype) * elem(k, ((size_t)j * Hkv + g) * D + d, dtype);
      s[j] = scale * acc;
      if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int j = 0; j < n; ++j) {
      double w = exp(s[j] - m);
      l += w;
      for (int d = 0; d < D; ++d) o[d] += w * elem(v, ((size_t)j * Hkv + g) * D + d, dtype);
    }
    for (int d = 0; d < D; ++d) o[d] /= l;
    free(s);
  }
}

/* Split-context form: the context is cut into spans of P tokens; each span
 * keeps its own maximum m_i, weight sum l_i and unnormalised output o_i, and
 * the spans are combined with M = max m_i, L = sum l_i e^(m_i - M),
 * O = sum o_i e^(m_i - M) / L.  Algebraically equal to orc_paged_attention. */
void orc_partitioned_attention(int dtype, int Hq, int Hkv, int D, const void *q,
                               const void *kpool, const void *vpool, const int32_t *tables,
                               int max_blocks, const int32_t *ctx, int B, double scale, int P,
                               double *out) {
  int G = Hq / Hkv, qt = row_type(dtype);
#pragma omp parallel for schedule(dynamic)
  for (int64_t bh = 0; bh < (int64_t)B * Hq; ++bh) {
    int b = (int)(bh / Hq), h = (int)(bh % Hq), g = h / G;
    int n = ctx[b];
    double *o = out + (size_t)bh * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (n <= 0) continue;
    int np = (n + P - 1) / P;
    double *pm = (double *)malloc(sizeof(double) * (size_t)np);
    double *pl = (double *)malloc(sizeof(double) * (size_t)np);
    double *po = (double *)calloc((size_t)np * D, sizeof(double));
    for (int p = 0; p < np; ++p) {
      int j0 = p * P, j1 = j0 + P < n ? j0 + P : n;
      double m = -INFINITY;
      for (int j = j0; j < j1; ++j) {
        int64_t blk = tables[(size_t)b * max_blocks + j / BLOCK];
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
          acc += elem(q, (size_t)bh * D + d, qt) * kval(kpool, blk, g, j % BLOCK, d, Hkv, D, dtype);
        if (scale * acc > m) m = scale * acc;
      }
      double l = 0.0;
      for (int j = j0; j < j1; ++j) {
        int64_t blk = tables[(size_t)b * max_blocks + j / BLOCK];
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
          acc += elem(q, (size_t)bh * D + d, qt) * kval(kpool, blk, g, j % BLOCK, d, Hkv, D, dtype);
        double w = exp(scale * acc - m);
        l += w;
        for (int d = 0; d < D; ++d) po[(size_t)p * D + d] += w * vval(vpool, blk, g, j % BLOCK, d, Hkv, D, dtype);
      }
      pm[p] = m;
      pl[p] = l;
    }
    double M = -INFINITY;
    for (int p = 0; p < np; ++p) if (pm[p] > M) M = pm[p];
    double L = 0.0;
    for (int p = 0; p < np; ++p) L += pl[p] * exp(pm[p] - M);
    for (int p = 0; p < np; ++p) {
      double f = exp(pm[p] - M);
      for (int d = 0; d < D; ++d) o[d] += po[(size_t)p * D + d] * f;
    }
    for (int d = 0; d < D; ++d) o[d] /= L;
    free(pm);
    free(pl);
    free(po);
  }
}

/* Read back the K or V of token j of a paged sequence into row-major
 * [Hkv][D] doubles (used to check that reads through different tables agree). */
/* Causal prefill over a paged cache [KV Cache 工程学 §15.1: a prompt of i
 * tokens is an i x i causal attention; §15.6 and 新一代 KV Cache 管理 §8.3:
 * the tokens of a cached prefix are not recomputed].  Sequence b holds
 * ctx[b] tokens in its table, the last nq_b = qstart[b+1] - qstart[b] of them
 * new; their K/V are already stored.  New token t (query row qstart[b] + t)
 * sits at position p_b + t with p_b = ctx[b] - nq_b and attends to positions
 * 0 .. p_b + t.  q: [T][Hq][D] (T = qstart[B]) of the row type; out:
 * [T][Hq][D] double. */
void orc_paged_prefill(int dtype, int Hq, int Hkv, int D, const void *q, const void *kpool,
                       const void *vpool, const int32_t *tables, int max_blocks, const int32_t *ctx,
                       const int32_t *qstart, int B, double scale, double *out) {
  int G = Hq / Hkv, qt = row_type(dtype);
  int64_t T = qstart[B];
#pragma omp parallel for schedule(dynamic)
  for (int64_t rh = 0; rh < T * Hq; ++rh) {
    int64_t r = rh / Hq;
    int h = (int)(rh % Hq), g = h / G;
    int b = 0;
    while (qstart[b + 1] <= r) ++b;
    int nq = qstart[b + 1] - qstart[b];
    int t = (int)(r - qstart[b]);
    int n = ctx[b] - nq + t + 1; /* keys 0 .. p_b + t */
    double *o = out + (size_t)rh * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
      int64_t blk = tables[(size_t)b * max_blocks + j / BLOCK];
      double acc = 0.0;
      for (int d = 0; d < D; ++d)
        acc += elem(q, (size_t)rh * D + d, qt) * kval(kpool, blk, g, j % BLOCK, d, Hkv, D, dtype);
      s[j] = scale * acc;
      if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int j = 0; j < n; ++j) {
      int64_t blk = tables[(size_t)b * max_blocks + j / BLOCK];
      double w = exp(s[j] - m);
      l += w;
      for (int d = 0; d < D; ++d) o[d] += w * vval(vpool, blk, g, j % BLOCK, d, Hkv, D, dtype);
    }
    for (int d = 0; d < D; ++d) o[d] /= l;
    free(s);
  }
}

void orc_gather_token(int dtype, int Hkv, int D, const void *kpool, const void *vpool,
                      const int32_t *table, int j, double *k_out, double *v_out) {
  int64_t blk = table[j / BLOCK];
  for (int g = 0; g < Hkv; ++g)
    for (int d = 0; d < D; ++d) {
      k_out[(size_t)g * D + d] = kval(kpool, blk, g, j % BLOCK, d, Hkv, D, dtype);
      v_out[(size_t)g * D + d] = vval(vpool, blk, g, j % BLOCK, d, Hkv, D, dtype);
    }
}

int orc_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
