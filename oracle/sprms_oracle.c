/*
 * sprms_oracle.c -- plain, slow, obviously-correct CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the CPU
 * baseline leg of the benchmark; never by the product path.  It shares no
 * code with the HIP implementation.  Built with gcc -O2 -ffp-contract=off so
 * every double operation is the one written here.
 *
 * What it computes, for one rank's shard (page tags as in sprms_oracle.h):
 *   1. the sum over the tp partial outputs, i.e. the reduction half of
 *      ReduceScatter -- an element-wise sum over ranks, after which each rank
 *      keeps its own contiguous block of tokens ([LongCat] o_proj K-axis TP;
 *      [SP/FC] §2.1-2.2);
 *   2. plus the rank's chunk of the deepstack embeddings when present
 *      ([SP/FC] §2.3: the deepstack add moves after the ReduceScatter and
 *      uses chunk [tp_rank]);
 *   3. plus the rank's chunk of the residual (maybe_chunk_residual,
 *      [SP/FC] §2.3); the sum is written back as the new residual (the fused
 *      add+norm op returns it);
 *   4. RMSNorm of that sum with weight and optional bias ([SP/FC] §2.3 and
 *      [SPquant] §1-§2: RMSNorm is per token);
 *   5. optional FP8 e4m3 output with a static per-tensor scale or a
 *      per-token scale max|y|/qmax ([SPquant] §4, quantisation table);
 *   6. zero on padding rows; their inputs are never read ([PR18671] §5.2,
 *      §5.3: padding rows of the shard are cleared).
 *
 * Readings where the pages leave a step open (each listed in the design
 * notes): eps inside the square root, mean over H; bias added after the
 * gain; deepstack added before the residual; the norm and quantiser use the
 * unrounded sum, not the stored residual; qmax = 448 (OCP e4m3fn);
 * an all-zero row in dynamic mode gets scale 0 and zero codes.
 *
 * NaN (the pages say nothing about it; inputs are normally finite): the
 * arithmetic is IEEE, so a NaN input element makes z NaN there, the row's
 * sum of squares and so every y of the row NaN; a NaN gain or bias element
 * makes y NaN in that column.  Every NaN reaches the output: bf16/f32 NaN,
 * the e4m3 NaN code 0x7F (never a saturated code), a NaN per-token scale
 * (the row maximum skips nothing) with every code of the row 0x7F, and the
 * E8M0 NaN byte 0xFF for a block holding a NaN.
 */
#include "sprms_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- formats */

/* bfloat16 is the upper half of an IEEE binary32: 1 sign bit, 8 exponent
 * bits (bias 127), 7 stored fraction bits, i.e. 8 significant bits. */
double orc_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Nearest bfloat16 value to x, ties to the even significand.  The spacing of
 * bfloat16 values in the binade [2^(k-1), 2^k) is 2^(k-8); below the
 * smallest normal 2^-126 it is the subnormal step 2^-133.  Dividing by a
 * power of two is exact, and rint() in the default rounding mode rounds to
 * the nearest integer with ties to even, so r*spacing is the correctly
 * rounded result (r = 256 simply lands on the next power of two).  A result
 * of 2^128 or more is an overflow: +-inf. */
uint16_t orc_bf16_from_double(double x) {
  if (isnan(x)) return 0x7FC0;
  double a = fabs(x);
  double r;
  if (a == 0.0) {
    r = 0.0;
  } else {
    double spacing;
    if (a < ldexp(1.0, -126)) {
      spacing = ldexp(1.0, -133);
    } else {
      int k;
      (void)frexp(a, &k); /* a = m * 2^k, 0.5 <= m < 1 */
      spacing = ldexp(1.0, k - 8);
    }
    r = rint(a / spacing) * spacing;
    if (r >= ldexp(1.0, 128)) r = INFINITY;
  }
  float f = (float)r; /* exact: r is a bfloat16 value */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  uint16_t bits = (uint16_t)(u >> 16);
  if (signbit(x)) bits |= 0x8000;
  return bits;
}

/* OCP FP8 E4M3 ("e4m3fn"): sign, 4 exponent bits with bias 7, 3 mantissa
 * bits.  Exponent field 0 holds subnormals m/8 * 2^-6; S.1111.111 is NaN and
 * there is no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448. */
double orc_e4m3_to_double(uint8_t code) {
  int s = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* Clamp to [-448, 448], then pick by exhaustive search the finite code whose
 * value is nearest to |x|; on an exact tie take the code with the even
 * mantissa (magnitude codes are monotone, so neighbours differ in the last
 * bit).  The sign bit follows the sign of x, zero included. */
uint8_t orc_e4m3_from_double(double x) {
  if (isnan(x)) return 0x7F;
  double a = fabs(x);
  if (a > 448.0) a = 448.0;
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double err = fabs(orc_e4m3_to_double((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(best | (signbit(x) ? 0x80 : 0x00));
}

/* OCP FP4 E2M1: sign, 2 exponent bits with bias 1, 1 mantissa bit.  Exponent
 * field 0 holds the subnormal m/2; no NaN, no infinity: magnitudes 0, 0.5, 1,
 * 1.5, 2, 3, 4, 6. */
double orc_e2m1_to_double(uint8_t code) {
  int s = (code >> 3) & 1;
  int e = (code >> 1) & 3;
  int m = code & 1;
  double v = e == 0 ? (double)m / 2.0 : ldexp(1.0 + (double)m / 2.0, e - 1);
  return s ? -v : v;
}

/* Clamp to [-6, 6], then the nearest of the 8 magnitudes by exhaustive search,
 * ties to the even mantissa; the sign bit follows the sign of x. */
uint8_t orc_e2m1_from_double(double x) {
  if (isnan(x)) return 0x7; /* no NaN code: saturate (never produced by the path) */
  double a = fabs(x);
  if (a > 6.0) a = 6.0;
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 7; ++c) {
    double err = fabs(orc_e2m1_to_double((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(best | (signbit(x) ? 0x8 : 0x0));
}

/* --------------------------------------------------------------- elements */

static size_t elt_size(int32_t dt) {
  switch (dt) {
    case ORC_F32: return 4;
    case ORC_BF16: return 2;
    case ORC_E4M3: return 1;
    default: return 0;  /* ORC_E2M1 rows are H/2 bytes: see row_bytes() */
  }
}

static double load(const void* base, int32_t dt, int64_t idx) {
  if (dt == ORC_F32) {
    float f;
    memcpy(&f, (const char*)base + 4 * idx, 4);
    return (double)f;
  }
  uint16_t b;
  memcpy(&b, (const char*)base + 2 * idx, 2);
  return orc_bf16_to_double(b);
}

/* Round once to the storage type (f32: C's conversion, which rounds to
 * nearest-even in the default mode; bf16: the definition above). */
static void store(void* base, int32_t dt, int64_t idx, double v) {
  if (dt == ORC_F32) {
    float f = (float)v;
    memcpy((char*)base + 4 * idx, &f, 4);
  } else if (dt == ORC_BF16) {
    uint16_t b = orc_bf16_from_double(v);
    memcpy((char*)base + 2 * idx, &b, 2);
  } else {
    ((uint8_t*)base)[idx] = orc_e4m3_from_double(v);
  }
}

static size_t row_bytes(int32_t dt, int64_t H) {
  return dt == ORC_E2M1 ? (size_t)H / 2 : (size_t)H * elt_size(dt);
}

/* -------------------------------------------------------------- geometry */

int orc_shard_geometry(int64_t num_tokens, int64_t num_tokens_pad, int32_t tp,
                       int32_t rank, int64_t* shard_rows, int64_t* local_start,
                       int64_t* valid_rows) {
  if (!shard_rows || !local_start || !valid_rows) return ORC_ERR_NULL;
  if (tp < 1 || rank < 0 || rank >= tp) return ORC_ERR_SHAPE;
  if (num_tokens < 0 || num_tokens_pad < 0 || num_tokens > num_tokens_pad) return ORC_ERR_SHAPE;
  if (num_tokens_pad % tp != 0) return ORC_ERR_SHAPE;
  int64_t S = num_tokens_pad / tp;
  int64_t start = (int64_t)rank * S;
  int64_t v = num_tokens - start;
  if (v > S) v = S;
  if (v < 0) v = 0;
  *shard_rows = S;
  *local_start = start;
  *valid_rows = v;
  return ORC_OK;
}

/* ------------------------------------------------------------ validation */

static int validate(const orc_problem* p, const void* partials, const void* residual,
                    const void* weight, int32_t quant_mode, const void* deepstack,
                    float static_scale, int64_t n_rows, const int64_t* rows,
                    const void* residual_out, const void* out, const void* out_scale) {
  if (!p) return ORC_ERR_NULL;
  if (p->tp < 1 || p->tp_rank < 0 || p->tp_rank >= p->tp) return ORC_ERR_SHAPE;
  if (p->shard_rows < 0 || p->hidden < 1 || p->num_tokens < 0) return ORC_ERR_SHAPE;
  if (!isfinite(p->partial_scale)) return ORC_ERR_SHAPE;
  if (p->num_tokens > (int64_t)p->tp * p->shard_rows) return ORC_ERR_SHAPE;
  int64_t S = p->shard_rows;
  if (p->residual_rows != S && p->residual_rows != (int64_t)p->tp * S) return ORC_ERR_SHAPE;
  if (deepstack == NULL) {
    if (p->deepstack_rows != 0) return ORC_ERR_SHAPE;
  } else if (p->deepstack_rows != S && p->deepstack_rows != (int64_t)p->tp * S) {
    return ORC_ERR_SHAPE;
  }
  if (p->partial_dtype != ORC_F32 && p->partial_dtype != ORC_BF16) return ORC_ERR_DTYPE;
  if (p->act_dtype != ORC_F32 && p->act_dtype != ORC_BF16) return ORC_ERR_DTYPE;
  if (quant_mode == ORC_QUANT_NONE) {
    if (p->out_dtype != ORC_F32 && p->out_dtype != ORC_BF16) return ORC_ERR_DTYPE;
  } else if (quant_mode == ORC_QUANT_STATIC_TENSOR || quant_mode == ORC_QUANT_DYNAMIC_TOKEN) {
    if (p->out_dtype != ORC_E4M3) return ORC_ERR_DTYPE;
  } else if (quant_mode == ORC_QUANT_MX_BLOCK) {
    if (p->out_dtype != ORC_E4M3 && p->out_dtype != ORC_E2M1) return ORC_ERR_DTYPE;
    if (p->hidden % 32 != 0) return ORC_ERR_SHAPE;
  } else {
    return ORC_ERR_UNSUPPORTED;
  }
  if (quant_mode == ORC_QUANT_STATIC_TENSOR && !(isfinite(static_scale) && static_scale > 0.0f))
    return ORC_ERR_SHAPE;
  if (n_rows < 0) return ORC_ERR_SHAPE;
  if (rows == NULL && n_rows != S) return ORC_ERR_SHAPE;
  if (n_rows > 0) {
    if (!partials || !residual || !weight || !residual_out || !out) return ORC_ERR_NULL;
    if ((quant_mode == ORC_QUANT_DYNAMIC_TOKEN || quant_mode == ORC_QUANT_MX_BLOCK) && !out_scale)
      return ORC_ERR_NULL;
  }
  if (rows)
    for (int64_t i = 0; i < n_rows; ++i)
      if (rows[i] < 0 || rows[i] >= S) return ORC_ERR_SHAPE;
  return ORC_OK;
}

/* ------------------------------------------------------------- the path */

int orc_reduce_add_rmsnorm(const orc_problem* p, const void* partials,
                           const void* residual, const void* weight,
                           const void* bias, float eps, int32_t quant_mode,
                           const void* deepstack, float static_scale,
                           int64_t n_rows, const int64_t* rows,
                           void* residual_out, void* out, void* out_scale,
                           double* z_dbg, double* y_dbg) {
  int rc = validate(p, partials, residual, weight, quant_mode, deepstack, static_scale,
                    n_rows, rows, residual_out, out, out_scale);
  if (rc != ORC_OK) return rc;

  const int64_t S = p->shard_rows;
  const int64_t H = p->hidden;
  const int64_t tp = p->tp;
  const int64_t r = p->tp_rank;

  /* valid rows of this shard ([PR18671] §5.2) */
  int64_t v = p->num_tokens - r * S;
  if (v > S) v = S;
  if (v < 0) v = 0;
  /* maybe_chunk_residual / chunk(deepstack)[tp_rank] ([SP/FC] §2.3): a tensor
   * holding every rank's rows contributes its block r; a shard-sized tensor
   * is used as it is. */
  const int64_t roff = (p->residual_rows == tp * S && tp > 1) ? r * S : 0;
  const int64_t doff = (deepstack && p->deepstack_rows == tp * S && tp > 1) ? r * S : 0;

  const size_t orow = row_bytes(p->out_dtype, H);
  const size_t az = elt_size(p->act_dtype);
  const int64_t nblk = H / 32;
  double* z = (double*)malloc((size_t)H * sizeof(double));
  double* y = (double*)malloc((size_t)H * sizeof(double));
  if (!z || !y) {
    free(z);
    free(y);
    return ORC_ERR_NULL;
  }

  for (int64_t i = 0; i < n_rows; ++i) {
    const int64_t s = rows ? rows[i] : i;
    if (s >= v) {
      /* padding row: every output is zero, no input is read */
      memset((char*)residual_out + (size_t)(i * H) * az, 0, (size_t)H * az);
      memset((char*)out + (size_t)i * orow, 0, orow);
      if (quant_mode == ORC_QUANT_DYNAMIC_TOKEN) ((float*)out_scale)[i] = 0.0f;
      if (quant_mode == ORC_QUANT_MX_BLOCK) memset((uint8_t*)out_scale + i * nblk, 0, (size_t)nblk);
      if (z_dbg) memset(z_dbg + i * H, 0, (size_t)H * sizeof(double));
      if (y_dbg) memset(y_dbg + i * H, 0, (size_t)H * sizeof(double));
      continue;
    }

    /* z = ((sum over ranks of the scaled partials) + deepstack) + residual; the
     * DSA-CP o_proj finalize multiplies each rank's output by a factor before
     * the reduction ([PR18671] §5.3) */
    for (int64_t h = 0; h < H; ++h) {
      double x = 0.0;
      for (int64_t q = 0; q < tp; ++q)
        x += p->partial_scale * load(partials, p->partial_dtype, (q * S + s) * H + h);
      if (deepstack) x += load(deepstack, p->act_dtype, (doff + s) * H + h);
      z[h] = x + load(residual, p->act_dtype, (roff + s) * H + h);
      store(residual_out, p->act_dtype, i * H + h, z[h]);
    }

    /* RMSNorm: mean of squares over H, eps inside the square root */
    double ss = 0.0;
    for (int64_t h = 0; h < H; ++h) ss += z[h] * z[h];
    const double rstd = 1.0 / sqrt(ss / (double)H + (double)eps);

    /* y = z * rstd * weight (+ bias) and its absolute maximum; a NaN
     * anywhere in y makes the maximum NaN (nothing is skipped) */
    double amax = 0.0;
    for (int64_t h = 0; h < H; ++h) {
      y[h] = z[h] * rstd * load(weight, p->act_dtype, h);
      if (bias) y[h] += load(bias, p->act_dtype, h);
      if (isnan(y[h]) || fabs(y[h]) > amax) amax = fabs(y[h]);
    }

    if (quant_mode == ORC_QUANT_NONE) {
      for (int64_t h = 0; h < H; ++h) store(out, p->out_dtype, i * H + h, y[h]);
    } else if (quant_mode == ORC_QUANT_STATIC_TENSOR) {
      /* codes encode y / scale, scale a calibrated per-tensor constant */
      for (int64_t h = 0; h < H; ++h) store(out, ORC_E4M3, i * H + h, y[h] / (double)static_scale);
    } else if (quant_mode == ORC_QUANT_DYNAMIC_TOKEN) {
      /* per-token scale = max|y| / qmax, qmax = 448; codes encode y / scale.
       * A zero row has scale 0 and zero codes; a row holding a NaN has a
       * NaN scale, so every code of it is the NaN code. */
      const float scale = (float)(amax / 448.0);
      ((float*)out_scale)[i] = scale;
      for (int64_t h = 0; h < H; ++h)
        store(out, ORC_E4M3, i * H + h, scale == 0.0f ? 0.0 : y[h] / (double)scale);
    } else {
      /* per-block scaling in the OCP microscaling form: for each block of 32
       * consecutive elements, X = 2^e with e = floor(log2(max|y|)) - emax
       * (emax = 8 for e4m3, 2 for e2m1; clamped to the E8M0 range [-127, 127];
       * an all-zero block takes -127), elements encode y / X with saturation,
       * the scale is stored as the E8M0 byte e + 127.  A block holding a NaN
       * takes the E8M0 NaN byte 0xFF, which makes the whole block NaN in that
       * format; its elements are then written as the e4m3 NaN code, or as 0
       * in e2m1, which has no NaN code. */
      const int emax = p->out_dtype == ORC_E4M3 ? 8 : 2;
      for (int64_t b = 0; b < nblk; ++b) {
        double bmax = 0.0;
        for (int64_t h = 32 * b; h < 32 * b + 32; ++h)
          if (isnan(y[h]) || fabs(y[h]) > bmax) bmax = fabs(y[h]);
        if (isnan(bmax)) {
          ((uint8_t*)out_scale)[i * nblk + b] = 0xFF;
          for (int64_t h = 32 * b; h < 32 * b + 32; ++h) {
            if (p->out_dtype == ORC_E4M3) {
              ((uint8_t*)out)[i * H + h] = 0x7F;
            } else {
              uint8_t* byte = (uint8_t*)out + (size_t)i * orow + (size_t)(h / 2);
              *byte = (h % 2 == 0) ? (uint8_t)(*byte & 0xF0) : (uint8_t)(*byte & 0x0F);
            }
          }
          continue;
        }
        int e = -127;
        if (bmax > 0.0) {
          int k;
          (void)frexp(bmax, &k); /* bmax = m * 2^k, 0.5 <= m < 1: floor(log2 bmax) = k - 1 */
          e = k - 1 - emax;
        }
        if (e < -127) e = -127;
        if (e > 127) e = 127;
        ((uint8_t*)out_scale)[i * nblk + b] = (uint8_t)(e + 127);
        for (int64_t h = 32 * b; h < 32 * b + 32; ++h) {
          const double t = ldexp(y[h], -e);
          if (p->out_dtype == ORC_E4M3) {
            ((uint8_t*)out)[i * H + h] = orc_e4m3_from_double(t);
          } else {
            uint8_t* byte = (uint8_t*)out + (size_t)i * orow + (size_t)(h / 2);
            const uint8_t c = orc_e2m1_from_double(t);
            *byte = (h % 2 == 0) ? (uint8_t)((*byte & 0xF0) | c) : (uint8_t)((*byte & 0x0F) | (c << 4));
          }
        }
      }
    }

    if (z_dbg) memcpy(z_dbg + i * H, z, (size_t)H * sizeof(double));
    if (y_dbg) memcpy(y_dbg + i * H, y, (size_t)H * sizeof(double));
  }
  free(z);
  free(y);
  return ORC_OK;
}

/* ------------------------------------------------------ array versions */

void orc_bf16_from_double_n(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_double(x[i]);
}

void orc_e4m3_from_double_n(const double* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_from_double(x[i]);
}

/* ------------------------------------------ the boundary's argument list */

/* [a, a+an) and [b, b+bn) share a byte; empty ranges share nothing */
static int spans_meet(const void* a, size_t an, const void* b, size_t bn) {
  if (!a || !b || an == 0 || bn == 0) return 0;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bn && b0 < a0 + an;
}

/* largest byte span the partials may cover: 2^47 bytes, beyond any device */
#define ORC_MAX_SPAN ((int64_t)1 << 47)

int sp_oracle_reduce_add_rmsnorm(const orc_abi_problem* a, const void* partials, void* residual,
                                 const void* weight, const void* bias, float eps, int quant_mode,
                                 const void* deepstack, void* out, void* out_scale, void* stream) {
  (void)stream;
  if (!a) return ORC_ERR_NULL;
  if (a->flags & ~1) return ORC_ERR_UNSUPPORTED;
  const orc_problem p = {a->tp, a->tp_rank, a->shard_rows, a->hidden, a->num_tokens,
                         a->partial_dtype, a->act_dtype, a->out_dtype, a->residual_rows,
                         a->deepstack_rows, a->partial_scale == 0.0f ? 1.0 : (double)a->partial_scale};
  const int64_t S = a->shard_rows, H = a->hidden, tp = a->tp;
  if (tp < 1 || S < 0 || H < 1) return ORC_ERR_SHAPE;
  if (S == 0) return ORC_OK;
  if (!residual || !out) return ORC_ERR_NULL;
  float static_scale = 1.0f;
  if (quant_mode == ORC_QUANT_STATIC_TENSOR) {
    if (!out_scale) return ORC_ERR_NULL;
    static_scale = ((const float*)out_scale)[0];
  }
  const int dyn = quant_mode == ORC_QUANT_DYNAMIC_TOKEN, blk = quant_mode == ORC_QUANT_MX_BLOCK;
  if ((dyn || blk) && !out_scale) return ORC_ERR_NULL;
  const size_t pe = elt_size(a->partial_dtype), az = elt_size(a->act_dtype);
  const size_t orow = row_bytes(a->out_dtype, H);
  if (!pe || !az || !orow) return ORC_ERR_DTYPE;
  const int64_t stride = a->partial_stride ? a->partial_stride : S * H;
  if (stride < S * H) return ORC_ERR_SHAPE;
  /* bytes from the first partial row to the end of the last: (tp-1)*stride
   * + S*H elements, which must neither overflow nor pass ORC_MAX_SPAN */
  int64_t span_elems, span_bytes;
  if (__builtin_mul_overflow(tp - 1, stride, &span_elems) ||
      __builtin_add_overflow(span_elems, S * H, &span_elems) ||
      __builtin_mul_overflow(span_elems, (int64_t)pe, &span_bytes) || span_bytes > ORC_MAX_SPAN)
    return ORC_ERR_SHAPE;

  /* The rows this call writes may share no byte with what it reads, nor
   * with each other: the residual rows updated in place (residual_out NULL,
   * or pointing at the block in use) only with the residual itself. */
  int64_t v = a->num_tokens - (int64_t)a->tp_rank * S;
  v = v < 0 ? 0 : (v > S ? S : v);
  const int64_t n = (a->flags & 1) ? v : S;  /* rows written */
  const int64_t roff = (a->residual_rows == tp * S && tp > 1) ? (int64_t)a->tp_rank * S : 0;
  const char* used = (const char*)residual + (size_t)(roff * H) * az;
  void* res_dst = a->residual_out ? a->residual_out : (void*)used;
  {
    const int in_place = res_dst == (const void*)used;
    const size_t row_az = (size_t)H * az;
    /* inputs; the static scale (one f32) is read, the other scales written */
    const void* in_p[6] = {partials, weight, bias, deepstack, residual, out_scale};
    const size_t in_n[6] = {(size_t)span_bytes, row_az, bias ? row_az : 0,
                            deepstack ? (size_t)a->deepstack_rows * row_az : 0,
                            (size_t)a->residual_rows * row_az,
                            quant_mode == ORC_QUANT_STATIC_TENSOR ? 4 : 0};
    const void* out_p[3] = {res_dst, out, out_scale};
    const size_t out_n[3] = {(size_t)n * row_az, (size_t)n * orow,
                             dyn ? (size_t)n * 4 : blk ? (size_t)n * (size_t)(H / 32) : 0};
    for (int o = 0; o < 3; ++o) {
      for (int k = 0; k < 6; ++k) {
        if (o == 0 && k == 4 && in_place) continue; /* the in-place update itself */
        if (spans_meet(out_p[o], out_n[o], in_p[k], in_n[k])) return ORC_ERR_SHAPE;
      }
      for (int o2 = o + 1; o2 < 3; ++o2)
        if (spans_meet(out_p[o], out_n[o], out_p[o2], out_n[o2])) return ORC_ERR_SHAPE;
    }
  }

  /* a strided set of partials is packed into [tp][S][H] first */
  void* packed = NULL;
  if (partials && stride != S * H) {
    packed = malloc((size_t)(tp * S * H) * pe);
    if (!packed) return ORC_ERR_NULL;
    for (int64_t q = 0; q < tp; ++q)
      memcpy((char*)packed + (size_t)(q * S * H) * pe, (const char*)partials + (size_t)(q * stride) * pe,
             (size_t)(S * H) * pe);
  }
  const size_t srow = blk ? (size_t)(H / 32) : 4;
  void* res_t = malloc((size_t)(S * H) * az);
  void* out_t = malloc((size_t)S * orow);
  void* sc_t = malloc((size_t)S * srow);
  int rc = ORC_ERR_NULL;
  if (res_t && out_t && sc_t)
    rc = orc_reduce_add_rmsnorm(&p, packed ? packed : partials, residual, weight, bias, eps,
                                quant_mode, deepstack, static_scale, S, NULL, res_t, out_t,
                                (dyn || blk) ? sc_t : NULL, NULL, NULL);
  if (rc == ORC_OK) {
    memcpy(res_dst, res_t, (size_t)(n * H) * az);
    memcpy(out, out_t, (size_t)n * orow);
    if (dyn || blk) memcpy(out_scale, sc_t, (size_t)n * srow);
  }
  free(packed);
  free(res_t);
  free(out_t);
  free(sc_t);
  return rc;
}

/* ------------------------------------------------------- all-gather + unpad */

/* AllGather followed by unpad ([SP/FC] §3.3: gather the shards along the
 * token dimension, then drop the padding rows): row t < T of the gathered
 * tensor is row t - q*S of shard q = t / S, and the same for the rows of the
 * scales.  Bytes are copied unchanged. */
int orc_all_gather_unpad(int32_t tp, int64_t S, int64_t row_bytes, int64_t T,
                         const void* const* shards, int64_t scale_row_bytes,
                         const void* const* scales, void* out, void* out_scale) {
  if (tp < 1 || S < 0 || row_bytes < 1 || T < 0 || T > (int64_t)tp * S) return ORC_ERR_SHAPE;
  if (scale_row_bytes < 0 || (scale_row_bytes > 0) != (scales != NULL)) return ORC_ERR_SHAPE;
  if (T > 0 && (!shards || !out)) return ORC_ERR_NULL;
  if (scales && !out_scale) return ORC_ERR_NULL;
  for (int64_t t = 0; t < T; ++t) {
    const int64_t q = t / S;
    const int64_t s = t - q * S;
    memcpy((char*)out + (size_t)(t * row_bytes), (const char*)shards[q] + (size_t)(s * row_bytes),
           (size_t)row_bytes);
    if (scales)
      memcpy((char*)out_scale + (size_t)(t * scale_row_bytes),
             (const char*)scales[q] + (size_t)(s * scale_row_bytes), (size_t)scale_row_bytes);
  }
  return ORC_OK;
}

void orc_e2m1_from_double_n(const double* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_from_double(x[i]);
}

/* -------------------------------------------------- FlashComm2 regrouping */

/* [SP/FC] §4.4: with odp = G / otp, destination position j of an ODP group
 * receives the token segments j, j + odp, j + 2*odp, ... (otp of them): for
 * G = 4, otp = 2 this is [[0, 2], [1, 3]].  ids is [odp][otp]. */
int orc_fc2_batch_ids(int32_t G, int32_t otp, int32_t* ids) {
  if (G < 2 || otp < 1 || otp >= G || G % otp != 0 || !ids) return ORC_ERR_SHAPE;
  const int odp = G / otp;
  for (int j = 0; j < odp; ++j)
    for (int k = 0; k < otp; ++k) ids[j * otp + k] = j + k * odp;
  return ORC_OK;
}

/* [SP/FC] §4.4, steps 1-3 written out: rank q holds features q of all N
 * tokens ([N][C], elt bytes each).  Each rank splits its tokens into G
 * segments and sends destination j of its ODP group (the odp consecutive
 * ranks g*odp .. g*odp+odp-1) the segments of batch ids row j; destination
 * r = g*odp + j concatenates what it receives along the features, in the
 * order of the senders: out[r] is [N/odp][odp*C]. */
int orc_fc2_regroup(int32_t G, int32_t otp, int64_t N, int64_t C, int32_t elt,
                    const void* const* src, void* const* dst) {
  if (G < 2 || otp < 1 || otp >= G || G % otp != 0 || N < 0 || N % G != 0 || C < 1)
    return ORC_ERR_SHAPE;
  if (N > 0 && (!src || !dst)) return ORC_ERR_NULL;
  const int odp = G / otp;
  const int64_t seg = N / G;
  int32_t ids[64 * 64];
  if (G > 64) return ORC_ERR_SHAPE;
  orc_fc2_batch_ids(G, otp, ids);
  const size_t piece = (size_t)C * (size_t)elt;
  for (int g = 0; g < G / odp; ++g)
    for (int j = 0; j < odp; ++j) {
      const int r = g * odp + j;
      int64_t t = 0; /* destination row */
      for (int k = 0; k < otp; ++k) {
        const int segment = ids[j * otp + k];
        for (int64_t u = 0; u < seg; ++u, ++t) {
          const int64_t n = segment * seg + u; /* source token */
          for (int i = 0; i < odp; ++i) {     /* sender i of the ODP group */
            const char* from = (const char*)src[g * odp + i] + (size_t)n * piece;
            char* to = (char*)dst[r] + (size_t)t * piece * odp + (size_t)i * piece;
            memcpy(to, from, piece);
          }
        }
      }
    }
  return ORC_OK;
}

/* ----------------------------------------- DSA-CP o_proj all-to-all (path B) */

/* [PR18671] §5.3, path B, the two steps before o_proj written out.  Rank p
 * holds attn[p], its S local tokens with every rank's heads, [S][tp*D].
 * Step 1 (view [S, tp, D], move the tp axis first, flatten): the send
 * buffer of rank p is [tp*S][D] with row q*S + s = columns [q*D, (q+1)*D)
 * of token s.  Step 2 (all_to_all_single over the tp group): the send
 * buffer is cut into tp equal chunks of S rows, chunk q goes to rank q, and
 * rank q stacks what it receives in sender order, so out[q] is [tp*S][D]
 * with row p*S + s from chunk q of rank p: every token of the group, rank
 * q's heads only.  piece = D * element bytes. */
int orc_dsacp_heads_to_tokens(int32_t tp, int64_t S, int64_t piece, const void* const* attn,
                              void* const* out) {
  if (tp < 1 || S < 0 || piece < 1) return ORC_ERR_SHAPE;
  if (S > 0 && (!attn || !out)) return ORC_ERR_NULL;
  if (S == 0) return ORC_OK;
  const size_t chunk = (size_t)S * (size_t)piece; /* S rows of one head block */
  char* send = (char*)malloc((size_t)tp * chunk);
  if (!send) return ORC_ERR_SHAPE;
  for (int p = 0; p < tp; ++p) {
    /* step 1 on rank p */
    for (int q = 0; q < tp; ++q)
      for (int64_t s = 0; s < S; ++s)
        memcpy(send + (size_t)q * chunk + (size_t)s * (size_t)piece,
               (const char*)attn[p] + ((size_t)s * (size_t)tp + (size_t)q) * (size_t)piece,
               (size_t)piece);
    /* step 2: rank p's chunk q lands in rank q's buffer at chunk position p */
    for (int q = 0; q < tp; ++q)
      memcpy((char*)out[q] + (size_t)p * chunk, send + (size_t)q * chunk, chunk);
  }
  free(send);
  return ORC_OK;
}

/* ------------------------------- row-parallel GEMM + scatter (the producer) */

/* [SPquant] §二, the GEMM + ReduceScatter at a block's exit, with o_proj
 * split along K over the tp ranks ([LongCat], o_proj TP K-axis split).
 * Rank q holds x_q [M][K] (its K-slice of the input for all M = tp*S
 * tokens) and w_q [N][K] (its K-slice of the weight, one row per output
 * column) and computes its unreduced partial P_q = x_q * w_q^T, [M][N].
 * The ReduceScatter along the tokens hands row block r (rows r*S .. r*S+S-1)
 * to rank r, which sums the tp blocks it receives; before that sum rank r
 * holds them as [tp][S][N], slot q coming from rank q.  This writes rank q's
 * share of those buffers: dst[r] slot q row s = P_q[r*S + s], each element
 * the dot product of bf16 inputs summed in fp64 (every product is exact)
 * and rounded once to out_dtype.  rows (n_rows entries, NULL = all M)
 * selects the token rows m computed; other rows of dst are not touched. */
int orc_matmul_scatter(int32_t tp, int32_t rank, int64_t S, int64_t K, int64_t N, int32_t out_dtype,
                       const uint16_t* x, const uint16_t* w, int64_t n_rows, const int64_t* rows,
                       void* const* dst) {
  if (tp < 1 || rank < 0 || rank >= tp || S < 0 || K < 1 || N < 1) return ORC_ERR_SHAPE;
  if (out_dtype != ORC_BF16 && out_dtype != ORC_F32) return ORC_ERR_DTYPE;
  const int64_t M = (int64_t)tp * S;
  const int64_t count = rows ? n_rows : M;
  if (count == 0) return ORC_OK;
  if (!x || !w || !dst) return ORC_ERR_NULL;
  for (int r = 0; r < tp; ++r)
    if (!dst[r]) return ORC_ERR_NULL;
  for (int64_t i = 0; i < count; ++i)
    if (rows && (rows[i] < 0 || rows[i] >= M)) return ORC_ERR_SHAPE;
  for (int64_t i = 0; i < count; ++i) {
    const int64_t m = rows ? rows[i] : i;
    const int64_t r = m / S;     /* destination rank of this token */
    const int64_t s = m - r * S; /* its row in that rank's shard */
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k)
        acc += orc_bf16_to_double(x[m * K + k]) * orc_bf16_to_double(w[n * K + k]);
      store(dst[r], out_dtype, ((int64_t)rank * S + s) * N + n, acc);
    }
  }
  return ORC_OK;
}

/* The FP8 form of the producer ([SPquant] §四: after SP the row-parallel
 * GEMM is an FP8 GEMM with its scales, fused with the ReduceScatter): x and
 * w hold OCP e4m3 codes; x_scale has 1 (per tensor) or M (per token) fp32
 * entries, w_scale 1 (per tensor) or N (per output column), and
 *   P[m][n] = (sum over k of dec(x[m][k]) * dec(w[n][k])) * x_scale[m] * w_scale[n]
 * with the dot product exact in fp64 (e4m3 products are exact) and one
 * rounding to out_dtype.  Scattered like orc_matmul_scatter. */
int orc_scaled_matmul_scatter(int32_t tp, int32_t rank, int64_t S, int64_t K, int64_t N,
                              int32_t out_dtype, const uint8_t* x, const float* x_scale,
                              int64_t x_scale_rows, const uint8_t* w, const float* w_scale,
                              int64_t w_scale_rows, int64_t n_rows, const int64_t* rows,
                              void* const* dst) {
  if (tp < 1 || rank < 0 || rank >= tp || S < 0 || K < 1 || N < 1) return ORC_ERR_SHAPE;
  if (out_dtype != ORC_BF16 && out_dtype != ORC_F32) return ORC_ERR_DTYPE;
  const int64_t M = (int64_t)tp * S;
  if (x_scale_rows != 1 && x_scale_rows != M) return ORC_ERR_SHAPE;
  if (w_scale_rows != 1 && w_scale_rows != N) return ORC_ERR_SHAPE;
  const int64_t count = rows ? n_rows : M;
  if (count == 0) return ORC_OK;
  if (!x || !w || !x_scale || !w_scale || !dst) return ORC_ERR_NULL;
  for (int r = 0; r < tp; ++r)
    if (!dst[r]) return ORC_ERR_NULL;
  for (int64_t i = 0; i < count; ++i)
    if (rows && (rows[i] < 0 || rows[i] >= M)) return ORC_ERR_SHAPE;
  for (int64_t i = 0; i < count; ++i) {
    const int64_t m = rows ? rows[i] : i;
    const int64_t r = m / S;     /* destination rank of this token */
    const int64_t s = m - r * S; /* its row in that rank's shard */
    const double sx = (double)x_scale[x_scale_rows == 1 ? 0 : m];
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k)
        acc += orc_e4m3_to_double(x[m * K + k]) * orc_e4m3_to_double(w[n * K + k]);
      const double sw = (double)w_scale[w_scale_rows == 1 ? 0 : n];
      store(dst[r], out_dtype, ((int64_t)rank * S + s) * N + n, acc * sx * sw);
    }
  }
  return ORC_OK;
}
