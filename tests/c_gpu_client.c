/* Plain-C GPU client of libsprms: compiled with gcc against include/sprms.h
 * and HIP's C runtime API only, no C++ and no Python.  It allocates device
 * buffers with hipMalloc, enqueues sp_reduce_add_rmsnorm on a stream it
 * creates, and checks the results against the oracle's
 * sp_oracle_reduce_add_rmsnorm handed the same arguments on host copies.
 * Test infrastructure: the oracle header is included here only.
 *
 * Bars (those of the parity tests): bf16 out within 1e-3 + 2^-7 |ref| of the
 * oracle's; updated bf16 residual within one bf16 step; e4m3 codes equal to
 * the oracle's on >= 99.9% of elements and within one e4m3 step on all;
 * per-token scales within 1e-5 relative; f32 residual within 4e-6. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "sprms.h"
#include "sprms_oracle.h"

#define HIPCHECK(x)                                                            \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(2);                                                                 \
    }                                                                          \
  } while (0)

static uint32_t g_rng = 0x12345u;
static float frand(void) { /* uniform in [-1, 1) */
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 17;
  g_rng ^= g_rng << 5;
  return (float)(g_rng >> 8) / 8388608.0f - 1.0f;
}
static uint16_t bf16_bits(float f) { /* inputs: any bf16 value will do, truncation */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static double e4m3_value(uint8_t c) { /* OCP e4m3fn */
  int e = (c >> 3) & 15, m = c & 7;
  double v = e == 0 ? m / 8.0 * ldexp(1.0, -6) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  return (c & 0x80) ? -v : v;
}
/* position of a code in value order, +0 and -0 both 0: neighbouring values
 * (one e4m3 step apart) differ by exactly 1 */
static int e4m3_ordinal(uint8_t c) { return (c & 0x80) ? -(int)(c & 0x7F) : (int)(c & 0x7F); }

static void* fill(size_t n, int dt, float scale) { /* n elements of SP_F32 or SP_BF16 */
  if (dt == SP_F32) {
    float* a = malloc(n * 4);
    for (size_t i = 0; i < n; ++i) a[i] = scale * frand();
    return a;
  }
  uint16_t* a = malloc(n * 2);
  for (size_t i = 0; i < n; ++i) a[i] = bf16_bits(scale * frand());
  return a;
}
static void* dev_copy(const void* h, size_t bytes) {
  void* d = NULL;
  if (!h) return NULL;
  HIPCHECK(hipMalloc(&d, bytes));
  HIPCHECK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  return d;
}
static void* host_back(const void* d, size_t bytes) {
  void* h = malloc(bytes);
  HIPCHECK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
  return h;
}

typedef struct {
  const char* name;
  int tp, rank, S, H, T, pdt, adt, quant, bias, deepstack, replicated, in_place;
  float static_scale;
} Case;

static int run(const Case* c, hipStream_t stream) {
  const int64_t S = c->S, H = c->H, tp = c->tp;
  const size_t pe = c->pdt == SP_F32 ? 4 : 2, ae = c->adt == SP_F32 ? 4 : 2;
  const int odt = c->quant == SP_QUANT_NONE ? SP_BF16 : SP_FP8_E4M3;
  const size_t oe = odt == SP_BF16 ? 2 : 1;
  const int64_t rrows = c->replicated ? tp * S : S;
  const int64_t v = c->T - (int64_t)c->rank * S < 0 ? 0 : (c->T - (int64_t)c->rank * S > S ? S : c->T - (int64_t)c->rank * S);

  void* hP = fill((size_t)(tp * S * H), c->pdt, 1.0f);
  void* hR = fill((size_t)(rrows * H), c->adt, 1.0f);
  void* hW = fill((size_t)H, c->adt, 0.2f);
  if (c->adt == SP_BF16) { /* gain around 1 */
    for (int64_t h = 0; h < H; ++h) ((uint16_t*)hW)[h] = bf16_bits(1.0f + 0.2f * frand());
  } else {
    for (int64_t h = 0; h < H; ++h) ((float*)hW)[h] = 1.0f + 0.2f * frand();
  }
  void* hB = c->bias ? fill((size_t)H, c->adt, 0.05f) : NULL;
  void* hD = c->deepstack ? fill((size_t)(tp * S * H), c->adt, 0.3f) : NULL;

  void* dP = dev_copy(hP, tp * S * H * pe);
  void* dR = dev_copy(hR, rrows * H * ae);
  void* dW = dev_copy(hW, H * ae);
  void* dB = dev_copy(hB, H * ae);
  void* dD = dev_copy(hD, tp * S * H * ae);
  void *dO = NULL, *dRO = NULL, *dSc = NULL;
  HIPCHECK(hipMalloc(&dO, S * H * oe));
  HIPCHECK(hipMemset(dO, 0xA5, S * H * oe));
  if (!c->in_place) {
    HIPCHECK(hipMalloc(&dRO, S * H * ae));
    HIPCHECK(hipMemset(dRO, 0xA5, S * H * ae));
  }
  float hStatic = c->static_scale;
  if (c->quant == SP_QUANT_STATIC_TENSOR) dSc = dev_copy(&hStatic, 4);
  if (c->quant == SP_QUANT_DYNAMIC_TOKEN) HIPCHECK(hipMalloc(&dSc, S * 4));

  sp_problem p;
  memset(&p, 0, sizeof p);
  p.tp = c->tp;
  p.tp_rank = c->rank;
  p.shard_rows = S;
  p.hidden = H;
  p.num_tokens = c->T;
  p.partial_dtype = c->pdt;
  p.act_dtype = c->adt;
  p.out_dtype = odt;
  p.residual_rows = rrows;
  p.deepstack_rows = c->deepstack ? tp * S : 0;
  p.residual_out = dRO;

  /* a rejected call first: nothing may be written */
  if (sp_reduce_add_rmsnorm(&p, dP, dR, dW, dB, 1e-6f, 3, dD, dO, dSc, stream) != SP_ERR_UNSUPPORTED) {
    fprintf(stderr, "%s: quant mode 3 not rejected\n", c->name);
    return 1;
  }
  HIPCHECK(hipStreamSynchronize(stream));
  uint8_t* untouched = host_back(dO, S * H * oe);
  for (int64_t i = 0; i < S * H * (int64_t)oe; ++i)
    if (untouched[i] != 0xA5) {
      fprintf(stderr, "%s: a rejected call wrote out\n", c->name);
      return 1;
    }
  free(untouched);

  int st = sp_reduce_add_rmsnorm(&p, dP, dR, dW, dB, 1e-6f, c->quant, dD, dO, dSc, stream);
  if (st != SP_OK) {
    fprintf(stderr, "%s: status %d: %s\n", c->name, st, sp_last_error());
    return 1;
  }
  HIPCHECK(hipStreamSynchronize(stream));
  void* gO = host_back(dO, S * H * oe);
  void* gR = c->in_place ? host_back(dR, rrows * H * ae) : host_back(dRO, S * H * ae);
  float* gS = c->quant == SP_QUANT_DYNAMIC_TOKEN ? host_back(dSc, S * 4) : NULL;

  /* the oracle, same arguments on host memory */
  orc_abi_problem q;
  memset(&q, 0, sizeof q);
  q.tp = c->tp;
  q.tp_rank = c->rank;
  q.shard_rows = S;
  q.hidden = H;
  q.num_tokens = c->T;
  q.partial_dtype = c->pdt;
  q.act_dtype = c->adt;
  q.out_dtype = odt;
  q.residual_rows = rrows;
  q.deepstack_rows = c->deepstack ? tp * S : 0;
  void* oR = malloc(rrows * H * ae);
  memcpy(oR, hR, rrows * H * ae);
  void* oRO = c->in_place ? NULL : malloc(S * H * ae);
  q.residual_out = oRO;
  void* oO = malloc(S * H * oe);
  float oS[4096];
  if (c->quant == SP_QUANT_STATIC_TENSOR) oS[0] = c->static_scale;
  if (sp_oracle_reduce_add_rmsnorm(&q, hP, oR, hW, hB, 1e-6f, c->quant, hD, oO, oS, NULL) != ORC_OK) {
    fprintf(stderr, "%s: oracle failed\n", c->name);
    return 1;
  }

  /* residual: the shard's rows against the oracle; in place, the other blocks unchanged */
  const int64_t roff = c->in_place && c->replicated ? (int64_t)c->rank * S : 0;
  for (int64_t i = 0; i < (c->in_place ? rrows : S) * H; ++i) {
    const int64_t row = i / H;
    const int in_shard = row >= roff && row < roff + S;
    const char* want = c->in_place ? (const char*)oR : (const char*)oRO;
    if (c->in_place && !in_shard) {
      if (memcmp((const char*)gR + i * ae, (const char*)hR + i * ae, ae)) {
        fprintf(stderr, "%s: residual row %lld of another rank changed\n", c->name, (long long)row);
        return 1;
      }
      continue;
    }
    double g, w;
    if (ae == 2) {
      g = bf16_value(((const uint16_t*)gR)[i]);
      w = bf16_value(((const uint16_t*)want)[i]);
      if (fabs(g - w) > ldexp(fabs(w), -7) + 1e-30) {  /* one bf16 step */
        fprintf(stderr, "%s: residual %lld: %g vs %g\n", c->name, (long long)i, g, w);
        return 1;
      }
    } else {
      g = ((const float*)gR)[i];
      w = ((const float*)want)[i];
      if (fabs(g - w) > 4e-6) {
        fprintf(stderr, "%s: residual %lld: %g vs %g\n", c->name, (long long)i, g, w);
        return 1;
      }
    }
  }
  /* normalised output */
  int64_t differ = 0;
  for (int64_t i = 0; i < S * H; ++i) {
    if (odt == SP_BF16) {
      const double g = bf16_value(((const uint16_t*)gO)[i]), w = bf16_value(((const uint16_t*)oO)[i]);
      if (fabs(g - w) > 1e-3 + ldexp(fabs(w), -7)) {
        fprintf(stderr, "%s: out %lld: %g vs %g\n", c->name, (long long)i, g, w);
        return 1;
      }
    } else {
      const uint8_t gc = ((const uint8_t*)gO)[i], wc = ((const uint8_t*)oO)[i];
      if (gc != wc && !(e4m3_value(gc) == 0.0 && e4m3_value(wc) == 0.0)) {
        ++differ;
        if (abs(e4m3_ordinal(gc) - e4m3_ordinal(wc)) > 1) {
          fprintf(stderr, "%s: code %lld: %#x vs %#x\n", c->name, (long long)i, gc, wc);
          return 1;
        }
      }
    }
  }
  if (differ * 1000 > S * H) {
    fprintf(stderr, "%s: %lld of %lld codes differ\n", c->name, (long long)differ, (long long)(S * H));
    return 1;
  }
  if (gS) {
    for (int64_t s = 0; s < S; ++s) {
      const double rel = fabs(gS[s] - oS[s]) / (oS[s] > 0 ? oS[s] : 1.0);
      if (rel > 1e-5 || (s >= v && gS[s] != 0.0f)) {
        fprintf(stderr, "%s: scale %lld: %g vs %g\n", c->name, (long long)s, gS[s], oS[s]);
        return 1;
      }
    }
  }
  /* padding rows of out are zero */
  for (int64_t i = v * H * (int64_t)oe; i < S * H * (int64_t)oe; ++i)
    if (((const uint8_t*)gO)[i]) {
      fprintf(stderr, "%s: padding row not zero\n", c->name);
      return 1;
    }
  printf("%s: tp=%d rank=%d S=%d H=%d T=%d valid=%lld ok (%lld codes differ by one step)\n", c->name,
         c->tp, c->rank, c->S, c->H, c->T, (long long)v, (long long)differ);

  hipFree(dP); hipFree(dR); hipFree(dW); hipFree(dB); hipFree(dD); hipFree(dO); hipFree(dRO); hipFree(dSc);
  free(hP); free(hR); free(hW); free(hB); free(hD); free(gO); free(gR); free(gS); free(oR); free(oRO); free(oO);
  return 0;
}

int main(void) {
  const Case cases[] = {
      /* name, tp, rank, S, H, T, partials, act, quant, bias, deepstack, replicated, in_place, static */
      {"bf16 + bias, 5 padding rows", 8, 7, 16, 512, 8 * 16 - 5, SP_BF16, SP_BF16, SP_QUANT_NONE, 1, 0, 0, 0, 0.0f},
      {"dynamic e4m3 + deepstack, in place", 4, 3, 24, 768, 4 * 24 - 3, SP_BF16, SP_BF16,
       SP_QUANT_DYNAMIC_TOKEN, 0, 1, 1, 1, 0.0f},
      {"static e4m3, f32 in", 2, 1, 8, 256, 16, SP_F32, SP_F32, SP_QUANT_STATIC_TENSOR, 0, 0, 1, 0, 0.02f},
  };
  hipStream_t stream;
  HIPCHECK(hipStreamCreate(&stream));
  for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) {
    printf("case: %s\n", cases[i].name);
    fflush(stdout);
    if (run(&cases[i], stream)) return 1;
  }
  HIPCHECK(hipStreamDestroy(stream));
  printf("c_gpu_client: all cases ok\n");
  return 0;
}
