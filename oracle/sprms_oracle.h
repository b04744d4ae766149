/*
 * sprms_oracle.h -- plain CPU oracle for the sequence-parallel
 * "reduce-scatter reduce -> residual add -> RMSNorm (+FP8)" shard path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes, links
 * or calls this code; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no source, header,
 * constant or table with the HIP implementation.
 *
 * Arithmetic is IEEE double throughout; results are rounded once, at the
 * end, to the requested storage type.
 *
 * Pages cited (full titles and addresses are listed in the design notes):
 *   [SP/FC]    vllm-ascend SP / FlashComm1 / FlashComm2 guide (ai6s.net)
 *   [LongCat]  LongCat-Flash inference tuning on Atlas A3 (openrokid.csdn.net)
 *   [SPquant]  vLLM SP / AsyncTP / quantisation notes (beaiera.top)
 *   [PR18671]  vllm-ascend PR #18671 walkthrough, GLM DSA-CP (huashanblogllm.xyz)
 */
#ifndef SPRMS_ORACLE_H
#define SPRMS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage types understood by the oracle */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3 = 2, ORC_E2M1 = 3 /* two per byte, even element low */ };

/* output quantisation modes.  Dynamic per-tensor scaling is absent on
 * purpose: its scale needs the max over every rank's rows, so it cannot be
 * computed on one shard ([SPquant] §4, table of per-tensor quantisation
 * correctness). */
enum { ORC_QUANT_NONE = 0, ORC_QUANT_STATIC_TENSOR = 1, ORC_QUANT_DYNAMIC_TOKEN = 2,
       ORC_QUANT_MX_BLOCK = 4 /* per 32-element block, power-of-two (E8M0) scales */ };

enum {
  ORC_OK = 0,
  ORC_ERR_NULL = -1,
  ORC_ERR_SHAPE = -2,
  ORC_ERR_DTYPE = -3,
  ORC_ERR_UNSUPPORTED = -5
};

typedef struct {
  int32_t tp;             /* number of partial sums (tensor-parallel size), >= 1 */
  int32_t tp_rank;        /* this shard's rank, 0 <= tp_rank < tp */
  int64_t shard_rows;     /* S: rows per rank after padding (T_pad / tp) */
  int64_t hidden;         /* H */
  int64_t num_tokens;     /* T: valid tokens over all ranks, 0 <= T <= tp*S */
  int32_t partial_dtype;  /* ORC_F32 | ORC_BF16 */
  int32_t act_dtype;      /* residual, deepstack, weight, bias, residual_out */
  int32_t out_dtype;      /* ORC_F32 | ORC_BF16 (no quant), ORC_E4M3 (quant), ORC_E2M1 (block) */
  int64_t residual_rows;  /* S (shard residual) or tp*S (replicated residual) */
  int64_t deepstack_rows; /* 0 (absent), S or tp*S */
  double partial_scale;   /* factor applied to every partial before the sum (1 = none) */
} orc_problem;

/* Shard layout of [PR18671] §2 and §5.2: contiguous rank shards of
 * S = T_pad / tp rows; rank r starts at r*S; its valid rows are
 * max(0, min(S, T - r*S)).  Returns ORC_ERR_SHAPE when T_pad is not a
 * positive multiple of tp, T > T_pad, or the rank is out of range. */
int orc_shard_geometry(int64_t num_tokens, int64_t num_tokens_pad, int32_t tp,
                       int32_t rank, int64_t* shard_rows, int64_t* local_start,
                       int64_t* valid_rows);

/* The whole shard computation for a list of shard rows.
 *
 * partials   [tp][S][H]   partial_dtype  (rank q's partial for this shard)
 * residual   [residual_rows][H] act_dtype
 * weight     [H] act_dtype;  bias [H] act_dtype or NULL
 * deepstack  [deepstack_rows][H] act_dtype or NULL
 * static_scale   used only by ORC_QUANT_STATIC_TENSOR (must be finite, > 0)
 * rows       n_rows shard-row indices in [0,S); NULL means 0..S-1 (n_rows = S)
 * Outputs are compact, one row per requested row, in request order:
 *   residual_out [n_rows][H] act_dtype
 *   out          [n_rows][H] out_dtype
 *   out_scale    [n_rows] f32 (dynamic mode), [n_rows][H/32] E8M0 bytes (block
 *                mode); may be NULL otherwise
 *   z_dbg, y_dbg [n_rows][H] doubles, optional: the pre-norm sum and the
 *                normalised value before output rounding (0 on pad rows).
 * Returns ORC_OK or a negative ORC_ERR_* code; on error nothing is written. */
int orc_reduce_add_rmsnorm(const orc_problem* p, const void* partials,
                           const void* residual, const void* weight,
                           const void* bias, float eps, int32_t quant_mode,
                           const void* deepstack, float static_scale,
                           int64_t n_rows, const int64_t* rows,
                           void* residual_out, void* out, void* out_scale,
                           double* z_dbg, double* y_dbg);

/* The fused call with the library boundary's own argument list, on host
 * memory: the descriptor below has the field layout of the library's
 * problem descriptor (written out here on its own: the oracle includes no
 * header of the library) and the arguments follow the library entry point,
 * so a caller can hand the same call to both.  The stream is ignored.
 * Semantics on top of orc_reduce_add_rmsnorm:
 *   residual_out NULL      the residual rows this shard uses (block tp_rank of a
 *                          replicated residual) are overwritten in place;
 *   partial_stride         elements from partial q's row s to partial q+1's
 *                          row s; 0 means S*H (packed);
 *   flags bit 0            outputs for the valid rows only, padding rows of
 *                          out / residual_out / out_scale untouched;
 *   partial_scale          0 is read as 1;
 *   out_scale              static: [1] read; dynamic: [S] f32 written; block:
 *                          [S][H/32] E8M0 bytes written.
 * Rejected with ORC_ERR_SHAPE before anything is read or written: partials
 * whose byte span, (tp-1)*stride + S*H elements, overflows or exceeds 2^47
 * bytes; a written byte (residual rows, out, out_scale) that the call also
 * reads (partials, gain, bias, deepstack, residual, the static scale) or
 * writes twice -- the one exception being the residual rows in use updated
 * in place (residual_out NULL or equal to them).
 * Every output is computed before the first write, so a call that returns
 * an error has written nothing. */
typedef struct {
  int32_t tp, tp_rank;
  int64_t shard_rows, hidden, num_tokens;
  int32_t partial_dtype, act_dtype, out_dtype;
  int64_t residual_rows, deepstack_rows;
  void* residual_out;
  int64_t partial_stride;
  int32_t flags;
  float partial_scale;
} orc_abi_problem;

int sp_oracle_reduce_add_rmsnorm(const orc_abi_problem* p, const void* partials, void* residual,
                                 const void* weight, const void* bias, float eps, int quant_mode,
                                 const void* deepstack, void* out, void* out_scale, void* stream);

/* AllGather + unpad of tp shard outputs of S rows (row_bytes each) into out
 * of T rows; shard scales of S rows (scale_row_bytes each) into out_scale of T
 * rows when scales != NULL (scale_row_bytes 0 otherwise). */
int orc_all_gather_unpad(int32_t tp, int64_t S, int64_t row_bytes, int64_t T,
                         const void* const* shards, int64_t scale_row_bytes,
                         const void* const* scales, void* out, void* out_scale);

/* FlashComm2 reorganised batch ids ([odp][otp]) and input regrouping of G
 * ranks' [N][C] inputs into [N/odp][odp*C] per rank. */
int orc_fc2_batch_ids(int32_t G, int32_t otp, int32_t* ids);
int orc_fc2_regroup(int32_t G, int32_t otp, int64_t N, int64_t C, int32_t elt,
                    const void* const* src, void* const* dst);

/* DSA-CP o_proj input exchange, [PR18671] §5.3 path B: attn[p] [S][tp*D] ->
 * out[q] [tp*S][D], row p*S + s = attn[p][s][q*D .. (q+1)*D). */
int orc_dsacp_heads_to_tokens(int32_t tp, int64_t S, int64_t piece, const void* const* attn,
                              void* const* out);

/* Row-parallel GEMM of rank `rank` with its ReduceScatter destinations
 * ([SPquant] §二): P = x w^T with x [tp*S][K], w [N][K] (bf16 bits); dst[r]
 * is rank r's [tp][S][N] receive buffer (out_dtype ORC_BF16 or ORC_F32),
 * slot `rank` row s = P[r*S + s].  rows selects token rows (NULL = all). */
int orc_matmul_scatter(int32_t tp, int32_t rank, int64_t S, int64_t K, int64_t N, int32_t out_dtype,
                       const uint16_t* x, const uint16_t* w, int64_t n_rows, const int64_t* rows,
                       void* const* dst);

/* FP8 producer: x [tp*S][K], w [N][K] e4m3 codes; x_scale 1 or tp*S fp32,
 * w_scale 1 or N fp32; P = (x w^T) * x_scale[m] * w_scale[n], scattered as
 * orc_matmul_scatter. */
int orc_scaled_matmul_scatter(int32_t tp, int32_t rank, int64_t S, int64_t K, int64_t N,
                              int32_t out_dtype, const uint8_t* x, const float* x_scale,
                              int64_t x_scale_rows, const uint8_t* w, const float* w_scale,
                              int64_t w_scale_rows, int64_t n_rows, const int64_t* rows,
                              void* const* dst);

/* Format helpers, exported so that the tests can pin them directly. */
uint16_t orc_bf16_from_double(double x);   /* round to nearest, ties to even */
double orc_bf16_to_double(uint16_t bits);
uint8_t orc_e4m3_from_double(double x);    /* clamp to +-448, nearest, ties to even */
double orc_e4m3_to_double(uint8_t code);   /* NaN for the two NaN codes */
void orc_bf16_from_double_n(const double* x, int64_t n, uint16_t* out);
void orc_e4m3_from_double_n(const double* x, int64_t n, uint8_t* out);
uint8_t orc_e2m1_from_double(double x);    /* clamp to +-6, nearest, ties to even */
double orc_e2m1_to_double(uint8_t code);
void orc_e2m1_from_double_n(const double* x, int64_t n, uint8_t* out);

#ifdef __cplusplus
}
#endif

#endif
