/*
 * sprms.h -- C ABI of libsprms: the fused per-shard hot path that sequence
 * parallelism puts between ReduceScatter and AllGather, on one MI355X
 * (gfx950).
 *
 * In the tensor-parallel tail "AllReduce -> RMSNorm", sequence parallelism
 * splits the AllReduce into ReduceScatter + AllGather and runs the per-token
 * norm (and any per-token quantiser) on each rank's contiguous token shard
 * in between (vllm-ascend SP / FlashComm1 / FlashComm2 guide, ai6s.net,
 * §2.1-§2.3; vLLM SP / AsyncTP / quantisation notes, beaiera.top, §1-§4).
 * For one rank's shard this library computes, in one kernel launch:
 *
 *   z[s][h]  = ((sum over q=0..tp-1 of c*P[q][s][h]) + D[s][h]) + R[s][h]  (fp32, rank order,
 *              c = partial_scale, 1 unless set)
 *   residual_out[s][h] = z[s][h]                                         (rounded to act dtype)
 *   y[s][h]  = z[s][h] * rsqrt(mean_h z[s][h]^2 + eps) * w[h] (+ b[h])
 *   out      = y (bf16 / f32), or FP8 e4m3 codes of y / scale with
 *              scale a static per-tensor constant or max_h |y[s][h]| / 448,
 *              or block-scaled e4m3 / e2m1 codes with one E8M0 scale per
 *              32 elements
 *   rows s >= valid_rows: residual_out, out and out_scale are 0; their
 *              inputs are not read.
 *
 * The sum over q is the reduction half of ReduceScatter: element-wise sum of
 * every rank's partial, each rank keeping its own block of tokens
 * (LongCat-Flash on Atlas A3, openrokid.csdn.net, "o_proj TP K-axis split").
 * One rank's input is emulated as partials[tp][S][H]: the slice
 * [r*S, (r+1)*S) of every rank's partial GEMM output.
 *
 * Around that call the library has the other steps of the same tail, each
 * one kernel, each for one rank's share or for every rank of a group held
 * on one GPU:
 *   sp_matmul_scatter, sp_scaled_matmul_scatter -- the producer: a rank's
 *       row-parallel GEMM (bf16, or e4m3 with scales) writing each token
 *       block into its destination rank's partials buffer;
 *   sp_all_gather_unpad -- the AllGather + unpad that follows the shard;
 *   sp_fc2_regroup, sp_dsacp_heads_to_tokens -- the two regroupings in front
 *       of o_proj (FlashComm2's ODP all-to-all, DSA-CP's head-to-token
 *       exchange);
 *   sp_shard_geometry, sp_validate, sp_error_string, sp_last_error -- host
 *       helpers.
 *
 * All entry points are plain C; pointers named "device" are HIP device
 * pointers (e.g. torch tensor data_ptr() on a ROCm build), everything else
 * is host memory.  The library allocates nothing, keeps no state between
 * calls other than the thread-local last-error text, and never synchronises.
 */
#ifndef SPRMS_H
#define SPRMS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage types.  SP_FP4_E2M1 packs two elements per byte, the even
 * element in the low nibble. */
typedef enum { SP_F32 = 0, SP_BF16 = 1, SP_FP8_E4M3 = 2, SP_FP4_E2M1 = 3 } sp_dtype;

/* Output quantisation.  Static per-tensor and dynamic per-token scales are
 * computable on one shard; dynamic per-tensor is not (its max spans every
 * rank's rows), so it is not offered (vLLM SP / AsyncTP / quantisation notes,
 * §4, per-tensor quantisation correctness table). */
typedef enum {
  SP_QUANT_NONE = 0,           /* out = y in out_dtype (SP_BF16 or SP_F32) */
  SP_QUANT_STATIC_TENSOR = 1,  /* out = e4m3(y / out_scale[0]), out_scale read */
  SP_QUANT_DYNAMIC_TOKEN = 2,  /* out_scale[s] = max_h|y| / 448, out = e4m3(y / out_scale[s]) */
  /* 3 is reserved for dynamic per-tensor scaling and always rejected */
  SP_QUANT_MX_BLOCK = 4        /* per-block scaling, blocks of 32 consecutive elements of a row
                                  (the per-block row of the quantisation table above), in the
                                  OCP microscaling form native to gfx950: per block
                                  e = floor(log2 max|y|) - emax (emax 8 for e4m3, 2 for e2m1),
                                  clamped to [-127, 127] (an all-zero block gets -127);
                                  out = elem(clamp(y * 2^-e)) in out_dtype SP_FP8_E4M3 (MXFP8)
                                  or SP_FP4_E2M1 (MXFP4); out_scale[s][b] = e + 127 (E8M0) */
} sp_quant;

typedef enum {
  SP_OK = 0,
  SP_ERR_NULL = -1,        /* a required pointer is NULL */
  SP_ERR_SHAPE = -2,       /* inconsistent sizes, rank or row counts */
  SP_ERR_DTYPE = -3,       /* unsupported dtype combination */
  SP_ERR_ALIGN = -4,       /* a device pointer is not aligned as the call requires */
  SP_ERR_UNSUPPORTED = -5, /* a quant mode (dynamic per-tensor included), flag or reserved
                              field the call does not support */
  SP_ERR_HIP = -6          /* the kernel launch failed */
} sp_status;

/* Problem descriptor (host memory, read during the call only). */
typedef struct {
  int32_t tp;             /* number of partials = tensor-parallel size, 1 <= tp <= 64 */
  int32_t tp_rank;        /* 0 <= tp_rank < tp */
  int64_t shard_rows;     /* S = T_pad / tp, 0 <= S <= 2^31 - 1 */
  int64_t hidden;         /* H, 8 <= H <= 32768, H % 8 == 0 */
  int64_t num_tokens;     /* valid tokens T over all ranks, 0 <= T <= tp * S */
  int32_t partial_dtype;  /* SP_F32 | SP_BF16 */
  int32_t act_dtype;      /* residual, deepstack, weight, bias, residual_out: SP_F32 | SP_BF16 */
  int32_t out_dtype;      /* SP_BF16 | SP_F32 with SP_QUANT_NONE; SP_FP8_E4M3 with the static or
                             per-token modes; SP_FP8_E4M3 | SP_FP4_E2M1 with SP_QUANT_MX_BLOCK */
  int64_t residual_rows;  /* S (shard residual) or tp*S (replicated: block tp_rank is used) */
  int64_t deepstack_rows; /* 0 iff deepstack == NULL, else S or tp*S (block tp_rank is used) */
  void* residual_out;     /* device [S][H] act_dtype, or NULL: write the used residual rows in place */
  int64_t partial_stride; /* elements from partial q's row s to partial q+1's row s; 0 means S*H
                             (a packed [tp][S][H] block).  T_pad*H lets partials be the rank's
                             row block of tp full [T_pad][H] partial tensors held in one buffer. */
  int32_t flags;          /* 0 or SP_FLAG_VALID_ROWS_ONLY */
  float partial_scale;    /* every partial is multiplied by this factor before it joins the
                             sum (the DSA-CP o_proj finalize scales its output before the
                             reduction: vllm-ascend PR #18671 walkthrough, §5.3); 0 is read as
                             1; must be finite */
} sp_problem;

/* Flag: write out, out_scale and residual_out for the shard's valid rows
 * [0, valid_rows) only and leave the padding rows untouched, so that `out`
 * may point at row r*S of an unpadded gathered [T][H] tensor (the AllGather
 * + unpad of FlashComm1, vllm-ascend SP / FlashComm guide, §3.3, written in
 * place by each rank). */
#define SP_FLAG_VALID_ROWS_ONLY 1

/*
 * sp_reduce_add_rmsnorm -- enqueue the fused shard path on `stream`.
 *
 * Defined by: the replacement pattern ReduceScatter -> maybe_chunk_residual
 * -> fused add + RMSNorm (+bias) -> AllGather, and the deepstack variant
 * that adds chunk [tp_rank] of the deepstack embeddings after the
 * ReduceScatter (vllm-ascend SP / FlashComm guide, §2.3); the quantiser
 * moved onto the shard (vLLM SP / AsyncTP / quantisation notes, §4); the
 * contiguous shard, valid-row rule and zeroed padding rows (vllm-ascend
 * PR #18671 walkthrough, §2, §5.2, §5.3).
 *
 * Arguments (device pointers, row-major, no row padding; 16-byte aligned except
 * out, which needs the width of one 8-element store: 16 bytes for bf16 and f32,
 * 8 for e4m3, 4 for packed e2m1):
 *   p          problem descriptor (host)
 *   partials   [tp][S][H] partial_dtype: partial q's rows of this shard
 *   residual   [residual_rows][H] act_dtype; written in place when
 *              p->residual_out == NULL (only the rows of block tp_rank)
 *   weight     [H] act_dtype
 *   bias       [H] act_dtype, or NULL (no bias)
 *   eps        >= 0, added to the mean of squares inside the square root
 *   quant_mode sp_quant
 *   deepstack  [deepstack_rows][H] act_dtype, or NULL
 *   out        [S][H] out_dtype (e4m3 codes are one byte each; e2m1 codes two per byte,
 *              i.e. [S][H/2] bytes)
 *   out_scale  SP_QUANT_STATIC_TENSOR: [1] f32 scale, read on the device (> 0);
 *              SP_QUANT_DYNAMIC_TOKEN: [S] f32, written;
 *              SP_QUANT_MX_BLOCK: [S][H/32] E8M0 bytes, written (H % 32 == 0);
 *              SP_QUANT_NONE: ignored
 *   stream     hipStream_t to enqueue on (NULL = default stream)
 *
 * Arithmetic: fp32 throughout; partial sums in ascending rank order, then
 * deepstack, then residual; the norm and the quantiser use the unrounded fp32
 * sum; stores round to nearest even; e4m3 numbers are clamped to +-448.
 * A dynamic row whose max |y| is 0 gets scale 0 and zero codes.
 * NaN (the pages do not cover it) propagates and is never turned into a
 * number: a NaN input element makes that residual_out element and every
 * output of its row NaN (through the sum of squares); a NaN gain or bias
 * element makes its column NaN.  NaN outputs are IEEE NaN in bf16/f32, the
 * code 0x7F in e4m3; a per-token row holding a NaN gets scale NaN
 * (0x7FC00000) and all codes 0x7F; a block holding a NaN gets the E8M0 NaN
 * byte 0xFF and element codes 0x7F (e4m3) or 0 (e2m1).
 *
 * Ownership and errors: the caller owns every buffer.  No byte the call
 * writes (residual_out or the residual rows updated in place, out,
 * out_scale) may be read by it (partials, weight, bias, deepstack, the
 * residual, the static scale) or written twice; the one exception is the
 * in-place update (residual_out NULL, or equal to the residual rows in
 * use).  The partials may span at most 2^47 bytes ((tp-1)*partial_stride +
 * S*H elements).  Every check runs on the host before anything is enqueued,
 * so a call that returns an error (SP_ERR_SHAPE for the rules above) has
 * written nothing.  Returns SP_OK or a negative sp_status; sp_last_error()
 * gives the detail.  S == 0 enqueues nothing.  Rows outside [0, S) of out /
 * residual_out are never touched.
 */
int sp_reduce_add_rmsnorm(const sp_problem* p, const void* partials, void* residual,
                          const void* weight, const void* bias, float eps, int quant_mode,
                          const void* deepstack, void* out, void* out_scale, void* stream);

/* Problem descriptor of sp_all_gather_unpad (host memory, read during the call only). */
typedef struct {
  int32_t tp;               /* number of shards, 1 <= tp <= 64 */
  int32_t dtype;            /* element type of the shard outputs (any sp_dtype) */
  int64_t shard_rows;       /* S, rows per shard (padded), 0 <= S <= 2^31 - 1 */
  int64_t hidden;           /* H, H % 8 == 0 (H % 16 for e2m1), 8 <= H <= 32768 */
  int64_t num_tokens;       /* T, valid tokens over all shards, 0 <= T <= tp * S, T < 2^31 */
  int64_t scale_row_bytes;  /* bytes of scale per row, 0 <= . <= 65536: 0 (none), 4 (one f32
                               per token), H/32 (one E8M0 byte per 32-element block) */
} sp_gather_problem;

/*
 * sp_all_gather_unpad -- the AllGather + unpad that follows the shard path:
 * shard q's rows [0, v_q), v_q = max(0, min(S, T - q*S)), become rows
 * [q*S, q*S + v_q) of the gathered tensor; padding rows are dropped
 * (vllm-ascend SP / FlashComm guide, §3.3, all_gather then unpad; the
 * quantised payload and its scales are gathered together: vLLM SP / AsyncTP /
 * quantisation notes, §4).
 *
 *   g             problem descriptor (host)
 *   shards        host array of tp device pointers, shard q's output [S][H] (dtype).
 *                 On one GPU these are local buffers; on a node they may be
 *                 peer-mapped buffers of the other ranks (the kernel pulls).
 *   shard_scales  host array of tp device pointers to [S][scale_row_bytes] scales, or
 *                 NULL (then scale_row_bytes must be 0)
 *   out           device [T][H] dtype; out and every shard 16-byte aligned when a
 *                 row is a multiple of 16 bytes, else 8-byte aligned
 *   out_scale     device [T][scale_row_bytes]; required iff shard_scales != NULL
 *   stream        hipStream_t (NULL = default stream)
 *
 * Bytes are copied unchanged (bit-exact).  Same error convention as
 * sp_reduce_add_rmsnorm: every check runs before anything is enqueued, and
 * neither out nor out_scale may overlap a shard, a shard's scales or each
 * other (SP_ERR_SHAPE).  T == 0 enqueues nothing.
 */
int sp_all_gather_unpad(const sp_gather_problem* g, const void* const* shards,
                        const void* const* shard_scales, void* out, void* out_scale,
                        void* stream);

/* Problem descriptor of sp_fc2_regroup (host memory, read during the call only). */
typedef struct {
  int32_t global_tp;  /* G, ranks of the tensor-parallel group, 2 <= G <= 64 */
  int32_t otp;        /* ranks that compute o_proj together, 1 <= otp < G, G % otp == 0 */
  int32_t dtype;      /* element type: SP_F32 | SP_BF16 | SP_FP8_E4M3 */
  int32_t rank;       /* -1: write every rank's dst (one GPU holding the whole group);
                         0 <= rank < G: write dst[rank] only (a rank's own call on a node,
                         the other dst entries are ignored and may be NULL) */
  int64_t tokens;     /* N, N % G == 0, 0 <= N < 2^31 */
  int64_t cols;       /* C = H / G, feature columns held by each rank, C * elt % 4 == 0 */
} sp_fc2_problem;

/*
 * sp_fc2_regroup -- the FlashComm2 input regrouping of o_proj (vllm-ascend SP
 * / FlashComm guide, §4.3-4.4): with odp = G / otp, the G ranks form ODP
 * groups of odp consecutive ranks; the N tokens form G equal segments; rank
 * r = g*odp + j ends up holding token segments j + k*odp (k = 0..otp-1, in
 * that order, the "reorganised batch ids") with the feature columns of the
 * odp ranks of its ODP group side by side, i.e. [N/odp][odp*C].  Ranks with
 * the same j form an OTP group: they hold the same tokens, different feature
 * columns, and their o_proj partials reduce-scatter so that rank r keeps
 * segment r, the sequence-parallel layout.
 *
 *   f    problem descriptor (host)
 *   src  host array of G device pointers, rank q's [N][C] input (its feature
 *        columns of every token); on a node, peer-mapped buffers
 *   dst  host array of G device pointers, rank r's [N/odp][odp*C] output
 *
 * Pointers 16-byte aligned (4-byte when C * elt % 16 != 0); a written dst
 * must not overlap any src or another written dst.  Bytes are copied
 * unchanged, one workgroup per destination row, so the rows written times
 * the workgroup size (up to 1024) must stay below 2^32.  N == 0 enqueues
 * nothing.  Same error convention as sp_reduce_add_rmsnorm.
 */
int sp_fc2_regroup(const sp_fc2_problem* f, const void* const* src, void* const* dst,
                   void* stream);

/* Problem descriptor of sp_dsacp_heads_to_tokens (host memory, read during the call only). */
typedef struct {
  int32_t tp;          /* ranks of the tensor-parallel group, 1 <= tp <= 64 */
  int32_t dtype;       /* element type: SP_F32 | SP_BF16 | SP_FP8_E4M3 */
  int32_t rank;        /* -1: every rank's output; 0 <= rank < tp: out[rank] only (the
                          other out entries are ignored and may be NULL) */
  int32_t reserved;    /* 0 */
  int64_t shard_rows;  /* S, tokens of each rank's (padded) shard, 0 <= tp*S < 2^31 */
  int64_t head_cols;   /* D, columns of one rank's heads (heads per rank x value head
                          dim), D * elt % 4 == 0 */
} sp_dsacp_problem;

/*
 * sp_dsacp_heads_to_tokens -- the exchange in front of o_proj on DSA-CP's
 * path B (vllm-ascend PR #18671 walkthrough, §5.3): under sequence
 * parallelism rank p's attention output holds its S local tokens with every
 * rank's heads, [S][tp*D]; o_proj is row-parallel over the heads, so each
 * rank needs every token with its own heads.  The page's view [S, tp, D],
 * permute(1, 0, 2) and all_to_all_single over the tp group amount to
 *
 *   out[q][p*S + s][d] = attn[p][s][q*D + d]
 *
 * after which o_proj (row-parallel, unreduced), the output scale and one
 * reduce-scatter hand rank p its S rows again: the fused call of this
 * library with partial_scale = the output scale.
 *
 *   f      problem descriptor (host)
 *   attn   host array of tp device pointers, rank p's [S][tp*D]; on a node,
 *          peer-mapped buffers
 *   out    host array of tp device pointers, rank q's [tp*S][D]
 *
 * Pointers 16-byte aligned (4-byte when D * elt % 16 != 0); a written out
 * must not overlap any attn or another written out.  Bytes are copied
 * unchanged.  S == 0 enqueues nothing.  Same error convention as
 * sp_reduce_add_rmsnorm.
 */
int sp_dsacp_heads_to_tokens(const sp_dsacp_problem* f, const void* const* attn,
                             void* const* out, void* stream);

/* Problem descriptor of sp_matmul_scatter (host memory, read during the call only). */
typedef struct {
  int32_t tp;          /* ranks of the tensor-parallel group, 1 <= tp <= 64 */
  int32_t rank;        /* the producing rank q, 0 <= rank < tp */
  int64_t shard_rows;  /* S; x has M = tp*S token rows (padded), 0 <= M < 2^31 */
  int64_t k;           /* K, this rank's slice of the input features, K % 8 == 0, 8 <= K <= 2^20 */
  int64_t n;           /* N, output columns (the hidden size H), N % 8 == 0, 8 <= N <= 2^20 */
  int32_t in_dtype;    /* x and w: SP_BF16 (sp_matmul_scatter) or SP_FP8_E4M3
                          (sp_scaled_matmul_scatter, then K % 16 == 0, 16 <= K) */
  int32_t out_dtype;   /* SP_BF16 | SP_F32: the partial dtype of the fused call */
  int64_t x_scale_rows;  /* e4m3 only: 1 (per-tensor scale) or M (per-token); 0 for bf16 */
  int64_t w_scale_rows;  /* e4m3 only: 1 (per-tensor scale) or N (per output column); 0 for bf16 */
} sp_matmul_problem;

/*
 * sp_matmul_scatter -- the producer in front of the shard path: rank q's
 * row-parallel GEMM with its ReduceScatter destinations (vLLM SP / AsyncTP
 * / quantisation notes, §2, GEMM + ReduceScatter at a block's exit; o_proj
 * split along K over the tp ranks: LongCat-Flash on Atlas A3, o_proj TP
 * K-axis split).  It computes the unreduced partial
 *
 *   P[m][n] = sum over k of x[m][k] * w[n][k]      (fp32 accumulation)
 *
 * and writes token row m to rank r = m / S, row s = m - r*S, slot q of r's
 * receive buffer:
 *
 *   dst[r][q][s][n] = P[m][n]   (rounded to out_dtype, nearest-even)
 *
 * so that dst[r], once every rank has written its slot, is exactly the
 * partials[tp][S][N] argument of rank r's sp_reduce_add_rmsnorm.
 *
 *   p    problem descriptor (host)
 *   x    device [M][K] bf16, this rank's K-slice of every token's input
 *   w    device [N][K] bf16, this rank's K-slice of the weight (one row per
 *        output column, the storage of a linear layer's weight)
 *   dst  host array of tp device pointers, rank r's [tp][S][N] receive
 *        buffer in out_dtype; only slot q (rows [q*S, (q+1)*S)) is written.
 *        On one GPU these are local; on a node, peer-mapped buffers.
 *
 * Pointers 16-byte aligned; the written slots must not overlap x, w or each
 * other.  x_scale_rows and w_scale_rows must be 0.  M == 0 enqueues nothing.
 * Same error convention as sp_reduce_add_rmsnorm.
 */
int sp_matmul_scatter(const sp_matmul_problem* p, const void* x, const void* w, void* const* dst,
                      void* stream);

/*
 * sp_scaled_matmul_scatter -- the FP8 form of the producer (vLLM SP /
 * AsyncTP / quantisation notes, §4: after sequence parallelism the
 * row-parallel GEMM is an FP8 GEMM with its scales, fused with the
 * ReduceScatter): x and w hold OCP e4m3 codes and
 *
 *   P[m][n] = (sum over k of x[m][k] * w[n][k]) * x_scale[m or 0] * w_scale[n or 0]
 *
 * (products exact, fp32 accumulation on the matrix cores, the two scales
 * applied to the fp32 sum), scattered and rounded exactly as
 * sp_matmul_scatter.  x_scale: device fp32 [x_scale_rows], w_scale: device
 * fp32 [w_scale_rows], 4-byte aligned.  Other arguments and errors as for
 * sp_matmul_scatter; p->in_dtype must be SP_FP8_E4M3.
 */
int sp_scaled_matmul_scatter(const sp_matmul_problem* p, const void* x, const float* x_scale,
                             const void* w, const float* w_scale, void* const* dst, void* stream);

/*
 * sp_validate -- the host-side checks of sp_reduce_add_rmsnorm, alone.
 * Same arguments (no stream); touches no device memory and makes no HIP
 * call.  Returns SP_OK or the status sp_reduce_add_rmsnorm would return
 * before launching.
 */
int sp_validate(const sp_problem* p, const void* partials, const void* residual,
                const void* weight, const void* bias, float eps, int quant_mode,
                const void* deepstack, const void* out, const void* out_scale);

/*
 * sp_shard_geometry -- contiguous shard layout (vllm-ascend PR #18671
 * walkthrough, §2 and §5.2): S = num_tokens_pad / tp, local_start = rank*S,
 * valid_rows = max(0, min(S, num_tokens - local_start)).  Host only.
 * Returns SP_ERR_SHAPE when num_tokens_pad is not a multiple of tp,
 * num_tokens > num_tokens_pad, a count is negative or rank is out of range;
 * SP_ERR_NULL for a NULL output pointer.
 */
int sp_shard_geometry(int64_t num_tokens, int64_t num_tokens_pad, int32_t tp, int32_t rank,
                      int64_t* shard_rows, int64_t* local_start, int64_t* valid_rows);

/* Static text for a status code (never NULL). */
const char* sp_error_string(int status);

/* Detail of the last failing call on this thread (static storage, never NULL). */
const char* sp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPRMS_H */
