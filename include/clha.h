/*
 * clha.h - C ABI of the CLHA calibration library for AMD Instinct MI355X (gfx950).
 *
 * CLHA (Cross-Layer Hessian Aggregation) calibrates Mixture-of-Experts weights
 * that adjacent layers share (cross-layer weight sharing, CLWS).  The method,
 * as the gist.science summary "CLHA - Cross-Layer Hessian Aggregation for
 * quantizing weight-shared MoE transformers" states it, has three phases
 * (section 2.2):
 *   1. collection  - per layer and per active expert, accumulate the Hessian
 *                    (activation second moment) and the token count;
 *   2. aggregation - per shared expert, H_comb = sum_i alpha_i H_i with
 *                    alpha_i = n_i / sum n (routing frequency) or 1/m (equal);
 *   3. quantization - standard GPTQ column-sequential updates on H_comb, at b
 *                    bits, or b+1 bits for always-active shared experts
 *                    (CLHA-MP, section 2.3).
 * Section 2.4 requires the Hessian accumulators to be keyed by layer, not by
 * the shared weight module; this ABI makes the layer an explicit argument of
 * every collection call and rejects two layers that alias one accumulator.
 *
 * Conventions
 *   - Every array argument marked "device" is a pointer into GPU memory that the
 *     caller allocated and owns.  The library never allocates or frees device
 *     memory: each context's status record (64 bytes) is one of 1024 records in
 *     a device array of the library's code object, and the library's only
 *     allocations are host-side (bookkeeping, page-locked staging of job tables).
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *     Every compute call only enqueues work on `stream` and returns; outputs are
 *     valid once the stream has been synchronised (clha_sync does that).
 *   - Argument, shape and alignment errors are detected on the host before
 *     anything is enqueued; the call then returns the error and enqueues
 *     nothing.  Numerical failures found on the device (non-finite router
 *     logits, a damped Hessian that is not positive definite or has a
 *     non-finite diagonal) are written to the failing GPTQ job's status, when
 *     it has one, and latched in the context's status record; the next
 *     clha_sync returns the first of them and names the layer, job or Hessian.
 *   - Matrices are row-major.  bf16 values are passed as their uint16 bit
 *     patterns.  Device pointers must be 16-byte aligned.
 *   - A context is used by one host thread at a time.  No C++ exception crosses
 *     this interface.
 */
#ifndef CLHA_H
#define CLHA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CLHA_API __attribute__((visibility("default")))

typedef enum clha_status {
  CLHA_OK = 0,
  CLHA_ERR_INVALID_ARG = 1,   /* null pointer, unknown layer, aliased buffers, bad enum */
  CLHA_ERR_SHAPE = 2,         /* a size outside the supported range */
  CLHA_ERR_ALIGN = 3,         /* a device pointer not 16-byte aligned */
  CLHA_ERR_HIP = 4,           /* the HIP runtime reported an error */
  CLHA_ERR_NOT_PD = 5,        /* a damped Hessian is not positive definite */
  CLHA_ERR_NONFINITE = 6,     /* a router logit is NaN or infinite */
  CLHA_ERR_WORKSPACE = 7      /* workspace smaller than the matching *_workspace_bytes */
} clha_status;

typedef enum clha_alpha_mode {
  CLHA_ALPHA_ROUTING_FREQ = 0, /* alpha_i = n_i / sum_j n_j ("CLHA-rt", section 2.2)      */
  CLHA_ALPHA_EQUAL = 1,        /* alpha_i = 1/m over the m non-empty layers ("CLHA-eq")    */
  CLHA_ALPHA_EXPLICIT = 2,     /* caller-given alpha_i; alpha = (1, 0) is PLIC (section 2.1) */
  CLHA_ALPHA_EXPLICIT_PER_SLOT = 3  /* caller-given alpha_i per expert slot (Proposition 1 holds
                                       for each shared weight separately, section 2.1) */
} clha_alpha_mode;

typedef enum clha_dtype { CLHA_F32 = 0, CLHA_BF16 = 1 } clha_dtype;

/* Shape of the MoE block whose routed experts a group of layers shares. */
typedef struct clha_moe_desc {
  int32_t d;            /* hidden size; columns of every calibrated matrix; multiple of 128, <= 8192 */
  int32_t n_routed;     /* E, routed experts; 1..256 */
  int32_t top_k;        /* K, experts per token; 1..min(E, 16) */
  int32_t n_shared;     /* always-active shared experts; 0 or more.  They all see the same
                           input, so one Hessian slot (index E) serves all of them. */
  int64_t max_tokens;   /* largest n_tokens of one clha_collect_hessians call; >= 1 */
} clha_moe_desc;

typedef struct clha_ctx clha_ctx;

/* Creates a context for one MoE block shape on the current HIP device.
 * Errors: INVALID_ARG (null), SHAPE (desc outside the ranges above), HIP (also when
 * 1024 contexts are already alive on the device). */
CLHA_API clha_status clha_create(const clha_moe_desc* desc, clha_ctx** out);

/* Frees the context (host bookkeeping; its status record returns to the pool).
 * Accepts NULL. */
CLHA_API clha_status clha_destroy(clha_ctx* ctx);

/* Text of the last error on this context (static storage owned by ctx). */
CLHA_API const char* clha_last_error(const clha_ctx* ctx);

/* Number of Hessian slots per layer: E, plus one when n_shared > 0. */
CLHA_API int32_t clha_num_slots(const clha_ctx* ctx);

/* Binds the accumulators of one layer (the layer-aware collection of section 2.4).
 *   S      device, float [slots][d][d]: Gram sums S[e] = sum_t x_t x_t^T over the tokens
 *          routed to slot e (slot E: all tokens).  Only the lower triangle (i >= j) is
 *          ever written; before the first collection the caller either zeroes the
 *          buffer or calls clha_reset_layer.
 *   counts device, int64 [slots]: token counts n[e]; zeroed by the caller (or by
 *          clha_reset_layer).
 * A layer may be registered again (rebinding it).  Registering a buffer range that
 * overlaps another layer's S or counts returns INVALID_ARG: two layers never share
 * one accumulator. */
CLHA_API clha_status clha_register_layer(clha_ctx* ctx, int32_t layer, float* S, int64_t* counts);

/* Starts a new accumulation for a registered layer (section 2.4: per-layer
 * accumulators, emptied between calibration runs) without clearing S:
 *   counts are zeroed on `stream` now; the next clha_collect_hessians of this
 *   layer that has tokens stores instead of adding: S[e] = X_e^T X_e (lower
 *   triangle; slots that receive no token are zeroed) and counts[e] = n_e.
 *   Later collections add as usual.
 * Until that collection S holds stale sums, but with zero counts every
 * aggregation treats the layer as empty and reads none of them.
 * Errors: INVALID_ARG (null ctx, unregistered layer), HIP. */
CLHA_API clha_status clha_reset_layer(clha_ctx* ctx, int32_t layer, void* stream);

/* Device workspace bytes that clha_collect_hessians needs for max_tokens tokens. */
CLHA_API size_t clha_collect_workspace_bytes(const clha_ctx* ctx);

/* Collection phase for one calibration batch of one layer (section 2.2, phase 1):
 *   1. routes each token to its top-K experts (larger logit first, ties to the lower index);
 *   2. buckets tokens per expert (counts, exclusive offsets, token lists ascending);
 *   3. S[e] += X_e^T X_e (fp32 accumulation of bf16 products) for every routed expert,
 *      and S[E] = X^T X over all of the layer's tokens so far when the block has shared
 *      experts; counts[e] += n_e, counts[E] += n_tokens (stored instead of added by the
 *      first collection with tokens after clha_reset_layer).  Each token goes to exactly
 *      K distinct routed experts, so X^T X = (sum_e S[e]) / K: S[E] is formed that way
 *      from the routed sums (fp64 sum in slot order, one rounding) after each batch.
 *   x        device, bf16 bits [n_tokens][d]
 *   logits   device, float [n_tokens][E]
 *   topk_out, offsets_out, token_ids_out: optional device outputs of this batch's
 *            routing (int32 [n_tokens][K], int64 [E+1], int32 [n_tokens*K]); NULL skips.
 *   workspace device, >= clha_collect_workspace_bytes(ctx) bytes.
 * Non-finite logits latch CLHA_ERR_NONFINITE (routing of that token is then undefined).
 * Errors: INVALID_ARG (unregistered layer, null x/logits), SHAPE (n_tokens outside
 * 0..max_tokens), ALIGN, WORKSPACE.  n_tokens == 0 enqueues nothing and reads none of
 * the pointers (they may be NULL). */
CLHA_API clha_status clha_collect_hessians(clha_ctx* ctx, int32_t layer, int64_t n_tokens,
                                           const uint16_t* x, const float* logits,
                                           int32_t* topk_out, int64_t* offsets_out,
                                           int32_t* token_ids_out,
                                           void* workspace, size_t workspace_bytes, void* stream);

/* Aggregation phase (section 2.1 Proposition 1, section 2.2 phase 2) over the given
 * layers, for every slot e:
 *   ROUTING_FREQ: H[e] = (sum_i S_i[e]) / (sum_i n_i[e])
 *   EQUAL:        H[e] = sum_i (1/m) (S_i[e] / n_i[e]) over the m layers with n_i[e] > 0
 *   EXPLICIT:     H[e] = sum_i alpha_i (S_i[e] / n_i[e]); layers with n_i[e] == 0 drop out
 *                 and, if a dropped layer had alpha_i != 0, the rest are renormalised.
 *   EXPLICIT_PER_SLOT: the same with weights alpha_i[e] of each slot.
 * A slot with no tokens in any layer gets H[e] = I and alpha 0.
 *   layers    host, int32 [n_layers]; registered layers; n_layers 1..8
 *   alpha     EXPLICIT: host, float [n_layers], finite and >= 0.
 *             EXPLICIT_PER_SLOT: device, float [slots][n_layers], finite and >= 0 (not
 *             checked: it is read on the device; other values give undefined H).
 *             Other modes: ignored (may be NULL).
 *   H_out     device, float [slots][d][d]; full symmetric matrices
 *   alpha_out device, float [slots][n_layers] (the weights used); may be NULL
 * Errors: INVALID_ARG, SHAPE, ALIGN. */
CLHA_API clha_status clha_aggregate(clha_ctx* ctx, int32_t n_layers, const int32_t* layers,
                                    clha_alpha_mode mode, const float* alpha,
                                    float* H_out, float* alpha_out, void* stream);

/* One GPTQ job: one weight matrix (e.g. an expert's gate and up stacked row-wise)
 * and the Hessian it is quantized against. */
typedef struct clha_gptq_job {
  const float* H;      /* device, float [cols][cols], symmetric PSD, undamped (e.g. H_comb) */
  const void* W;       /* device, [rows][cols] row-major, float or bf16 bits (w_dtype) */
  int32_t w_dtype;     /* clha_dtype */
  int32_t rows;        /* >= 1 */
  int32_t bits;        /* 2..8; b, or b+1 for always-active shared experts (CLHA-MP) */
  int32_t pad_;
  uint8_t* codes;      /* device out, uint8 [rows][cols]: q in [0, 2^bits - 1] */
  float* scales;       /* device out, float [rows][cols/group] */
  uint8_t* zeros;      /* device out, uint8 [rows][cols/group] */
  float* loss;         /* device out, float [1]: tr[(Wq - W) H (Wq - W)^T]; may be NULL */
  const float* H_eval; /* device, float [cols][cols], may be NULL: a second Hessian to evaluate
                          the result under (e.g. one layer's H_l, the calibration-Hessian
                          error of section 4); H_eval may equal H */
  float* loss_eval;    /* device out, float [1]: tr[(Wq - W) H_eval (Wq - W)^T], computed
                          directly (2 rows cols^2 flops); needed iff H_eval is given */
  uint8_t* dead;       /* device out, uint8 [cols], may be NULL: 1 where H_ii == 0 (the column
                          was treated as dead), in natural column order */
  int32_t* status;     /* device out, int32 [1], may be NULL: CLHA_OK, CLHA_ERR_NOT_PD (the
                          damped H is not positive definite) or CLHA_ERR_NONFINITE (a diagonal
                          entry of H is NaN or infinite); the job's outputs are undefined
                          unless CLHA_OK.  Off-diagonal entries of H and the weights must be
                          finite; they are not checked. */
} clha_gptq_job;

/* Device workspace bytes clha_gptq_quantize needs for these jobs. */
CLHA_API size_t clha_gptq_workspace_bytes(const clha_ctx* ctx, int32_t n_jobs,
                                          const clha_gptq_job* jobs, int32_t cols);

/* Quantization phase (section 2.2 phase 3, "standard GPTQ") for a batch of jobs.
 * For every distinct H (jobs sharing an H pointer share one factorisation):
 *   dead columns (H_ii == 0) get H_ii := 1 and their weights are treated as 0;
 *   lambda = damp * mean(diag H); Hd = H + lambda I;
 *   U = upper Cholesky factor of Hd^-1.
 * Then for each job, blocks of `block` columns, column by column: at each group's first
 * column fit the per-row asymmetric grid on the group's current weights (range widened
 * to contain 0; an all-zero group uses (-1, 1); s = (max - min)/maxq; z = rint(-min/s));
 * q = clamp(rint(w/s) + z, 0, maxq); err = (w - s(q - z))/U_jj; propagate err into the
 * later columns of the block through row j of U, and after the block into all later
 * columns.  Codes, scales and zero points are decided in fp32 with IEEE division and
 * round-half-to-even.  loss = sum_j err_j^2 - lambda ||Wq - W||^2, which equals
 * tr[(Wq - W) H (Wq - W)^T] on the undamped H.
 *   cols      columns of every job; multiple of `block`, <= 8192
 *   group     g; divides block
 *   block     64 or 128
 *   damp      relative damping, >= 0 (0.01 is customary)
 * Errors: INVALID_ARG, SHAPE, ALIGN, WORKSPACE.  A Hessian that is not positive definite
 * after damping, or one with a non-finite diagonal entry, sets CLHA_ERR_NOT_PD or
 * CLHA_ERR_NONFINITE in the status of every job on it (the other jobs are unaffected) and
 * latches it for clha_sync, which names the lowest failing job index of the call. */
CLHA_API clha_status clha_gptq_quantize(clha_ctx* ctx, int32_t n_jobs, const clha_gptq_job* jobs,
                                        int32_t cols, int32_t group, int32_t block, float damp,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* Options of clha_gptq_quantize_ex (bit flags).  Neither is on the CLHA pages, which
 * name only "standard GPTQ"; both are common GPTQ settings.
 *   CLHA_GPTQ_ACT_ORDER      process the columns by decreasing H_ii (a dead column counts
 *                            as 1; ties by column index); a grid is fitted at every
 *                            group-th processed column over the next `group` processed
 *                            columns, so a column's grid is given by g_idx.
 *   CLHA_GPTQ_STATIC_GROUPS  fit the grid of every row and natural group (columns
 *                            k*group .. k*group+group-1) once, before any update, on the
 *                            weights with dead columns zeroed; every column is then
 *                            quantized on its natural group's grid (g_idx[i] = i/group),
 *                            also under CLHA_GPTQ_ACT_ORDER. */
typedef enum clha_gptq_flag {
  CLHA_GPTQ_ACT_ORDER = 1,
  CLHA_GPTQ_STATIC_GROUPS = 2
} clha_gptq_flag;

/* Device workspace bytes clha_gptq_quantize_ex needs for these jobs and flags.  Activation
 * order adds a permuted copy of every distinct H (4 cols^2 bytes each). */
CLHA_API size_t clha_gptq_workspace_bytes_ex(const clha_ctx* ctx, int32_t n_jobs,
                                             const clha_gptq_job* jobs, int32_t cols, uint32_t flags);

/* clha_gptq_quantize with options.  Codes are always returned in natural column order
 * (codes[r][i] is column i's code); column i dequantizes as
 *   scales[r][g_idx[i]] * (codes[r][i] - zeros[r][g_idx[i]]).
 * The loss is that of the returned Wq (the same identity as clha_gptq_quantize).
 *   flags      0 or an OR of clha_gptq_flag values; 0 gives clha_gptq_quantize exactly
 *   g_idx      NULL, or a host array of n_jobs pointers, each NULL or device int32 [cols]
 *              (4-byte aligned) that receives the job's g_idx
 * Errors: as clha_gptq_quantize; INVALID_ARG for unknown flags, ALIGN for a misaligned
 * g_idx pointer. */
CLHA_API clha_status clha_gptq_quantize_ex(clha_ctx* ctx, int32_t n_jobs, const clha_gptq_job* jobs,
                                           int32_t cols, int32_t group, int32_t block, float damp,
                                           uint32_t flags, int32_t* const* g_idx, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* Device workspace bytes clha_inverse_cholesky needs for n Hessians of size cols. */
CLHA_API size_t clha_inverse_cholesky_workspace_bytes(const clha_ctx* ctx, int32_t n, int32_t cols);

/* The damping and factorisation steps of clha_gptq_quantize on their own (GPTQ's
 * "Cholesky of H^-1"), for inspection: for each of the n Hessians H[i],
 *   dead columns (H_ii == 0) get H_ii := 1; lambda = damp * mean(diag H);
 *   U = upper Cholesky factor of (H + lambda I)^-1.
 *   H          host array of n device pointers, each float [cols][cols] symmetric
 *   U_out      device float [n][cols][cols]; only the upper triangle (with the
 *              diagonal) is written
 *   lambda_out device float [n] (may be NULL); dead_out device uint8 [n][cols] (may be NULL)
 *   cols       multiple of 64, <= 8192
 * Errors: INVALID_ARG, SHAPE, ALIGN, WORKSPACE; NOT_PD is latched as in clha_gptq_quantize. */
CLHA_API clha_status clha_inverse_cholesky(clha_ctx* ctx, int32_t n, const float* const* H,
                                           int32_t cols, float damp, float* U_out,
                                           float* lambda_out, uint8_t* dead_out,
                                           void* workspace, size_t workspace_bytes, void* stream);

/* Device workspace bytes clha_loss needs. */
CLHA_API size_t clha_loss_workspace_bytes(const clha_ctx* ctx, int32_t rows, int32_t cols);

/* Reconstruction loss of a quantized matrix under any Hessian, computed directly:
 *   loss = sum_r (Wq_r - W_r) H (Wq_r - W_r)^T,  Wq = s (q - z) per group
 * (the objective of section 2.1 for one layer term; with H = H_a or H_b it is the
 * per-layer calibration error of a shared weight).
 *   W device [rows][cols] (w_dtype); codes/scales/zeros as produced by clha_gptq_quantize;
 *   H device float [cols][cols] symmetric; loss_out device float [1].
 * Errors: INVALID_ARG, SHAPE, ALIGN, WORKSPACE. */
CLHA_API clha_status clha_loss(clha_ctx* ctx, int32_t rows, int32_t cols, int32_t group,
                               const void* W, int32_t w_dtype, const uint8_t* codes,
                               const float* scales, const uint8_t* zeros, const float* H,
                               float* loss_out, void* workspace, size_t workspace_bytes,
                               void* stream);

/* clha_loss for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same loss, computed by the same
 * kernels, with the tile partials in a static scratch array of the library (1 MiB per device,
 * held until the process ends) instead of a workspace.  The call allocates nothing.
 *   sizes: ceil(rows/64) * (cols/64) must be at most 131072 (e.g. rows <= 65536 at
 *          cols 8192), else CLHA_ERR_WORKSPACE is returned and nothing is enqueued
 *   Every call on one device shares that device's scratch: calls that overlap on one
 *   device (e.g. on two streams) race; calls ordered on one stream do not.  The scratch
 *   needs no clearing: every partial is written before it is read.
 * Errors: as clha_loss, with WORKSPACE for sizes beyond the scratch. */
CLHA_API clha_status clha_loss_static(clha_ctx* ctx, int32_t rows, int32_t cols, int32_t group,
                                      const void* W, int32_t w_dtype, const uint8_t* codes,
                                      const float* scales, const uint8_t* zeros, const float* H,
                                      float* loss_out, void* stream);

/* Inputs of the experts' second matrix (down_proj).  Section 2.2 collects the Hessian
 * of every shared weight over that weight's own input; the input of an expert's
 * down_proj is its SwiGLU intermediate
 *   h = bf16( silu(x Wg^T) * (x Wu^T) ),  silu(g) = g / (1 + e^-g)
 * from the full-precision gate and up weights.  Each routed expert (over its routed
 * tokens) and each shared expert (over all tokens, with its own weights) has its own
 * down_proj Hessian, so these run on a separate "down_proj context":
 *   desc.d = f (intermediate size, multiple of 128), desc.n_routed = routed + shared
 *   experts (one slot each), desc.n_shared = 0, desc.top_k and max_tokens as the block's.
 * Its layers are registered, reset, aggregated and quantized like any other
 * (clha_register_layer, clha_aggregate, clha_gptq_quantize with cols = f).
 *   n_routed  the block's routed experts E: slots 0..E-1 are routed, E.. shared
 *   x         device bf16 bits [n_tokens][d_model], the layer's model-width activations
 *   token_ids, offsets  device, the routing of this batch on the block's main context
 *             (the token_ids_out / offsets_out of clha_collect_hessians: int32 [n*K],
 *             int64 [E+1])
 *   wgu       host array [slots] of device pointers, bf16 bits [2f][d_model] each:
 *             gate rows 0..f-1, up rows f..2f-1
 *   S[e] += h_e^T h_e (lower triangle) and counts[e] += n_e for the registered layer,
 *   stored instead of added by the first collection after clha_reset_layer.
 * Errors: INVALID_ARG (not a down_proj context, unregistered layer, null pointer),
 * SHAPE (d_model not a multiple of 64 or > 8192, n_routed, n_tokens), ALIGN, WORKSPACE.
 * n_tokens == 0 enqueues nothing and reads no pointer. */
CLHA_API size_t clha_down_workspace_bytes(const clha_ctx* ctx, int32_t n_routed);
CLHA_API clha_status clha_collect_down_hessians(clha_ctx* ctx, int32_t layer, int64_t n_tokens,
                                                int32_t d_model, int32_t n_routed, const uint16_t* x,
                                                const int32_t* token_ids, const int64_t* offsets,
                                                const uint16_t* const* wgu, void* workspace,
                                                size_t workspace_bytes, void* stream);

/* Packed storage of codes at b bits (section 2.3, CLHA-MP: routed experts at b bits,
 * shared ones at b+1).  Code j of the stream occupies bits j*b .. j*b+b-1 of a
 * little-endian bit stream (bit 0 = least significant bit of byte 0); n_codes codes
 * take n_codes*b/8 bytes.  A [rows][cols] code matrix with cols a multiple of 8 packs
 * row by row into [rows][cols*b/8].
 *   n_codes  multiple of 8, >= 0 (0 enqueues nothing and reads no pointer)
 *   bits     2..8; codes must lie in 0 .. 2^bits - 1 (GPTQ's codes do); higher bits
 *            of a code are dropped
 *   codes    device uint8 [n_codes], 16-byte aligned
 *   packed   device uint8 [n_codes*bits/8]
 * Errors: INVALID_ARG (null pointer), SHAPE (n_codes or bits), ALIGN, HIP. */
CLHA_API clha_status clha_pack_codes(clha_ctx* ctx, int64_t n_codes, int32_t bits, const uint8_t* codes,
                                     uint8_t* packed, void* stream);

/* The inverse of clha_pack_codes: codes[j] = bits j*b .. j*b+b-1 of the stream. */
CLHA_API clha_status clha_unpack_codes(clha_ctx* ctx, int64_t n_codes, int32_t bits, const uint8_t* packed,
                                       uint8_t* codes, void* stream);

/* Stages timed by the optional per-stage timers. */
typedef enum clha_stage {
  CLHA_STAGE_ROUTE = 0,      /* top-K routing kernel */
  CLHA_STAGE_BUCKET = 1,     /* histogram, scan and scatter kernels */
  CLHA_STAGE_GATHER = 2,     /* down_proj inputs: the grouped SwiGLU GEMM (clha_collect_down_hessians) */
  CLHA_STAGE_SYRK = 3,       /* Gram-sum kernel (one launch per collect call) */
  CLHA_STAGE_AGGREGATE = 4,  /* aggregation kernel */
  CLHA_STAGE_FACTOR = 5,     /* damping, Cholesky and triangular inverse (clha_inverse_cholesky) */
  CLHA_STAGE_GPTQ = 6,       /* clha_gptq_quantize: factorisation and GPTQ, which overlap */
  CLHA_STAGE_LOSS = 7,       /* explicit loss kernels */
  CLHA_STAGE_SYRK_REDUCE = 8, /* Gram sums: partial sums of token-split slots into S, empty slots zeroed */
  CLHA_NUM_STAGES = 9
} clha_stage;

/* Enables (1) or disables (0) per-stage timing: each stage of each later call records a
 * pair of hipEvents on the call's stream around its kernels.  Off by default. */
CLHA_API clha_status clha_set_timing(clha_ctx* ctx, int32_t enable);

/* Waits for every recorded event pair, adds the elapsed milliseconds of stage s to
 * ms_out[s] and the number of recorded calls to calls_out[s] (host arrays of n entries,
 * n <= CLHA_NUM_STAGES; either may be NULL), then forgets the records. */
CLHA_API clha_status clha_read_timing(clha_ctx* ctx, double* ms_out, int64_t* calls_out, int32_t n);

/* Waits for `stream`, then returns and clears the latched device errors: NONFINITE (a router
 * logit, naming the first layer that had one; or a Hessian's diagonal) before NOT_PD, or
 * CLHA_OK.  clha_last_error names the lowest failing GPTQ job index and Hessian index of the
 * calls since the last clha_sync (Hessians numbered in order of first use within a call). */
CLHA_API clha_status clha_sync(clha_ctx* ctx, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CLHA_H */
