/*
 * gsq.h -- C ABI of the GSQ relaxed-quantization step on AMD MI355X (gfx950).
 *
 * The method (paper "GSQ: Highly-Accurate Low-Precision Scalar Quantization for
 * LLMs via Gumbel-Softmax Sampling"): every weight coordinate of a linear layer
 * W [rows x cols] carries learnable logits over a symmetric scalar grid with one
 * scale per group of 128 consecutive in-features; a Gumbel-Softmax sample of
 * the logits at temperature tau gives a soft weight; the layer's output
 * reconstruction error on calibration activations is minimised over the logits
 * and the group scales with Lion while tau is annealed; the logits are then
 * collapsed to hard codes that existing scalar kernels consume
 * (agihunt.info summary: idea, method and optimizer paragraphs; atlas.scime.ai
 * summary: Approach; thelatestinai.com abstract).
 *
 * One optimisation step is four calls, in this order, on one stream:
 *   gsq_relax_fwd        soft weights -> dW = W_soft - W (bf16)
 *   gsq_recon_loss_grad  R = X dW^T, loss = sum R^2, G = 2 R^T X
 *   gsq_relax_bwd_lion   dLoss/dlogits, dLoss/dscales, Lion on both, in place
 * and, once after the last step,
 *   gsq_harden_pack      argmax codes, packed bit-stream, fp16 scales.
 * gsq_relax_bwd_lion_fwd fuses a step's backward + Lion with the next step's
 * forward (same results, one pass over the logits).
 *
 * Conventions for every call:
 *  - Pointers named as tensors are DEVICE pointers, allocated and owned by the
 *    caller; the library allocates and frees no memory and keeps no mutable
 *    global state, except the static scratch array of
 *    gsq_recon_loss_grad_noalloc and the per-device table of its address.
 *    Host pointers are marked "host".
 *  - Device tensors must be 16-byte aligned (GSQ_ERR_ALIGN otherwise).
 *  - Layouts are row-major. Logits and their Lion momentum are planar
 *    [L][rows][cols] fp32 (plane k holds logit k of every coordinate), with
 *    L = 4 (2-bit), 2 (ternary: plane 0 mask, plane 1 sign), 5 (3-bit local
 *    shift: planes for offsets -2..+2), 8 (full 3-bit grid). Scales and their momentum are
 *    [rows][cols/128] fp32. bf16 and fp16 tensors are passed as uint16_t bits.
 *  - All arguments are checked before anything is launched; a failed check
 *    returns its status and launches nothing. A HIP launch error returns
 *    GSQ_ERR_HIP. Work is asynchronous and ordered on `stream` (a hipStream_t,
 *    NULL for the default stream). Calls on distinct streams are thread-safe
 *    when their output tensors do not overlap.
 *  - Noise is counter-based Philox4x32-10 (Salmon et al., SC'11), so the
 *    forward and backward of one step regenerate identical noise and a step is
 *    a pure function of (seed, stream id, step, inputs). Coordinate
 *    i = row*cols + col uses stream elements e = i*L + k (k = 0..L-1); element
 *    e is word (e & 3) of the block with counter (lo32(e>>2), hi32(e>>2),
 *    step, stream id) and key (lo32(seed), hi32(seed)); its uniform is
 *    ((word >> 8) | 1) * 2^-24.
 */
#ifndef GSQ_H_
#define GSQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GSQ_ABI_VERSION 1

typedef enum {
    GSQ_OK = 0,
    GSQ_ERR_NULL = 1,   /* a required pointer is NULL */
    GSQ_ERR_SHAPE = 2,  /* a size is out of range or not a required multiple */
    GSQ_ERR_ALIGN = 3,  /* a device tensor is not 16-byte aligned */
    GSQ_ERR_GRID = 4,   /* unknown grid, or a grid-specific argument missing */
    GSQ_ERR_PARAM = 5,  /* a scalar is out of range (tau, noise scale, Lion) */
    GSQ_ERR_HIP = 6,    /* the HIP runtime reported an error at launch */
    GSQ_ERR_SCRATCH = 7 /* gsq_recon_loss_grad_noalloc: the call needs more than
                           the library's static scratch array holds */
} gsq_status;

/* Grids (agihunt.info summary, method paragraph). Values in scale units:
 *  INT2        4 levels {-3,-1,1,3}, 4 logits per coordinate;
 *  TERNARY     {-1,0,1} as a binary mask times a binary sign, 2 logits;
 *  INT3_LOCAL  8 levels {-7,-5,...,7}; 5 logits for the codes
 *              clamp(c0 + d, 0, 7), d = -2..2, around a warm-start code c0;
 *  INT3        the same 8 levels with one logit each (8 logits): the full
 *              grid that local shift stands in for. */
typedef enum {
    GSQ_GRID_INT2 = 0,
    GSQ_GRID_TERNARY = 1,
    GSQ_GRID_INT3_LOCAL = 2,
    GSQ_GRID_INT3 = 3
} gsq_grid;

typedef enum { GSQ_DTYPE_F32 = 0, GSQ_DTYPE_BF16 = 1 } gsq_dtype;

/* One layer being quantised. */
typedef struct {
    int32_t grid;      /* gsq_grid */
    int32_t group;     /* scale group size along cols; must be 128 */
    int64_t rows;      /* out features M (> 0) */
    int64_t cols;      /* in features K (> 0, multiple of 128) */
    int32_t w_dtype;   /* gsq_dtype of W */
    uint32_t stream;   /* noise stream id (e.g. a layer index) */
    uint64_t seed;     /* noise key */
} gsq_layer;

/* Lion hyper-parameters (Chen et al. 2023; the pages pick Lion for the logits:
 * agihunt.info optimizer paragraph). For each parameter theta with gradient g
 * and momentum m: c = beta1*m + (1-beta1)*g; theta -= lr*(sign(c) + wd*theta);
 * m = beta2*m + (1-beta2)*g. Logits use lr_logit, scales lr_scale. */
typedef struct {
    float lr_logit;
    float lr_scale;
    float beta1;        /* in [0, 1) */
    float beta2;        /* in [0, 1) */
    float weight_decay; /* >= 0 */
} gsq_lion;

/* ABI version of the loaded library (GSQ_ABI_VERSION). */
int gsq_abi_version(void);

/* Static, NUL-terminated name of a status code. */
const char* gsq_status_str(int status);

/* Number of logits per coordinate of a grid (4, 2, 5, 8), or 0 if unknown. */
int gsq_num_logits(int grid);

/* Warm start by round-to-nearest (the pages start from GPTQ or a GGUF
 * K-Quant, agihunt.info optimizer paragraph; the solve itself only needs codes
 * and scales). Per group: s = maxabs / q_max (q_max = 3, 1, 7), a correctly
 * rounded fp32 division; x = w / s (0 if s = 0); codes: 2-bit and 3-bit
 * c0 = clamp(rint((x + q_max) * 0.5), 0, 2^b - 1), ternary t0 + 1 with
 * t0 = clamp(rint(x), -1, 1) (rint: ties to even). Logits: init_logit on the
 * warm-start level and 0 elsewhere (local shift: plane 2, offset 0); ternary
 * mask = +init_logit if t0 != 0 else -init_logit, sign = +init_logit if w >= 0
 * else -init_logit.
 *   W       [rows][cols] in layer->w_dtype
 *   scales  out [rows][cols/128] fp32
 *   codes   out [rows][cols] uint8 (warm-start codes; INT3_LOCAL needs them
 *           at every later call)
 *   logits  out [L][rows][cols] fp32
 * Momenta are not touched: the caller zeroes them. */
gsq_status gsq_init_rtn(const gsq_layer* layer, const void* W, float* scales,
                        uint8_t* codes, float* logits, float init_logit,
                        void* stream);

/* Workspace bytes of gsq_init_gptq for a layer of rows x cols: the fp32 Gram
 * matrix, one fp64 cols x cols factor, the fp64 error feedback of the whole
 * layer and one 128-column block of rounding errors (about 12*cols^2 +
 * 8*rows*cols bytes). 0 for invalid sizes. */
size_t gsq_gptq_workspace_bytes(int64_t rows, int64_t cols);

/* GPTQ warm start (Frantar et al. 2022), the initialisation the pages start
 * from (agihunt.info optimizer paragraph; atlas.scime.ai Approach), in place
 * of gsq_init_rtn: the same absmax group scales (GPTQ's static groups), then
 * codes chosen column by column with every rounding error fed into the later
 * columns through H = X^T X + damp * mean(diag H) * I (a zero diagonal entry
 * counts as 1), and logits set from the codes as gsq_init_rtn sets them.
 *   W          [rows][cols] in layer->w_dtype
 *   tokens     calibration tokens T (> 0, multiple of 64; zero rows pad)
 *   XT         [cols][T] bf16 (gsq_transpose_tokens with one expert)
 *   damp       >= 0 (GPTQ uses 0.01)
 *   workspace  device scratch of at least gsq_gptq_workspace_bytes()
 *   scales, codes, logits  out, as gsq_init_rtn
 *   info       out device int32: 0, or j+1 when the damped Gram matrix was
 *              not positive definite at (reversed) column j; read it after the
 *              stream has finished. */
gsq_status gsq_init_gptq(const gsq_layer* layer, const void* W, int64_t tokens,
                         const uint16_t* XT, float damp, float init_logit,
                         void* workspace, size_t workspace_bytes, float* scales,
                         uint8_t* codes, float* logits, int32_t* info,
                         void* stream);

/* ---------------------------------------------------------------------------
 * Block forward pieces for the staged schedule: the pages optimise a decoder
 * block in stages (query/key, then value/output, then the MLP on the block
 * output), each stage's calibration inputs computed from the block with the
 * earlier stages quantized and frozen (agihunt.info optimizer paragraph).
 * bf16 tensors in and out, fp32 arithmetic, row-major; device pointers owned
 * by the caller, 16-byte aligned.
 * ------------------------------------------------------------------------- */

/* C[i][j] = sum_r A[i][r] B[j][r] (bf16 operands, fp32 accumulation, bf16
 * result, round to nearest even). Rd a multiple of 64; lda, ldb >= Rd and
 * ldc >= J, all leading dimensions and J multiples of 8 elements. */
gsq_status gsq_matmul_nt_bf16(int64_t I, int64_t J, int64_t Rd, const uint16_t* A,
                              int64_t lda, const uint16_t* B, int64_t ldb,
                              uint16_t* C, int64_t ldc, void* stream);

/* y = x / sqrt(mean_j x^2 + eps) * gamma per row; x, y [rows][cols] bf16,
 * gamma [cols] fp32, eps > 0. */
gsq_status gsq_rmsnorm_bf16(int64_t rows, int64_t cols, const uint16_t* x,
                            const float* gamma, float eps, uint16_t* y, void* stream);

/* P[i][j] = softmax over j <= i of scale * S[i][j] (causal), 0 for j > i;
 * S, P [n][n] bf16. */
gsq_status gsq_softmax_causal_bf16(int64_t n, const uint16_t* S, float scale,
                                   uint16_t* P, void* stream);

/* act = silu(gate) * up elementwise (SwiGLU), n elements. */
gsq_status gsq_silu_mul_bf16(int64_t n, const uint16_t* gate, const uint16_t* up,
                             uint16_t* act, void* stream);

/* out = a + b elementwise (residual), n elements. */
gsq_status gsq_add_bf16(int64_t n, const uint16_t* a, const uint16_t* b,
                        uint16_t* out, void* stream);

/* out = a - b elementwise, n elements (the offsets of the staged schedule). */
gsq_status gsq_sub_bf16(int64_t n, const uint16_t* a, const uint16_t* b, uint16_t* out,
                        void* stream);

/* Hard weights W = s * v(code) in bf16 from gsq_harden_pack's codes (uint8
 * [rows][cols]) and fp16 scales ([rows][cols/128]); v as in gsq_harden_pack
 * (ternary codes are t + 1; local-shift codes are final 3-bit codes). */
gsq_status gsq_dequant_bf16(const gsq_layer* layer, const uint8_t* codes,
                            const uint16_t* scales_f16, uint16_t* W, void* stream);

/* Relaxed forward (agihunt.info method paragraph: soft weighted sum of grid
 * points). With noise n_k drawn for `step` and eta = noise_scale:
 *   2-bit / 3-bit (local shift or full grid): p = softmax((l + eta*g)/tau),
 *                        g standard Gumbel,
 *                        w_hat = sum_k p_k v_k;
 *   ternary: a = sigmoid((l_m + eta*n_m)/tau), b = sigmoid((l_s + eta*n_s)/tau),
 *            n standard logistic, w_hat = a * (2b - 1);
 *   w_soft = s * w_hat;  dW = w_soft - W, rounded to bf16 (nearest even).
 *   logits      [L][rows][cols] fp32
 *   scales      [rows][cols/128] fp32
 *   init_codes  [rows][cols] uint8, required for INT3_LOCAL, else ignored
 *   W           [rows][cols] in layer->w_dtype
 *   dW_bf16     out [rows][cols] bf16
 *   w_soft_dbg  optional out [rows][cols] fp32 (NULL to skip)
 * tau must be finite and > 0; noise_scale in [0, 1]. */
gsq_status gsq_relax_fwd(const gsq_layer* layer, const float* logits,
                         const float* scales, const uint8_t* init_codes,
                         const void* W, uint32_t step, float tau,
                         float noise_scale, uint16_t* dW_bf16,
                         float* w_soft_dbg, void* stream);

/* Workspace bytes gsq_recon_loss_grad needs (loss partials), for E experts
 * whose token blocks are given by tok_offsets (host, E+1 entries). */
size_t gsq_recon_workspace_bytes(int32_t n_experts, const int64_t* tok_offsets,
                                 int64_t rows_per_expert, int64_t cols);

/* Output reconstruction objective on calibration activations (agihunt.info
 * method paragraph) and its gradient, for one layer (n_experts = 1) or for a
 * batch of experts that each see their own routed tokens:
 *   R_e = X_e dW_e^T,  loss = sum_e sum R_e^2 = sum_e ||X_e W_soft_e^T - X_e W_e^T||^2,
 *   G_e = dLoss/d(dW_e) = 2 R_e^T X_e.
 * bf16 operands, fp32 accumulation on the matrix cores.
 *   tok_offsets   host [E+1], tok_offsets[0] = 0, non-decreasing, every entry a
 *                 multiple of 64 (pad token blocks with zero rows: a zero token
 *                 adds nothing to loss or gradient)
 *   rows_per_expert  rows of dW owned by each expert (the layer's rows if E = 1)
 *   cols          in features (multiple of 128)
 *   X             [T][cols] bf16, T = tok_offsets[E]
 *   XT            [cols][T] bf16 laid out per expert: block e is X_e^T
 *                 [cols][n_e] row-major at element offset cols*tok_offsets[e]
 *                 (gsq_transpose_tokens builds it)
 *   dW_bf16       [E*rows_per_expert][cols] bf16
 *   workspace     device scratch of at least gsq_recon_workspace_bytes()
 *   RT            out, block e is R_e^T [rows_per_expert][n_e] bf16 at element
 *                 offset rows_per_expert*tok_offsets[e]
 *   G             out [E*rows_per_expert][cols] fp32
 *   loss          out device scalar, fp64 (deterministic fixed-order sum) */
gsq_status gsq_recon_loss_grad(int32_t n_experts, const int64_t* tok_offsets,
                               int64_t rows_per_expert, int64_t cols,
                               const uint16_t* X, const uint16_t* XT,
                               const uint16_t* dW_bf16, void* workspace,
                               size_t workspace_bytes, uint16_t* RT, float* G,
                               double* loss, void* stream);

/* gsq_recon_loss_grad without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). Same arguments, results and
 * kernels as gsq_recon_loss_grad (bit-identical), with the loss partials in
 * a static device array of the library instead of a caller workspace:
 *  - Limit: 65536 fp32 partials (256 KiB), one per workgroup of the first
 *    product: sum over experts with tokens of ceil(rows_per_expert/256) *
 *    ceil(n_e/256) (a single layer whose last round of tiles is split may
 *    use up to twice that). A call that needs more returns GSQ_ERR_SCRATCH
 *    and launches nothing; use gsq_recon_loss_grad then.
 *  - Each device holds its own copy of the array until the process ends; the
 *    library looks up its address on the first call on a device (the
 *    current device, which must be the device of `stream`) and keeps it.
 *    That first call may return GSQ_ERR_HIP if the lookup fails.
 *  - The call allocates nothing and needs no clearing (every partial is
 *    written before it is read within the call).
 *  - Calls that overlap in time on one device (on different streams) share
 *    the array and race; serialise them (one stream, or events). */
gsq_status gsq_recon_loss_grad_noalloc(int32_t n_experts, const int64_t* tok_offsets,
                                       int64_t rows_per_expert, int64_t cols,
                                       const uint16_t* X, const uint16_t* XT,
                                       const uint16_t* dW_bf16, uint16_t* RT, float* G,
                                       double* loss, void* stream);

/* The objective and its gradient split differently, so that the second
 * product can be fused with the backward (agihunt.info summary, method
 * paragraph: the gradient of the output reconstruction error drives the
 * logits and scales). gsq_recon_residual followed by gsq_recon_bwd_lion_fwd
 * reproduces gsq_recon_loss_grad followed by gsq_relax_bwd_lion_fwd (or, with
 * with_next = 0, gsq_relax_bwd_lion) bit for bit (R^T, loss, logits, momenta,
 * scales, scale momenta, next dW), but G = 2 R^T X is formed tile by tile on
 * the matrix cores and consumed where it is formed, never stored: 8 bytes
 * per weight per step less HBM traffic. It pays where the second product is
 * bound by storing G, i.e. few tokens per expert; for a dense layer with
 * thousands of tokens the separate, MFMA-tuned product is faster.
 *
 * gsq_recon_residual: the first product alone, R_e^T = dW_e X_e^T (bf16) for
 * every expert, and the loss partials (sums of R^2, one per workgroup) in
 * `workspace`. Arguments as gsq_recon_loss_grad. */
gsq_status gsq_recon_residual(int32_t n_experts, const int64_t* tok_offsets,
                              int64_t rows_per_expert, int64_t cols, const uint16_t* X,
                              const uint16_t* dW_bf16, void* workspace, size_t workspace_bytes,
                              uint16_t* RT, void* stream);

/* The second product fused with backward + Lion and, with with_next = 1, the
 * next step's forward; the loss is summed from the partials the preceding
 * gsq_recon_residual left in `workspace` (same experts and token offsets,
 * same stream).
 *   layer         the whole layer (rows = n_experts * rows per expert)
 *   n_experts, tok_offsets, XT, RT, loss
 *                 as gsq_recon_loss_grad (the total token count must be below
 *                 2^31)
 *   workspace     the workspace gsq_recon_residual filled (read only)
 *   logits, mom, scales, scale_mom, init_codes, step, tau, noise_scale, lion
 *                 as gsq_relax_bwd_lion (no debug outputs)
 *   with_next     1: then the forward of next_step at next_tau on the updated
 *                 state into dW_bf16 (W and dW_bf16 needed), as
 *                 gsq_relax_bwd_lion_fwd; 0: backward + Lion only (the last
 *                 step); W, next_tau and dW_bf16 are then ignored */
gsq_status gsq_recon_bwd_lion_fwd(const gsq_layer* layer, int32_t n_experts,
                                  const int64_t* tok_offsets, const uint16_t* XT,
                                  const uint16_t* RT, const void* workspace,
                                  size_t workspace_bytes, double* loss, float* logits, float* mom,
                                  float* scales, float* scale_mom, const uint8_t* init_codes,
                                  const void* W, uint32_t step, float tau, float noise_scale,
                                  const gsq_lion* lion, int32_t with_next, uint32_t next_step,
                                  float next_tau, uint16_t* dW_bf16, void* stream);

/* The objective of one dense layer fitted to a target downstream of itself:
 * R = X dW^T + E0 with E0 fixed, loss = sum R^2, G = 2 R^T X. With
 * E0 = X W^T - Y the loss is ||X W_soft^T - Y||^2: the staged schedule
 * (agihunt.info summary, optimizer paragraph) fits the output projection to
 * the full-precision attention output and the MLP's last projection to the
 * full-precision block output this way. E0 enters the first product's
 * epilogue (one fp32 add before the square and the bf16 rounding of R^T).
 *   rows, cols, tokens  the layer and its calibration tokens (tokens > 0, a
 *                 multiple of 64; cols a multiple of 128)
 *   X, XT, dW_bf16, workspace, RT, G, loss
 *                 as gsq_recon_loss_grad with one expert
 *                 (workspace of gsq_recon_workspace_bytes(1, {0, tokens}, ...))
 *   E0T           [rows][tokens] bf16, E0 transposed (the layout of R^T) */
gsq_status gsq_recon_loss_grad_offset(int64_t rows, int64_t cols, int64_t tokens,
                                      const uint16_t* X, const uint16_t* XT,
                                      const uint16_t* dW_bf16, const uint16_t* E0T,
                                      void* workspace, size_t workspace_bytes, uint16_t* RT,
                                      float* G, double* loss, void* stream);

/* Per-expert transpose of the calibration tokens: XT block e = X_e^T (see
 * gsq_recon_loss_grad for the layout). Done once per layer. */
gsq_status gsq_transpose_tokens(int32_t n_experts, const int64_t* tok_offsets,
                                int64_t cols, const uint16_t* X, uint16_t* XT,
                                void* stream);

/* Gram form of the same objective, for one dense layer. The reconstruction
 * error is a quadratic form in dW, ||X dW^T||^2 = tr(dW H dW^T) with
 * H = X^T X (agihunt.info method paragraph: the objective is the output
 * reconstruction error), so H, formed once per layer, replaces X in every
 * step: one product of 2*rows*cols^2 flops instead of two of
 * 2*rows*tokens*cols, fewer when cols < 2*tokens.
 *
 * gsq_gram: H = X^T X, fp32 accumulation, rounded to bf16 (nearest even).
 *   tokens  T, a multiple of 64 (zero rows pad it)
 *   cols    in features (multiple of 128)
 *   XT      [cols][T] bf16 (gsq_transpose_tokens with one expert)
 *   H       out [cols][cols] bf16 (symmetric) */
gsq_status gsq_gram(int64_t tokens, int64_t cols, const uint16_t* XT, uint16_t* H,
                    void* stream);

/* Workspace bytes gsq_recon_gram needs (loss partials). */
size_t gsq_recon_gram_workspace_bytes(int64_t rows, int64_t cols);

/* P = dW H (bf16 operands, fp32 accumulation), G = 2 P, loss = sum dW * P
 * (equal to gsq_recon_loss_grad's loss and G up to rounding, with the bf16
 * rounding of H in place of that of R).
 *   H          [cols][cols] bf16 from gsq_gram
 *   dW_bf16    [rows][cols] bf16
 *   workspace  device scratch of at least gsq_recon_gram_workspace_bytes()
 *   G          out [rows][cols] fp32
 *   loss       out device scalar, fp64 (deterministic fixed-order sum) */
gsq_status gsq_recon_gram(int64_t rows, int64_t cols, const uint16_t* H,
                          const uint16_t* dW_bf16, void* workspace,
                          size_t workspace_bytes, float* G, double* loss,
                          void* stream);

/* Relaxed backward and Lion, in place (agihunt.info method and optimizer
 * paragraphs). Regenerates the step's noise (same `step`, `tau` and
 * `noise_scale` as the forward) and, with G = dLoss/dW_soft:
 *   2-bit / 3-bit: dL/dl_k = G * s * p_k * (v_k - w_hat) / tau;
 *   ternary: dL/dl_m = G * s * a(1-a)(2b-1) / tau, dL/dl_s = G * s * 2a b(1-b) / tau;
 *   dL/ds_g = sum over the 128 coordinates of the group of G * w_hat;
 * then one Lion update of every logit and every scale with its momentum,
 * taking sign(c) of c = fma(beta1, m, fp32((1-beta1)*g)).
 *   G                [rows][cols] fp32
 *   logits, mom      in/out [L][rows][cols] fp32
 *   scales, scale_mom in/out [rows][cols/128] fp32
 *   init_codes       [rows][cols] uint8 for INT3_LOCAL, else ignored
 *   grad_logits_dbg  optional out [L][rows][cols] fp32, gradient before Lion
 *   grad_scales_dbg  optional out [rows][cols/128] fp32; give both debug
 *                    outputs or neither (GSQ_ERR_NULL otherwise) */
gsq_status gsq_relax_bwd_lion(const gsq_layer* layer, const float* G,
                              float* logits, float* mom, float* scales,
                              float* scale_mom, const uint8_t* init_codes,
                              uint32_t step, float tau, float noise_scale,
                              const gsq_lion* lion, float* grad_logits_dbg,
                              float* grad_scales_dbg, void* stream);

/* Backward + Lion of step `step` followed by the relaxed forward of step
 * `next_step` (temperature `next_tau`) on the updated logits and scales, in
 * one pass over the layer. The results equal gsq_relax_bwd_lion(step, tau)
 * followed by gsq_relax_fwd(next_step, next_tau, w_soft_dbg = NULL) bit for
 * bit; the logits are read once instead of twice per step. Arguments as in
 * those two calls (no debug outputs); noise_scale applies to both steps.
 *   W        [rows][cols] in layer->w_dtype
 *   dW_bf16  out [rows][cols] bf16, the next step's W_soft - W */
gsq_status gsq_relax_bwd_lion_fwd(const gsq_layer* layer, const float* G, float* logits,
                                  float* mom, float* scales, float* scale_mom,
                                  const uint8_t* init_codes, const void* W, uint32_t step,
                                  float tau, float noise_scale, const gsq_lion* lion,
                                  uint32_t next_step, float next_tau, uint16_t* dW_bf16,
                                  void* stream);

/* Collapse to hard codes after annealing (agihunt.info method paragraph) in
 * the symmetric group-128 format with 16-bit scales (takeaway paragraph;
 * the 2.13 / 3.13 / 1.71 bits per parameter of the results table).
 *   codes: 2-bit and full 3-bit argmax_k l_k (first index on ties); local
 *   shift clamp(c0 + argmax - 2, 0, 7); ternary t + 1,
 *   t = [l_m >= 0]*(l_s >= 0 ? 1 : -1).
 *   codes       optional out [rows][cols] uint8
 *   packed      optional out [rows][cols*b/32] uint32, b = 2 (2-bit,
 *               ternary) or 3 (3-bit); per
 *               row a little-endian LSB-first bit-stream, code j in bits
 *               [b*j, b*j + b)
 *   scales_f16  optional out [rows][cols/128] fp16 bits (nearest even) */
gsq_status gsq_harden_pack(const gsq_layer* layer, const float* logits,
                           const float* scales, const uint8_t* init_codes,
                           uint8_t* codes, uint32_t* packed,
                           uint16_t* scales_f16, void* stream);

/* Raw Philox words of the noise stream of `step`: out[j] = element first + j
 * (layout above). For checking the generator. */
gsq_status gsq_noise_dump(const gsq_layer* layer, uint32_t step, int64_t first,
                          int64_t count, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GSQ_H_ */
