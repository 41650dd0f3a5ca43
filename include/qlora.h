/*
 * qlora.h -- C ABI of the QLoRA linear layer for MI355X (gfx950).
 *
 * The method (the "qlora" encyclopedia entry on tonho.wtf, sections "a ideia"
 * and "como funciona"; the LoRA formula from the nexusinovation tutorial
 * "Tutorial fine-tuning LLM LoRA/QLoRA", section "LoRA: O Padrão Ouro de
 * Eficiência"):
 *   - a frozen base weight W [n_out x n_in] is stored in a 4-bit type (NF4)
 *     built from standard-normal quantiles, normalised to [-1, 1] by the
 *     absolute maximum of each 64-element block, with an exact zero;
 *   - the per-block constants are quantized again, to FP8 (e4m3) in groups of
 *     256, with one fp32 scale per group and one fp32 mean per tensor
 *     (double quantization: 4.127 bits per parameter in total);
 *   - every use of the weight dequantizes it to BFloat16 inside the matrix
 *     product; a 16-bit LoRA adapter path is added, W' = W + s.B.A with
 *     A [r x n_in] and B [n_out x r];
 *   - the backward pass sends the gradient through the frozen weight into the
 *     adapters only (grad_x, grad_A, grad_B; never a gradient for W).
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers (memory the caller allocated on the
 *     current HIP device), 16-byte aligned, row-major and densely packed.
 *     bf16 tensors are passed as uint16_t bit patterns.
 *   - The caller owns every buffer, including the workspace.  The library
 *     allocates and frees no device memory.  Its only mutable global state is
 *     the timing diagnostics (qlora_kernel_timing_*, not thread-safe) and the
 *     per-device scratch array of qlora_linear_fwd_noalloc (with the cache of
 *     its device addresses).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls validate
 *     their arguments on the host, enqueue kernels on `stream` and return
 *     without waiting.  Buffers must stay alive until the stream has run the
 *     work.  Calls on different streams are independent; two calls that share
 *     a workspace must be ordered by the caller.
 *   - Host-checkable problems return a non-zero qlora_status BEFORE anything
 *     is enqueued.  A launch failure returns QLORA_ERR_HIP.  Data-dependent
 *     problems (a NaN or Inf in the weight given to qlora_quantize) set a flag
 *     in the workspace that qlora_status_read reports.  Nothing throws.
 *   - Outputs are overwritten, never accumulated into.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = 1,       /* a required pointer is NULL                          */
  QLORA_ERR_SHAPE = 2,      /* a dimension is out of range (see each call)          */
  QLORA_ERR_ALIGN = 3,      /* a pointer is not 16-byte aligned                     */
  QLORA_ERR_WORKSPACE = 4,  /* workspace smaller than the size helper returns      */
  QLORA_ERR_DTYPE = 5,      /* unknown dtype code                                   */
  QLORA_ERR_HIP = 6,        /* the HIP runtime reported an error at launch          */
  QLORA_ERR_NONFINITE = 7,  /* (deferred) NaN or Inf met while quantizing           */
  QLORA_ERR_VALUE = 8,      /* a scalar argument is not finite or out of range      */
  QLORA_ERR_MEMORY = 9,     /* a buffer is neither device nor pinned host memory    */
  QLORA_ERR_SCRATCH = 10    /* the call needs more than the fixed scratch array     */
} qlora_status;

typedef enum { QLORA_F32 = 0, QLORA_BF16 = 1 } qlora_dtype;

/* Packed NF4 weight.  All buffers are device memory owned by the caller.
 * Element e of the row-major [n_out x n_in] weight belongs to block e/64 and
 * to double-quantization group (e/64)/256; a partial last block or group is
 * zero padded.
 * flags = 0 (the default): double quantization, the four buffers below.
 * flags = QLORA_NF4_FP32_CONSTANTS: no double quantization ("qlora" entry,
 * section "como funciona": the fp32 constants cost 0.5 bit/param before
 * their FP8 stage); absmax_scale then holds nblocks fp32 block constants
 * c1_b themselves, decoded as c1hat_b = c1_b, and absmax_fp8 / absmax_mean
 * are unused (may be NULL): 4.5 bits per parameter.                          */
#define QLORA_NF4_FP32_CONSTANTS 1u
typedef struct {
  int64_t n_out;         /* rows of W (output features)                        */
  int64_t n_in;          /* columns of W (input features), contiguous          */
  uint8_t *codes;        /* ceil(numel/2) bytes: element 2i in the low nibble,
                            element 2i+1 in the high nibble; an odd tail's high
                            nibble is the zero code 7                           */
  uint8_t *absmax_fp8;   /* nblocks = ceil(numel/64) e4m3 bytes, q_b          */
  float *absmax_scale;   /* ngroups = ceil(nblocks/256) fp32 scales, s2_g
                            (nblocks fp32 constants c1_b with FP32_CONSTANTS) */
  float *absmax_mean;    /* 1 fp32, the mean mu of the block absmax values     */
  uint32_t flags;        /* 0 or QLORA_NF4_FP32_CONSTANTS; other bits are
                            rejected with QLORA_ERR_VALUE                       */
} qlora_nf4_weight;

/* ---- host-only helpers (no GPU needed) ----------------------------------- */

/* Sizes of the four buffers of a packed [n_out x n_in] weight; any out-pointer
 * may be NULL.  Returns QLORA_ERR_SHAPE for a non-positive dimension or more
 * than 2^37 elements.                                                          */
qlora_status qlora_nf4_sizes(int64_t n_out, int64_t n_in, int64_t *codes_bytes,
                             int64_t *nblocks, int64_t *ngroups);

/* Total bytes of the packed format (codes + constants + scales + mean): the
 * storage cost is 8 * this / numel bits per parameter.  0 on a bad shape.     */
size_t qlora_nf4_bytes(int64_t n_out, int64_t n_in);

/* The same total for a storage form chosen by `flags` (0: as qlora_nf4_bytes;
 * QLORA_NF4_FP32_CONSTANTS: codes + 4 * nblocks).  0 on a bad shape or flag. */
size_t qlora_nf4_bytes_flags(int64_t n_out, int64_t n_in, uint32_t flags);

/* Workspace bytes needed by qlora_quantize for a weight of this shape.        */
size_t qlora_quantize_workspace_bytes(int64_t n_out, int64_t n_in);

/* Workspace bytes needed by qlora_linear_fwd and qlora_linear_bwd for T
 * tokens, this weight shape and adapter rank r (one size covers both calls).
 * Its contents need no initialisation; calls that may overlap in time must
 * not share a workspace.                                                     */
size_t qlora_linear_workspace_bytes(int64_t T, int64_t n_out, int64_t n_in, int r);

/* The library's 16 NF4 levels (fp32, code k -> out[k]), computed on the host
 * from the definition: standard-normal quantiles at equal probability steps,
 * 8 positive and 7 negative levels plus an exact zero, divided by the largest
 * quantile; see "como funciona" in the qlora entry.                          */
void qlora_nf4_codebook(float out[16]);

const char *qlora_status_string(qlora_status s);

/* Library version string.                                                    */
const char *qlora_version(void);

/* ---- device calls (enqueue on `stream`) ---------------------------------- */

/* Quantize W (fp32 or bf16, [q->n_out x q->n_in], device) into *q: blockwise
 * NF4 with one absmax constant per 64 elements, the constants quantized again
 * to FP8 in groups of 256 ("qlora" entry, section "como funciona"):
 *   c1_b  = max |x| over block b (exact);
 *   code  = index of the NF4 level nearest to the exact real x / c1_b, ties
 *           toward the level of smaller magnitude (c1_b = 0 gives code 7);
 *   mu    = fp32 round-to-nearest of the exact mean of all c1_b;
 *   per group g: s2_g = fl32(max_b |fl32(c1_b - mu)| / 448) and
 *   q_b   = e4m3 nearest to the exact real fl32(c1_b - mu) / s2_g (ties to
 *           the even mantissa, saturating at 448; q_b = 0 when s2_g = 0).
 * With q->flags = QLORA_NF4_FP32_CONSTANTS the mean and FP8 stages are
 * skipped and c1_b is written to absmax_scale[b] as it is.
 * Any numel up to 2^37 is accepted.  ws: qlora_quantize_workspace_bytes, 16-B
 * aligned; after the call it holds the status word read by qlora_status_read.
 * A NaN/Inf in W raises QLORA_ERR_NONFINITE there; that block's codes are
 * then unspecified.                                                           */
qlora_status qlora_quantize(const void *w, qlora_dtype w_dtype, const qlora_nf4_weight *q,
                            void *ws, size_t ws_bytes, void *stream);

/* Dequantize *q to bf16 w_bf16 [n_out x n_in] (device), the decode that every
 * use of the weight applies ("qlora" entry, section "a ideia": the 4-bit
 * weight is dequantized to BFloat16 when it is used):
 *   c1hat_b = fl32(fl32(e4m3(q_b) * s2_g) + mu)     (no fused multiply-add;
 *             c1hat_b = c1_b with QLORA_NF4_FP32_CONSTANTS)
 *   w_hat   = bf16_round_nearest_even(fl32(CB[code] * c1hat_b))
 * This is the same decode the fused linear calls apply on the fly.           */
qlora_status qlora_dequantize(const qlora_nf4_weight *q, uint16_t *w_bf16, void *stream);

/* The same decode for count = 1..8 weights in one launch (for instance the
 * seven linears of a decoder layer, streamed back to bf16 layer by layer, the
 * 16-bit copy existing only for the layer in use: "qlora" entry, section
 * "a ideia").  q[i] -> w_bf16[i]; either storage form, mixed freely.         */
qlora_status qlora_dequantize_many(const qlora_nf4_weight *q, int count, uint16_t *const *w_bf16,
                                   void *stream);

/* Forward of the adapted linear layer for T tokens: the 4-bit weight decoded
 * to BFloat16 inside the product ("qlora" entry, section "a ideia") plus the
 * LoRA path W' = W + s.B.A (nexusinovation tutorial, section "LoRA: O Padrão
 * Ouro de Eficiência"):
 *   u = x A^T                      (bf16, [T x r]; written to u_out if non-NULL)
 *   y = bf16( x W_hat^T + scale * u B^T )          [T x n_out]
 * x [T x n_in] bf16, A [r x n_in] bf16, B [n_out x r] bf16, all device.
 * Requires n_in % 64 == 0, T >= 1, 1 <= r <= 256, finite scale.  W_hat is
 * never written to memory: it is decoded tile by tile inside the product.
 * ws: qlora_linear_workspace_bytes(T, n_out, n_in, r), 16-B aligned.        */
qlora_status qlora_linear_fwd(const uint16_t *x, int64_t T, const qlora_nf4_weight *q,
                              const uint16_t *A, const uint16_t *B, int r, float scale,
                              uint16_t *y, uint16_t *u_out, void *ws, size_t ws_bytes,
                              void *stream);

/* qlora_linear_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same computation, kernels, shape rules and
 * errors as qlora_linear_fwd (results bit-identical to it), plus
 * QLORA_ERR_SCRATCH, returned before anything is enqueued, when the call needs
 * more scratch than the library's fixed array holds (the partial sums of
 * u = x A^T, and u itself when u_out is NULL; qlora_linear_fwd_noalloc_max_bytes
 * gives the limit).  The array is a device global of the library: every GPU the
 * library runs on holds one copy of it until the process ends, and every call on
 * that GPU shares it, so two calls that may overlap in time on one GPU race
 * (order them on one stream).  Nothing in it has to start at zero: each call
 * writes every scratch value it reads.  The call allocates nothing and runs on
 * the current HIP device, which must be the one that owns `stream` and the
 * buffers.                                                                  */
size_t qlora_linear_fwd_noalloc_max_bytes(void);
qlora_status qlora_linear_fwd_noalloc(const uint16_t *x, int64_t T, const qlora_nf4_weight *q,
                                      const uint16_t *A, const uint16_t *B, int r, float scale,
                                      uint16_t *y, uint16_t *u_out, void *stream);

/* Backward of the adapted linear layer: the gradient passes through the
 * frozen 4-bit weight into the 16-bit adapters only ("qlora" entry, section
 * "a ideia"):
 *   v      = dy B                                   (bf16, internal)
 *   grad_x = bf16( dy W_hat + scale * v A )         [T x n_in]   (skipped if NULL)
 *   grad_A = scale * v^T x                          [r x n_in]   fp32
 *   grad_B = scale * dy^T u                         [n_out x r]  fp32
 * dy [T x n_out] bf16.  u is the forward's u_out; pass NULL to recompute it.
 * Same shape rules and workspace as qlora_linear_fwd.                         */
qlora_status qlora_linear_bwd(const uint16_t *dy, const uint16_t *x, int64_t T,
                              const qlora_nf4_weight *q, const uint16_t *A, const uint16_t *B,
                              int r, float scale, const uint16_t *u, uint16_t *grad_x,
                              float *grad_A, float *grad_B, void *ws, size_t ws_bytes,
                              void *stream);

/* ---- projection sets --------------------------------------------------------- */

/* The adapters go on every linear layer, not only on query and value ("qlora"
 * entry, section "como funciona"; "LoRA vs. QLoRA vs. Full Fine-Tuning",
 * section "Um LoRA Rank Mais Alto Sempre Melhora a Qualidade?"), so linears
 * that read the same input -- the attention projections q, k, v, or the
 * MLP's gate and up -- each carry an adapter.  A set runs them together:
 *   u_set = x A_set^T                      one adapter product for all members
 *   y_i   = bf16( x W_hat_i^T + scale * u_i B_i^T )     one fused GEMM launch
 *   grad_x = bf16( sum_i dy_i W_hat_i + scale * v_set A_set ),  v_i = dy_i B_i
 *                                          one GEMM over every member's rows
 *   grad_A_set = scale * v_set^T x,        grad_B_i = scale * dy_i^T u_i
 * count = 1..4 members; q[i] is member i's weight [n_out_i x n_in] (the same
 * n_in and the same flags for all); A_set [count r x n_in] holds the members'
 * A matrices back to back (member i: rows i r .. i r + r - 1), and u_set,
 * v_set [T x count r] the members' u / v side by side (member i: columns
 * i r ..).  B[i] [n_out_i x r], y[i] [T x n_out_i], dy[i] [T x n_out_i] and
 * grad_B[i] [n_out_i x r] are arrays of count device pointers; grad_x is the
 * gradient of x summed over the members (NULL skips it).  The few-token
 * kernels run the forward for T <= 16 (and up to 64 while the tokens' x tile
 * stays within 40 KB of LDS, which the shorter spans of smaller weights
 * allow) as one pass over the members' concatenated rows when every member
 * but the last has a multiple of 64 rows (else member by member), and the
 * backward for T <= 4 (T <= 3 for sets above 128 M weights in all; for a set
 * of one as for a single linear: T <= 2, or T <= 4 for weights of at most
 * 4096 x 4096 elements) as
 * one pass over every member's rows (grad_x summed over the members in fp32,
 * rounded to bf16 once); same layouts.  No
 * dropout here: each adapter draws its own mask, so sets with dropout go per
 * linear.                                                                   */
size_t qlora_linear_set_workspace_bytes(int64_t T, int count, const int64_t *n_out, int64_t n_in, int r);

qlora_status qlora_linear_set_fwd(const uint16_t *x, int64_t T, int count, const qlora_nf4_weight *q,
                                  const uint16_t *A_set, const uint16_t *const *B, int r, float scale,
                                  uint16_t *const *y, uint16_t *u_out, void *ws, size_t ws_bytes,
                                  void *stream);

qlora_status qlora_linear_set_bwd(const uint16_t *const *dy, const uint16_t *x, int64_t T, int count,
                                  const qlora_nf4_weight *q, const uint16_t *A_set,
                                  const uint16_t *const *B, int r, float scale, const uint16_t *u,
                                  uint16_t *grad_x, float *grad_A_set, float *const *grad_B, void *ws,
                                  size_t ws_bytes, void *stream);

/* ---- LoRA dropout -------------------------------------------------------- */

/* The recipe sets a dropout probability p on the adapters ("Tutorial
 * fine-tuning LLM LoRA/QLoRA", section "Código Completo", step "4.
 * Configuração LoRA").  Dropout acts on the adapter input only, kept values
 * scaled by 1 / (1 - p); the backward uses the same mask:
 *   u      = bf16( (1 / (1 - p)) (keep (.) x) A^T )
 *   y      = bf16( x W_hat^T + scale * u B^T )
 *   grad_x = bf16( dy W_hat + (scale / (1 - p)) keep (.) (v A) ),  v = dy B
 *   grad_A = (scale / (1 - p)) v^T (keep (.) x),   grad_B = scale * dy^T u
 * The mask is a pure function of (seed, position): element e = t K + k of
 * x [T x K] takes 32-bit word e mod 8 of the Philox4x64-10 block (Salmon et
 * al., SC 2011) for counter (e div 8, 0, 0, 0) and key (seed, 0) -- the four
 * 64-bit outputs in order, low half first -- and is kept iff that word is
 * >= min(2^32 - 1, floor(p 2^32 + 1/2)).  The forward and the backward each
 * regenerate it, so pass them the same seed (and a new seed per step).
 * 0 <= dropout_p < 1 (QLORA_ERR_VALUE otherwise); p = 0 keeps everything
 * (the results then equal those of the plain calls up to rounding order).   */

/* Workspace of the two dropout calls: the plain one plus the mask words and
 * the masked input (4 ceil(T/32) n_in + 2 T n_in bytes, 256-B aligned).     */
size_t qlora_linear_dropout_workspace_bytes(int64_t T, int64_t n_out, int64_t n_in, int r);

/* qlora_linear_fwd with LoRA dropout (same shapes, rules and errors).        */
qlora_status qlora_linear_fwd_dropout(const uint16_t *x, int64_t T, const qlora_nf4_weight *q,
                                      const uint16_t *A, const uint16_t *B, int r, float scale,
                                      double dropout_p, uint64_t seed, uint16_t *y, uint16_t *u_out,
                                      void *ws, size_t ws_bytes, void *stream);

/* qlora_linear_bwd with LoRA dropout; u = NULL recomputes it with the mask.  */
qlora_status qlora_linear_bwd_dropout(const uint16_t *dy, const uint16_t *x, int64_t T,
                                      const qlora_nf4_weight *q, const uint16_t *A, const uint16_t *B,
                                      int r, float scale, double dropout_p, uint64_t seed,
                                      const uint16_t *u, uint16_t *grad_x, float *grad_A,
                                      float *grad_B, void *ws, size_t ws_bytes, void *stream);

/* The mask itself, as the linear calls form it, for x [T x K] bf16 (device,
 * K % 8 == 0): keep_words [ceil(T/32) x K] uint32, bit b of word [tb][k] set
 * iff (32 tb + b, k) is kept (0 past T); x_drop [T x K] bf16 = x where kept,
 * +0 where dropped.  Device buffers, 16-B aligned, caller-owned.            */
qlora_status qlora_dropout_mask(const uint16_t *x, int64_t T, int64_t K, double dropout_p,
                                uint64_t seed, uint32_t *keep_words, uint16_t *x_drop, void *stream);

/* AdamW update of n adapter values held in one flat buffer (the caller lays
 * the A and B matrices of its adapters out back to back).  Only the adapters
 * train, and the optimizer keeps two moments per trained value ("LoRA vs.
 * QLoRA vs. Full Fine-Tuning", section "Quanta VRAM cada método precisa?").
 * For step t >= 1, with the scalars formed in fp64 and rounded once to fp32
 *   c_m = 1 - beta1, c_v = 1 - beta2, decay = 1 - lr * weight_decay,
 *   step_size = lr / (1 - beta1^t), bc2_sqrt = sqrt(1 - beta2^t)   (C pow),
 * every element is updated with one fp32 rounding per operation, no fused
 * multiply-add, in this order:
 *   m <- fl32(beta1) m + c_m g;       v <- fl32(beta2) v + c_v (g g);
 *   d  = sqrt(v) / bc2_sqrt + eps;     p <- p decay;
 *   p <- p - step_size (m / d);        param_bf16 = bf16_round_nearest_even(p).
 * param (fp32 master copy), exp_avg (m) and exp_avg_sq (v) are updated in
 * place; param_bf16 receives the copy the linear calls read; grad is fp32
 * (e.g. the grad_A / grad_B of qlora_linear_bwd).  All five are 16-B aligned
 * and hold n elements; they must not overlap.
 * Paged states ("qlora" entry, section "como funciona"): exp_avg and
 * exp_avg_sq (and any other buffer) may be pinned host memory allocated with
 * hipHostMalloc instead of device memory; the kernel then reads and writes
 * them in place across the host link, and nothing is copied beforehand.
 * Pageable host memory (plain malloc) is rejected with QLORA_ERR_MEMORY.
 * Errors: QLORA_ERR_SHAPE if n < 0 or n > 2^37; QLORA_ERR_VALUE if step < 1,
 * a beta is outside [0, 1), lr, eps or weight_decay is negative or not finite,
 * or step_size is not finite; n == 0 enqueues nothing.  A NaN or Inf in grad
 * or in the states propagates into the outputs of that element only.          */
qlora_status qlora_adamw_step(float *param, uint16_t *param_bf16, const float *grad,
                              float *exp_avg, float *exp_avg_sq, int64_t n, int64_t step,
                              double lr, double beta1, double beta2, double eps,
                              double weight_decay, void *stream);

/* ---- diagnostics ---------------------------------------------------------- */

/* Kernel timing for benchmarks.  While enabled (non-zero), every launch of
 * the main kernel of each kind below is bracketed by two HIP events recorded
 * on the call's stream.  The events are created by the library (no device
 * memory is allocated).  Not thread-safe: one host thread at a time.        */
enum {
  QLORA_TIMED_QGEMM_FWD = 0, /* dequant-fused GEMM, forward: x W_hat^T (+ LoRA)       */
  QLORA_TIMED_QGEMM_DX = 1,  /* dequant-fused GEMM, grad_x: dy W_hat (+ LoRA)         */
  QLORA_TIMED_GEMV_FWD = 2,  /* few-token forward, weight pass (T <= 16, to 64 by shape) */
  QLORA_TIMED_GEMV_BWD = 3,  /* few-token backward, weight and adapter pass (T <= 2, or 4 by shape; sets T <= 4) */
  QLORA_TIMED_ADAMW = 4,     /* adapter AdamW update, whole 4096-element tiles          */
  QLORA_TIMED_KINDS = 5
};
void qlora_kernel_timing_enable(int enable);

/* Synchronise the recorded events and write, for each kind k, the number of
 * timed launches to launches[k] and their summed duration in milliseconds to
 * total_ms[k] (arrays of QLORA_TIMED_KINDS; either may be NULL); then forget
 * them.  QLORA_ERR_HIP if an event could not be read.                       */
qlora_status qlora_kernel_timing_read(int64_t *launches, double *total_ms);

/* Wait for `stream`, then read the status word a previous call left in `ws`:
 * QLORA_OK or QLORA_ERR_NONFINITE (the word is not cleared).                  */
qlora_status qlora_status_read(const void *ws, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QLORA_H */
