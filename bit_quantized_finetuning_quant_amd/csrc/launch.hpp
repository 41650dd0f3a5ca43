// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace qlora {

// Packed weight as the kernels see it.  dq: the block constants are FP8
// codes (fp8) with fp32 group scales (s2) and a tensor mean (mu); otherwise
// s2 holds one fp32 constant per block and fp8, mu are unused.
struct QWeight {
  const uint8_t *codes;
  const uint8_t *fp8;
  const float *s2;
  const float *mu;
  int64_t n_out, n_in;
  bool dq;
};

// Copies of the 256 exponent bins of the quantizer's exact mean: workgroup g
// adds into copy g % kBinCopies, which keeps the global atomics on any one
// address few.  Quantize workspace: status (256 B), the bins
// (kBinCopies x 256 u64), fp32 block absmax.
constexpr int kBinCopies = 16;
constexpr size_t kQuantizeBinBytes = (size_t)kBinCopies * 256 * 8;

// dq = false: the block constants go to c1 (the caller's fp32 constants) and
// the mean and FP8 stages are skipped; fp8, s2 and mu are then unused.
hipError_t launch_quantize(const void *w, bool bf16_src, bool dq, int64_t numel, uint8_t *codes, uint8_t *fp8,
                           float *s2, float *mu, uint32_t *status, unsigned long long *bins, float *c1,
                           const Midpoints &mid, hipStream_t st);

hipError_t launch_dequantize(const QWeight &w, uint16_t *out, const Codebook &cb, hipStream_t st);

// Several weights decoded in one launch (codec.hip); pass0 is set by the launcher.
constexpr int kMaxDequantSet = 8;
struct DequantSet {
  int count;
  QWeight w[kMaxDequantSet];
  uint16_t *out[kMaxDequantSet];
  int64_t pass0[kMaxDequantSet];
};
hipError_t launch_dequantize_set(const DequantSet &set, const Codebook &cb, hipStream_t st);

// Few-token path (gemv.hip): the forward for 1 <= T <= kGemvFwdMaxT (its
// matrix tiles pad the tokens to a multiple of 16), the backward of a single linear for
// 1 <= T <= kGemvLinearBwdMaxT (to kGemvMaxT for weights of at most
// kGemvSmallWeight elements) and of a projection set for 1 <= T <= kGemvMaxT
// (its dot products cost per token; beyond these counts the fused GEMM's
// backward is faster).  `part` is fp32 scratch of gemv_part_floats(T, N, K, r)
// floats, or gemv_fwd_part_floats for a forward alone.  launch_gemv_fwd with
// y == nullptr only computes u; launch_gemv_bwd with grad_x == nullptr skips
// the weight pass.
constexpr int64_t kGemvMaxT = 4;
constexpr int64_t kGemvLinearBwdMaxT = 2;
constexpr int64_t kGemvSmallWeight = (int64_t)4096 * 4096;
constexpr int64_t kGemvFwdMaxT = 64;
bool gemv_fwd_applies(int64_t T, int64_t N, int64_t K);  // the forward over N rows (a set: all members' rows)
bool gemv_bwd_applies(int64_t T, int64_t N, int64_t K, int count);  // the backward of `count` linears sharing x, N rows in all
size_t gemv_part_floats(int64_t T, int64_t N, int64_t K, int r);
size_t gemv_fwd_part_floats(int64_t T, int64_t N, int64_t K, int r);
// The adapter input xa (x, or the dropped-out x) feeds u = u_scale * xa A^T
// and grad_A = scale_ax * v^T xa; scale_ax also scales the adapter term of
// grad_x, which `keep` (nullptr: no dropout) masks element by element.
hipError_t launch_gemv_fwd(int64_t T, const uint16_t *x, const uint16_t *xa, const QWeight &w, const uint16_t *A,
                           const uint16_t *B, int r, float scale, float u_scale, uint16_t *y, uint16_t *u,
                           float *part, const Codebook &cb, hipStream_t st);
// Few-token forward of a projection set in one pass over the members' concatenated rows (every
// member but the last a multiple of 64 rows: gemv_set_fusable); u_set [T x count r].  `part` holds
// gemv_part_floats(T, sum of n_out, K, count r) floats.
bool gemv_set_fusable(const int64_t *N, int count);
hipError_t launch_gemv_fwd_set(int64_t T, const uint16_t *x, const QWeight *w, int count, const uint16_t *A_set,
                               const uint16_t *const *B, int r, float scale, uint16_t *const *y, uint16_t *u_set,
                               float *part, const Codebook &cb, hipStream_t st);
// Few-token backward of a projection set in one pass over every member's rows: grad_x summed over
// the members, grad_A_set [count r x K], grad_B[i]; u_set and v [T x count r].  `part` holds
// gemv_set_part_floats(T, n_out, count, K, r) floats (which also covers launch_gemv_fwd_set;
// gemv_set_fwd_part_floats covers it alone).
size_t gemv_set_part_floats(int64_t T, const int64_t *N, int count, int64_t K, int r);
size_t gemv_set_fwd_part_floats(int64_t T, const int64_t *N, int count, int64_t K, int r);
hipError_t launch_gemv_bwd_set(int64_t T, const uint16_t *const *dy, const uint16_t *x, const QWeight *w, int count,
                               const uint16_t *A_set, const uint16_t *const *B, int r, float scale,
                               const uint16_t *u_set, uint16_t *grad_x, float *grad_A_set, float *const *grad_B,
                               float *part, const Codebook &cb, hipStream_t st);
hipError_t launch_gemv_bwd(int64_t T, const uint16_t *dy, const uint16_t *xa, const QWeight &w, const uint16_t *A,
                           const uint16_t *B, int r, float scale, float scale_ax, const uint32_t *keep,
                           const uint16_t *u, uint16_t *grad_x, float *grad_A, float *grad_B, float *part,
                           const Codebook &cb, hipStream_t st);

// Workspace plan of the linear calls (byte offsets into the caller's buffer).
struct LinearPlan {
  int64_t T, N, K;
  int r;
  bool dropout;
  size_t off_status, off_u, off_v, off_part, off_qpart, off_keep, off_xd, total;
};

// LoRA dropout of one linear call (dropout.hip): the mask of the adapter input
// is regenerated from (thresh, seed) by the forward and by the backward.
struct Dropout {
  bool on;
  uint32_t thresh;  // a uniform 32-bit word below it drops the element
  uint64_t seed;
  float inv_keep;   // fl32(1 / (1 - p))
};
size_t dropout_keep_words(int64_t T, int64_t K);
hipError_t launch_dropout_mask(const uint16_t *x, int64_t T, int64_t K, uint32_t thresh, uint64_t seed,
                               uint32_t *keep, uint16_t *xd, hipStream_t st);

// Adapter-side products (lora.hip).
enum class LoraKind { kU, kV, kGrad };
int lora_splits(int64_t tiles, int64_t kc);
int64_t lora_tiles(int64_t m, int64_t n);
size_t lora_part_floats(int64_t m, int64_t n, int64_t kc);
hipError_t launch_lora(LoraKind kind, const uint16_t *P, int64_t ldp, const uint16_t *Q, int64_t ldq, int64_t M,
                       int64_t Nc, int64_t Kc, float scale, void *out, float *part, hipStream_t st);
// grad_A = s v^T x and grad_B = s dy^T u in one launch (plus one reduction); the
// partials of grad_A take the first part_a_floats of `part`, those of grad_B follow.
hipError_t launch_lora_grads(const uint16_t *v, const uint16_t *x, const uint16_t *dy, const uint16_t *u, int64_t T,
                             int64_t N, int64_t K, int r, float scale_a, float scale_b, float *grad_A, float *grad_B,
                             float *part, size_t part_a_floats, hipStream_t st);

// A projection set: linears that share their input (q/k/v, gate/up), run as
// one fused GEMM launch (qgemm.hip).  Members share n_in and the storage form.
constexpr int kMaxSetMembers = 4;
struct QgemmMember {
  QWeight w;
  const uint16_t *act;  // grad_x: this member's dy [M x n_out]
  const uint16_t *lb;   // forward: this member's B [n_out x r]
  uint16_t *out;        // forward: this member's y [M x n_out]
  int64_t tile0;        // forward: first column tile (set by the launcher)
};
struct QgemmSet {
  int count;
  int64_t ld_la;  // row stride of the adapter left factor (u_set or v_set)
  QgemmMember m[kMaxSetMembers];
  // columns of a split's fp32 partial tiles (set by launch_qgemm_set): grad_x
  // n_in; forward the members' column tiles side by side (tile t at columns
  // [128 t, 128 t + 128))
  int64_t part_cols;
};
// forward: x shared, la = u_set (member i reads columns [i r, i r + r)); grad_x:
// gx = sum over members of dy_i W_hat_i + keep (.) (scale * la lb^T) with la =
// v_set, lb = A_set and r the total rank.
// part: fp32 scratch for a split contraction (qgemm_split_floats of the shape; nullptr: never split).
hipError_t launch_qgemm_set(bool trans_w, const QgemmSet &set, int64_t M, const uint16_t *x, const uint16_t *la,
                            const uint16_t *lb, int r, float scale, uint16_t *gx, const Codebook &cb, hipStream_t st,
                            const uint32_t *keep = nullptr, float *part = nullptr);

// Split contraction of a single linear's fused GEMM (out [M x Ncols], contraction Kc): `splits`
// workgroups per output tile, `steps` contraction steps of 64 each (splits == 1: none).
struct QgemmSplit {
  int splits;
  int64_t steps;
};
QgemmSplit qgemm_split(int64_t M, int64_t Ncols, int64_t Kc, double *cost = nullptr);
// fp32 scratch of a set's grad_x run member by member at a few tokens (0: never)
size_t qgemm_set_dx_member_floats(int64_t M, int count, const int64_t *n_out, int64_t n_in);
size_t qgemm_split_floats(int64_t M, int64_t Ncols, int64_t Kc);

// Adapter products of a projection set (lora.hip); each product has its own
// region of `part`, lora_set_part_floats in all.
size_t lora_set_part_floats(int64_t T, int count, const int64_t *N, int64_t K, int r);
hipError_t launch_lora_set_v(const uint16_t *const *dy, const uint16_t *const *B, const int64_t *N, int count,
                             int64_t T, int r, uint16_t *v_set, float *part, hipStream_t st);
hipError_t launch_lora_set_grads(const uint16_t *v_set, const uint16_t *x, const uint16_t *const *dy,
                                 const uint16_t *u_set, const int64_t *N, int count, int64_t T, int64_t K, int r,
                                 float scale, float *grad_A_set, float *const *grad_B, float *part, hipStream_t st);

// Dequant-fused GEMM: out = keep (.) (scale * la lb^T) + act W_op (see
// qgemm.hip); keep (dropout words, [ceil(M/32)][Ncols]) may be nullptr.
hipError_t launch_qgemm(bool trans_w, const uint16_t *act, int64_t M, int64_t Ncols, int64_t Kc, const QWeight &w,
                        const uint16_t *la, const uint16_t *lb, int r, float scale, uint16_t *out,
                        const Codebook &cb, hipStream_t st, const uint32_t *keep = nullptr, float *part = nullptr);

LinearPlan plan_linear(int64_t T, int64_t N, int64_t K, int r, bool dropout = false);

// Optional event bracketing of the fused GEMM launches (diagnostics).
// Diagnostics: HIP events around the main kernel of each kind (linear.hip).
enum TimedKind : int {
  kTimedQgemmFwd = 0,
  kTimedQgemmDx = 1,
  kTimedGemvFwd = 2,
  kTimedGemvBwd = 3,
  kTimedAdamw = 4,
  kTimedKinds = 5
};
struct TimedLaunch {
  hipEvent_t start, stop;
  int kind;
};
bool timing_begin(hipStream_t st, TimedLaunch &t, int kind);  // false when timing is off
void timing_end(hipStream_t st, TimedLaunch &t);
void kernel_timing_enable(bool on);
bool kernel_timing_read(int64_t *launches, double *ms);  // arrays of kTimedKinds

hipError_t launch_linear_fwd(const LinearPlan &p, const uint16_t *x, const QWeight &w, const uint16_t *A,
                             const uint16_t *B, float scale, uint16_t *y, uint16_t *u_out, char *ws,
                             const Codebook &cb, hipStream_t st, const Dropout &d = Dropout{false, 0u, 0ull, 1.f});

hipError_t launch_linear_bwd(const LinearPlan &p, const uint16_t *dy, const uint16_t *x, const QWeight &w,
                             const uint16_t *A, const uint16_t *B, float scale, const uint16_t *u,
                             uint16_t *grad_x, float *grad_A, float *grad_B, char *ws, const Codebook &cb,
                             hipStream_t st, const Dropout &d = Dropout{false, 0u, 0ull, 1.f});

// AdamW update of a flat fp32 adapter buffer (optim.hip).  The scalars that
// depend only on the hyperparameters and the step, each formed in fp64 and
// rounded once to fp32 on the host.
struct AdamwScalars {
  float b1, b2;        // fl32(beta1), fl32(beta2)
  float c_m, c_v;      // fl32(1 - beta1), fl32(1 - beta2)
  float decay;         // fl32(1 - lr * weight_decay)
  float step_size;     // fl32(lr / (1 - beta1^t))
  float bc2_sqrt;      // fl32(sqrt(1 - beta2^t))
  float eps;           // fl32(eps)
};
hipError_t launch_adamw(float *param, uint16_t *param_bf16, const float *grad, float *exp_avg, float *exp_avg_sq,
                        int64_t n, const AdamwScalars &s, hipStream_t st);

// Few-token sets (gemv.hip helper): a strided 2-D copy of bf16 rows.
hipError_t launch_copy_rows(const uint16_t *src, int64_t ld_src, uint16_t *dst, int64_t ld_dst, int64_t rows,
                            int64_t cols, hipStream_t st);

// Projection sets (linear.hip): members share x [T x K] and the adapter
// rank r; A_set [count r x K] holds the members' A back to back, u_set and
// v_set are [T x count r].  The few-token kernels run the set's forward for
// T <= kGemvFwdMaxT and its backward where gemv_bwd_applies (a [T x r] u block
// in the workspace for a member-by-member forward).
struct SetPlan {
  int64_t T, K;
  int r, count;
  int64_t N[kMaxSetMembers];
  size_t off_u, off_v, off_part, off_um, off_qpart, total;  // off_qpart: 0 when neither direction splits
  bool fwd_few;  // the forward on the few-token kernels (gemv_fwd_applies over all members' rows)
  bool bwd_few;  // the backward on the few-token kernels (gemv_bwd_applies over all members' rows)
};
SetPlan plan_linear_set(int64_t T, int count, const int64_t *N, int64_t K, int r);
hipError_t launch_linear_set_fwd(const SetPlan &p, const uint16_t *x, const QWeight *w, const uint16_t *A_set,
                                 const uint16_t *const *B, float scale, uint16_t *const *y, uint16_t *u_out, char *ws,
                                 const Codebook &cb, hipStream_t st);
hipError_t launch_linear_set_bwd(const SetPlan &p, const uint16_t *const *dy, const uint16_t *x, const QWeight *w,
                                 const uint16_t *A_set, const uint16_t *const *B, float scale, const uint16_t *u,
                                 uint16_t *grad_x, float *grad_A_set, float *const *grad_B, char *ws,
                                 const Codebook &cb, hipStream_t st);

}  // namespace qlora
