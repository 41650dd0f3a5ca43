// C ABI of the QLoRA linear layer library (declared in include/qlora.h):
// argument validation, workspace plans and kernel launches.  Host code only.

#include <math.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "../../include/qlora.h"
#include "common.hpp"
#include "launch.hpp"

using namespace qlora;

namespace {

// ---- NF4 levels, computed on the host from the definition ------------------
// Standard-normal quantiles at equal probability steps on each side of 1/2:
// 8 positive levels up to probability delta and 7 negative levels down to
// 1 - delta, plus an exact zero, all divided by the largest quantile so that
// the range is [-1, 1]; delta = 1 - (1/32 + 1/30)/2 is the mean of the
// half-bin offsets of a 16-level and a 15-level equal-probability grid.
double normal_cdf(double z) { return 0.5 * std::erfc(-z / std::sqrt(2.0)); }
double normal_pdf(double z) { return std::exp(-0.5 * z * z) / std::sqrt(2.0 * M_PI); }

// Phi^-1(p) for p in (1/2, 1): bisection to full double resolution, then two
// Newton steps on the upper-tail form 1 - Phi(z) = erfc(z/sqrt2)/2.
double normal_quantile_upper(double p) {
  double lo = 0.0, hi = 40.0;
  for (int i = 0; i < 200 && hi - lo > 0; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (normal_cdf(mid) < p) lo = mid; else hi = mid;
  }
  double z = 0.5 * (lo + hi);
  const double q = 1.0 - p;  // exact for the probabilities used here
  for (int i = 0; i < 2; ++i) z += (0.5 * std::erfc(z / std::sqrt(2.0)) - q) / normal_pdf(z);
  return z;
}

struct Tables {
  Codebook cb;
  Midpoints mid;
  Tables() {
    const double delta = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0);
    const double top = normal_quantile_upper(delta);
    double lv[16];
    for (int j = 1; j <= 7; ++j) lv[7 - j] = -normal_quantile_upper(0.5 + j * (delta - 0.5) / 7.0) / top;
    lv[7] = 0.0;
    for (int j = 1; j <= 8; ++j) lv[7 + j] = normal_quantile_upper(0.5 + j * (delta - 0.5) / 8.0) / top;
    lv[0] = -1.0;
    lv[15] = 1.0;
    for (int k = 0; k < 16; ++k) cb.v[k] = (float)lv[k];
    for (int j = 0; j < 15; ++j) mid.m[j] = ((double)cb.v[j] + (double)cb.v[j + 1]) * 0.5;  // exact
  }
};

const Tables &tables() {
  static const Tables t;
  return t;
}

constexpr int64_t kMaxNumel = (int64_t)1 << 37;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// a * b <= kMaxNumel for positive a, b, without forming a product that could overflow
bool product_ok(int64_t a, int64_t b) { return a > 0 && b > 0 && a <= kMaxNumel / b; }

bool shape_ok(int64_t n_out, int64_t n_in) { return product_ok(n_out, n_in); }

bool double_quantized(const qlora_nf4_weight *q) { return (q->flags & QLORA_NF4_FP32_CONSTANTS) == 0u; }

qlora_status check_weight(const qlora_nf4_weight *q) {
  if (!q) return QLORA_ERR_NULL;
  if (!shape_ok(q->n_out, q->n_in)) return QLORA_ERR_SHAPE;
  if ((q->flags & ~QLORA_NF4_FP32_CONSTANTS) != 0u) return QLORA_ERR_VALUE;
  if (!q->codes || !q->absmax_scale) return QLORA_ERR_NULL;
  if (!aligned16(q->codes) || !aligned16(q->absmax_scale)) return QLORA_ERR_ALIGN;
  if (double_quantized(q)) {
    if (!q->absmax_fp8 || !q->absmax_mean) return QLORA_ERR_NULL;
    if (!aligned16(q->absmax_fp8) || !aligned16(q->absmax_mean)) return QLORA_ERR_ALIGN;
  }
  return QLORA_OK;
}

QWeight qweight(const qlora_nf4_weight *q) {
  return QWeight{q->codes, q->absmax_fp8, q->absmax_scale, q->absmax_mean, q->n_out, q->n_in, double_quantized(q)};
}

qlora_status check_linear(int64_t T, const qlora_nf4_weight *q, int r, float scale) {
  qlora_status s = check_weight(q);
  if (s != QLORA_OK) return s;
  if (T < 1 || T > kMaxNumel || q->n_in % kBlock != 0 || r < 1 || r > 256) return QLORA_ERR_SHAPE;
  if (!product_ok(T, q->n_in) || !product_ok(T, q->n_out)) return QLORA_ERR_SHAPE;
  if (!std::isfinite(scale)) return QLORA_ERR_VALUE;
  return QLORA_OK;
}

// Dropout arguments: 0 <= p < 1 (finite); thresh = min(2^32 - 1, floor(p 2^32 + 1/2))
// in fp64, and the fp32 factor 1 / (1 - p) of the kept values.
bool make_dropout(double p, uint64_t seed, Dropout *d) {
  if (!std::isfinite(p) || p < 0.0 || p >= 1.0) return false;
  const double t = std::floor(p * 4294967296.0 + 0.5);
  d->on = true;
  d->thresh = t >= 4294967295.0 ? 0xFFFFFFFFu : (uint32_t)t;
  d->seed = seed;
  d->inv_keep = (float)(1.0 / (1.0 - p));
  return true;
}

// The address a kernel uses for p: p itself for device or managed memory, the
// mapped device address for pinned host memory (hipHostMalloc), and false for
// memory the GPU cannot reach (pageable host memory, unknown pointers).
bool device_address(const void *p, void **dev) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  switch (a.type) {
    case hipMemoryTypeDevice:
    case hipMemoryTypeManaged:
    case hipMemoryTypeUnified:
      *dev = const_cast<void *>(p);
      return true;
    case hipMemoryTypeHost:
      if (!a.devicePointer || !a.hostPointer) return false;
      *dev = (char *)a.devicePointer + ((const char *)p - (const char *)a.hostPointer);
      return true;
    default:
      return false;
  }
}

// A projection set: 1..kMaxSetMembers members sharing n_in and the storage
// form, adapter rank r per member.
qlora_status check_set(int64_t T, int count, const qlora_nf4_weight *q, int r, float scale, int64_t *N) {
  if (!q) return QLORA_ERR_NULL;
  if (count < 1 || count > kMaxSetMembers) return QLORA_ERR_SHAPE;
  for (int i = 0; i < count; ++i) {
    const qlora_status s = check_linear(T, &q[i], r, scale);
    if (s != QLORA_OK) return s;
    if (q[i].n_in != q[0].n_in) return QLORA_ERR_SHAPE;
    if (q[i].flags != q[0].flags) return QLORA_ERR_VALUE;
    N[i] = q[i].n_out;
  }
  if (!product_ok(T, (int64_t)count * r)) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

// ---- scratch of the forward without a caller workspace --------------------
// For callers that cannot allocate (graph capture, serving loops): a fixed
// device array, one copy per GPU for the life of the process.  In host code
// its name stands for a host-side shadow, not a device address, so host code
// only ever uses the address hipGetSymbolAddress returns for the current
// device (looked up on the first call on that device and kept).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

qlora_status noalloc_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return QLORA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return QLORA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QLORA_OK;
}

// Bytes of a linear workspace the forward touches: u (when the caller does not
// take it), the partial sums of its own adapter product and, when its fused
// GEMM splits the contraction, the split partials, at the offsets of the
// linear plan.
size_t forward_scratch_bytes(const LinearPlan &p) {
  if (gemv_fwd_applies(p.T, p.N, p.K)) return p.off_part + gemv_fwd_part_floats(p.T, p.N, p.K, p.r) * 4;
  const size_t qsplit = qgemm_split_floats(p.T, p.N, p.K);
  return std::max(p.off_part + lora_part_floats(p.T, p.r, p.K) * 4, qsplit ? p.off_qpart + qsplit * 4 : 0);
}

}  // namespace

extern "C" {

qlora_status qlora_nf4_sizes(int64_t n_out, int64_t n_in, int64_t *codes_bytes, int64_t *nblocks,
                             int64_t *ngroups) {
  if (!shape_ok(n_out, n_in)) return QLORA_ERR_SHAPE;
  const int64_t numel = n_out * n_in;
  const int64_t nb = (numel + kBlock - 1) / kBlock;
  if (codes_bytes) *codes_bytes = (numel + 1) / 2;
  if (nblocks) *nblocks = nb;
  if (ngroups) *ngroups = (nb + kGroup - 1) / kGroup;
  return QLORA_OK;
}

size_t qlora_nf4_bytes(int64_t n_out, int64_t n_in) {
  int64_t cb, nb, ng;
  if (qlora_nf4_sizes(n_out, n_in, &cb, &nb, &ng) != QLORA_OK) return 0;
  return (size_t)(cb + nb + 4 * ng + 4);
}

size_t qlora_nf4_bytes_flags(int64_t n_out, int64_t n_in, uint32_t flags) {
  if ((flags & ~QLORA_NF4_FP32_CONSTANTS) != 0u) return 0;
  if (!(flags & QLORA_NF4_FP32_CONSTANTS)) return qlora_nf4_bytes(n_out, n_in);
  int64_t cb, nb;
  if (qlora_nf4_sizes(n_out, n_in, &cb, &nb, nullptr) != QLORA_OK) return 0;
  return (size_t)(cb + 4 * nb);
}

size_t qlora_quantize_workspace_bytes(int64_t n_out, int64_t n_in) {
  int64_t nb;
  if (qlora_nf4_sizes(n_out, n_in, nullptr, &nb, nullptr) != QLORA_OK) return 0;
  // status (256 B) + exponent bins + fp32 block absmax
  return 256 + kQuantizeBinBytes + (size_t)nb * 4;
}

// the shapes every linear call accepts (check_linear), for the size helpers
bool linear_shape_ok(int64_t T, int64_t n_out, int64_t n_in, int r) {
  return shape_ok(n_out, n_in) && n_in % kBlock == 0 && r >= 1 && r <= 256 && product_ok(T, n_in) &&
         product_ok(T, n_out);
}

size_t qlora_linear_workspace_bytes(int64_t T, int64_t n_out, int64_t n_in, int r) {
  if (!linear_shape_ok(T, n_out, n_in, r)) return 0;
  return plan_linear(T, n_out, n_in, r).total;
}

size_t qlora_linear_dropout_workspace_bytes(int64_t T, int64_t n_out, int64_t n_in, int r) {
  if (!linear_shape_ok(T, n_out, n_in, r)) return 0;
  return plan_linear(T, n_out, n_in, r, true).total;
}

void qlora_nf4_codebook(float out[16]) {
  if (!out) return;
  memcpy(out, tables().cb.v, sizeof(float) * 16);
}

const char *qlora_status_string(qlora_status s) {
  // C callers and bindings may pass any integer: read the code as one (loading an enum object that
  // holds a value outside the enumeration is undefined in C++)
  int code;
  memcpy(&code, &s, sizeof code);
  switch (code) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "a required pointer is NULL";
    case QLORA_ERR_SHAPE: return "a dimension is out of range";
    case QLORA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case QLORA_ERR_WORKSPACE: return "workspace too small";
    case QLORA_ERR_DTYPE: return "unknown dtype";
    case QLORA_ERR_HIP: return "HIP runtime error at launch";
    case QLORA_ERR_NONFINITE: return "NaN or Inf in the quantized weight";
    case QLORA_ERR_VALUE: return "a scalar argument is not finite or out of range";
    case QLORA_ERR_MEMORY: return "a buffer is not reachable by the GPU (pageable host memory?)";
    case QLORA_ERR_SCRATCH: return "the call needs more scratch than the library's fixed array holds";
  }
  return "unknown status";
}

const char *qlora_version(void) { return "qlora-gfx950 0.1"; }

qlora_status qlora_quantize(const void *w, qlora_dtype w_dtype, const qlora_nf4_weight *q, void *ws,
                            size_t ws_bytes, void *stream) {
  qlora_status s = check_weight(q);
  if (s != QLORA_OK) return s;
  if (!w || !ws) return QLORA_ERR_NULL;
  if (!aligned16(w) || !aligned16(ws)) return QLORA_ERR_ALIGN;
  int dtype;  // read as an integer: a caller may pass any value (see qlora_status_string)
  memcpy(&dtype, &w_dtype, sizeof dtype);
  if (dtype != QLORA_F32 && dtype != QLORA_BF16) return QLORA_ERR_DTYPE;
  if (ws_bytes < qlora_quantize_workspace_bytes(q->n_out, q->n_in)) return QLORA_ERR_WORKSPACE;
  char *base = (char *)ws;
  // without double quantization the block constants go straight to absmax_scale
  const bool dq = double_quantized(q);
  float *c1 = dq ? (float *)(base + 256 + kQuantizeBinBytes) : q->absmax_scale;
  hipError_t e = launch_quantize(w, dtype == QLORA_BF16, dq, q->n_out * q->n_in, q->codes, q->absmax_fp8,
                                 q->absmax_scale, q->absmax_mean, (uint32_t *)base,
                                 (unsigned long long *)(base + 256), c1, tables().mid, (hipStream_t)stream);
  return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

qlora_status qlora_dequantize(const qlora_nf4_weight *q, uint16_t *w_bf16, void *stream) {
  qlora_status s = check_weight(q);
  if (s != QLORA_OK) return s;
  if (!w_bf16) return QLORA_ERR_NULL;
  if (!aligned16(w_bf16)) return QLORA_ERR_ALIGN;
  hipError_t e = launch_dequantize(qweight(q), w_bf16, tables().cb, (hipStream_t)stream);
  return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

qlora_status qlora_dequantize_many(const qlora_nf4_weight *q, int count, uint16_t *const *w_bf16, void *stream) {
  if (!q || !w_bf16) return QLORA_ERR_NULL;
  if (count < 1 || count > kMaxDequantSet) return QLORA_ERR_SHAPE;
  DequantSet set{};
  set.count = count;
  for (int i = 0; i < count; ++i) {
    const qlora_status s = check_weight(&q[i]);
    if (s != QLORA_OK) return s;
    if (!w_bf16[i]) return QLORA_ERR_NULL;
    if (!aligned16(w_bf16[i])) return QLORA_ERR_ALIGN;
    set.w[i] = qweight(&q[i]);
    set.out[i] = w_bf16[i];
  }
  hipError_t e = launch_dequantize_set(set, tables().cb, (hipStream_t)stream);
  return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

qlora_status qlora_linear_fwd(const uint16_t *x, int64_t T, const qlora_nf4_weight *q, const uint16_t *A,
                              const uint16_t *B, int r, float scale, uint16_t *y, uint16_t *u_out, void *ws,
                              size_t ws_bytes, void *stream) {
  qlora_status s = check_linear(T, q, r, scale);
  if (s != QLORA_OK) return s;
  if (!x || !A || !B || !y || !ws) return QLORA_ERR_NULL;
  if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(y) || !aligned16(ws) ||
      (u_out && !aligned16(u_out)))
    return QLORA_ERR_ALIGN;
  const LinearPlan p = plan_linear(T, q->n_out, q->n_in, r);
  if (ws_bytes < p.total) return QLORA_ERR_WORKSPACE;
  hipError_t e = launch_linear_fwd(p, x, qweight(q), A, B, scale, y, u_out, (char *)ws, tables().cb,
                                   (hipStream_t)stream);
  return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

size_t qlora_linear_fwd_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

qlora_status qlora_linear_fwd_noalloc(const uint16_t *x, int64_t T, const qlora_nf4_weight *q, const uint16_t *A,
                                      const uint16_t *B, int r, float scale, uint16_t *y, uint16_t *u_out,
                                      void *stream) {
  qlora_status s = check_linear(T, q, r, scale);
  if (s != QLORA_OK) return s;
  if (!x || !A || !B || !y) return QLORA_ERR_NULL;
  if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(y) || (u_out && !aligned16(u_out)))
    return QLORA_ERR_ALIGN;
  const LinearPlan p = plan_linear(T, q->n_out, q->n_in, r);
  if (forward_scratch_bytes(p) > kNoAllocScratchBytes) return QLORA_ERR_SCRATCH;
  void *ws = nullptr;
  s = noalloc_scratch(&ws);
  if (s != QLORA_OK) return s;
  hipError_t e = launch_linear_fwd(p, x, qweight(q), A, B, scale, y, u_out, (char *)ws, tables().cb,
                                   (hipStream_t)stream);
  return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

qlora_status qlora_linear_bwd(const uint16_t *dy, const uint16_t *x, int64_t T, const qlora_nf4_weight *q,
                              const uint16_t *A, const uint16_t *B, int r, float scale, const uint16_t *u,
                              uint16_t *grad_x, float *grad_A, float *grad_B, void *ws, size_t ws_bytes,
                              void *stream) {
  qlora_status s = check_linear(T, q, r, scale);
  if (s != QLORA_OK) return s;
  if (!dy || !x || !A || !B || !grad_A || !grad_B || !ws) return QLORA_ERR_NULL;
  if (!aligned16(dy) || !aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(grad_A) ||
      !aligned16(grad_B) || !aligned16(ws) || (u && !aligned16(u)) || (grad_x && !aligned16(grad_x)))
    return QLORA_ERR_ALIGN;
  const LinearPlan p = plan_linear(T, q->n_out, q->n_in, r);
  if (ws_bytes < p.total) return QLORA_ERR_WORKSPACE;
  hipError_t e = launch_linear_bwd(p, dy, x, qweight(q), A, B, scale, u, grad_x, grad_A, grad_B, (char *)ws,
                                   tables().cb, (hipStream_t)stream);
  return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

qlora_status qlora_adamw_step(float *param, uint16_t *param_bf16, const float *grad, float *exp_avg,
                              float *exp_avg_sq, int64_t n, int64_t step, double lr, double beta1, double beta2,
                              double eps, double weight_decay, void *stream) {
  if (n < 0 || n > kMaxNumel) return QLORA_ERR_SHAPE;
  if (step < 1 || !std::isfinite(lr) || !std::isfinite(eps) || !std::isfinite(weight_decay) || lr < 0 ||
      eps < 0 || weight_decay < 0 || !(beta1 >= 0 && beta1 < 1) || !(beta2 >= 0 && beta2 < 1))
    return QLORA_ERR_VALUE;
  if (n == 0) return QLORA_OK;
  if (!param || !param_bf16 || !grad || !exp_avg || !exp_avg_sq) return QLORA_ERR_NULL;
  if (!aligned16(param) || !aligned16(param_bf16) || !aligned16(grad) || !aligned16(exp_avg) ||
      !aligned16(exp_avg_sq))
    return QLORA_ERR_ALIGN;
  void *d[5];
  const void *h[5] = {param, param_bf16, grad, exp_avg, exp_avg_sq};
  for (int i = 0; i < 5; ++i)
    if (!device_address(h[i], &d[i]) || !aligned16(d[i])) return QLORA_ERR_MEMORY;
  // Scalars of this step: fp64 from the hyperparameters, one rounding to fp32.
  const double bc1 = 1.0 - std::pow(beta1, (double)step);
  const double bc2 = 1.0 - std::pow(beta2, (double)step);
  AdamwScalars sc;
  sc.b1 = (float)beta1;
  sc.b2 = (float)beta2;
  sc.c_m = (float)(1.0 - beta1);
  sc.c_v = (float)(1.0 - beta2);
  sc.decay = (float)(1.0 - lr * weight_decay);
  sc.step_size = (float)(lr / bc1);
  sc.bc2_sqrt = (float)std::sqrt(bc2);
  sc.eps = (float)eps;
  if (!std::isfinite(sc.step_size) || !(sc.bc2_sqrt > 0.0f)) return QLORA_ERR_VALUE;
  hipError_t e = launch_adamw((float *)d[0], (uint16_t *)d[1], (const float *)d[2], (float *)d[3], (float *)d[4], n,
                              sc, (hipStream_t)stream);
  return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

qlora_status qlora_linear_fwd_dropout(const uint16_t *x, int64_t T, const qlora_nf4_weight *q, const uint16_t *A,
                                      const uint16_t *B, int r, float scale, double dropout_p, uint64_t seed,
                                      uint16_t *y, uint16_t *u_out, void *ws, size_t ws_bytes, void *stream) {
  qlora_status s = check_linear(T, q, r, scale);
  if (s != QLORA_OK) return s;
  Dropout d;
  if (!make_dropout(dropout_p, seed, &d)) return QLORA_ERR_VALUE;
  if (!x || !A || !B || !y || !ws) return QLORA_ERR_NULL;
  if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(y) || !aligned16(ws) ||
      (u_out && !aligned16(u_out)))
    return QLORA_ERR_ALIGN;
  const LinearPlan p = plan_linear(T, q->n_out, q->n_in, r, true);
  if (ws_bytes < p.total) return QLORA_ERR_WORKSPACE;
  hipError_t e = launch_linear_fwd(p, x, qweight(q), A, B, scale, y, u_out, (char *)ws, tables().cb,
                                   (hipStream_t)stream, d);
  return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

qlora_status qlora_linear_bwd_dropout(const uint16_t *dy, const uint16_t *x, int64_t T, const qlora_nf4_weight *q,
                                      const uint16_t *A, const uint16_t *B, int r, float scale, double dropout_p,
                                      uint64_t seed, const uint16_t *u, uint16_t *grad_x, float *grad_A,
                                      float *grad_B, void *ws, size_t ws_bytes, void *stream) {
  qlora_status s = check_linear(T, q, r, scale);
  if (s != QLORA_OK) return s;
  Dropout d;
  if (!make_dropout(dropout_p, seed, &d)) return QLORA_ERR_VALUE;
  if (!dy || !x || !A || !B || !grad_A || !grad_B || !ws) return QLORA_ERR_NULL;
  if (!aligned16(dy) || !aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(grad_A) ||
      !aligned16(grad_B) || !aligned16(ws) || (u && !aligned16(u)) || (grad_x && !aligned16(grad_x)))
    return QLORA_ERR_ALIGN;
  const LinearPlan p = plan_linear(T, q->n_out, q->n_in, r, true);
  if (ws_bytes < p.total) return QLORA_ERR_WORKSPACE;
  hipError_t e = launch_linear_bwd(p, dy, x, qweight(q), A, B, scale, u, grad_x, grad_A, grad_B, (char *)ws,
                                   tables().cb, (hipStream_t)stream, d);
  return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

size_t qlora_linear_set_workspace_bytes(int64_t T, int count, const int64_t *n_out, int64_t n_in, int r) {
  if (!n_out || count < 1 || count > kMaxSetMembers || T < 1 || T > kMaxNumel) return 0;
  if (n_in % kBlock != 0 || r < 1 || r > 256 || !product_ok(T, (int64_t)count * r)) return 0;
  for (int i = 0; i < count; ++i)
    if (!linear_shape_ok(T, n_out[i], n_in, r)) return 0;
  return plan_linear_set(T, count, n_out, n_in, r).total;
}

qlora_status qlora_linear_set_fwd(const uint16_t *x, int64_t T, int count, const qlora_nf4_weight *q,
                                  const uint16_t *A_set, const uint16_t *const *B, int r, float scale,
                                  uint16_t *const *y, uint16_t *u_out, void *ws, size_t ws_bytes, void *stream) {
  int64_t N[kMaxSetMembers];
  qlora_status s = check_set(T, count, q, r, scale, N);
  if (s != QLORA_OK) return s;
  if (!x || !A_set || !B || !y || !ws) return QLORA_ERR_NULL;
  if (!aligned16(x) || !aligned16(A_set) || !aligned16(ws) || (u_out && !aligned16(u_out))) return QLORA_ERR_ALIGN;
  QWeight w[kMaxSetMembers];
  for (int i = 0; i < count; ++i) {
    if (!B[i] || !y[i]) return QLORA_ERR_NULL;
    if (!aligned16(B[i]) || !aligned16(y[i])) return QLORA_ERR_ALIGN;
    w[i] = qweight(&q[i]);
  }
  const SetPlan p = plan_linear_set(T, count, N, q[0].n_in, r);
  if (ws_bytes < p.total) return QLORA_ERR_WORKSPACE;
  hipError_t e = launch_linear_set_fwd(p, x, w, A_set, B, scale, y, u_out, (char *)ws, tables().cb,
                                       (hipStream_t)stream);
  return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

qlora_status qlora_linear_set_bwd(const uint16_t *const *dy, const uint16_t *x, int64_t T, int count,
                                  const qlora_nf4_weight *q, const uint16_t *A_set, const uint16_t *const *B, int r,
                                  float scale, const uint16_t *u, uint16_t *grad_x, float *grad_A_set,
                                  float *const *grad_B, void *ws, size_t ws_bytes, void *stream) {
  int64_t N[kMaxSetMembers];
  qlora_status s = check_set(T, count, q, r, scale, N);
  if (s != QLORA_OK) return s;
  if (!dy || !x || !A_set || !B || !grad_A_set || !grad_B || !ws) return QLORA_ERR_NULL;
  if (!aligned16(x) || !aligned16(A_set) || !aligned16(grad_A_set) || !aligned16(ws) || (u && !aligned16(u)) ||
      (grad_x && !aligned16(grad_x)))
    return QLORA_ERR_ALIGN;
  QWeight w[kMaxSetMembers];
  for (int i = 0; i < count; ++i) {
    if (!dy[i] || !B[i] || !grad_B[i]) return QLORA_ERR_NULL;
    if (!aligned16(dy[i]) || !aligned16(B[i]) || !aligned16(grad_B[i])) return QLORA_ERR_ALIGN;
    w[i] = qweight(&q[i]);
  }
  const SetPlan p = plan_linear_set(T, count, N, q[0].n_in, r);
  if (ws_bytes < p.total) return QLORA_ERR_WORKSPACE;
  hipError_t e = launch_linear_set_bwd(p, dy, x, w, A_set, B, scale, u, grad_x, grad_A_set, grad_B, (char *)ws,
                                       tables().cb, (hipStream_t)stream);
  return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

qlora_status qlora_dropout_mask(const uint16_t *x, int64_t T, int64_t K, double dropout_p, uint64_t seed,
                                uint32_t *keep_words, uint16_t *x_drop, void *stream) {
  if (K % 8 != 0 || !product_ok(T, K)) return QLORA_ERR_SHAPE;
  Dropout d;
  if (!make_dropout(dropout_p, seed, &d)) return QLORA_ERR_VALUE;
  if (!x || !keep_words || !x_drop) return QLORA_ERR_NULL;
  if (!aligned16(x) || !aligned16(keep_words) || !aligned16(x_drop)) return QLORA_ERR_ALIGN;
  hipError_t e = launch_dropout_mask(x, T, K, d.thresh, d.seed, keep_words, x_drop, (hipStream_t)stream);
  return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

void qlora_kernel_timing_enable(int enable) { kernel_timing_enable(enable != 0); }

qlora_status qlora_kernel_timing_read(int64_t *launches, double *total_ms) {
  int64_t n[kTimedKinds];
  double ms[kTimedKinds];
  const bool ok = kernel_timing_read(n, ms);
  for (int k = 0; k < kTimedKinds; ++k) {
    if (launches) launches[k] = n[k];
    if (total_ms) total_ms[k] = ms[k];
  }
  return ok ? QLORA_OK : QLORA_ERR_HIP;
}

qlora_status qlora_status_read(const void *ws, void *stream) {
  if (!ws) return QLORA_ERR_NULL;
  if (!aligned16(ws)) return QLORA_ERR_ALIGN;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return QLORA_ERR_HIP;
  uint32_t word = 0;
  if (hipMemcpy(&word, ws, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return QLORA_ERR_HIP;
  return (word & 1u) ? QLORA_ERR_NONFINITE : QLORA_OK;
}

}  // extern "C"
