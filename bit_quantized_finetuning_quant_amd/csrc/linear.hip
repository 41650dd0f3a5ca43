// QLoRA linear layer kernels for gfx950: dequant-fused bf16 MFMA GEMMs for
// the forward product and grad_x, and the LoRA side products.
//
// Method ("qlora" encyclopedia entry, tonho.wtf, section "a ideia"): the
// frozen 4-bit weight is dequantized to BFloat16 every time it enters a
// matrix product and is never kept in 16 bits; the gradient flows through it
// into the 16-bit adapters only.  Adapter algebra from the nexusinovation
// tutorial, section "LoRA: O Padrão Ouro de Eficiência": W' = W + s.B.A.
//
//   y      = x W_hat^T + s (x A^T) B^T        qgemm.hip (forward form), u from lora.hip
//   grad_x = dy W_hat + s (dy B) A            qgemm.hip (transposed form), v from lora.hip
//   grad_A = s (dy B)^T x                     lora.hip
//   grad_B = s dy^T (x A^T)                   lora.hip
//
// MFMA lane layouts used (v_mfma_f32_32x32x16_bf16, 64 lanes, l = lane):
//   A operand: lane l holds A[i = l%32][k = 8(l/32) .. 8(l/32)+7]
//   B operand: lane l holds B[k = 8(l/32) .. +7][j = l%32]
//   D:         lane l, register q holds D[8(q/4) + 4(l/32) + q%4][l%32]

#include <vector>

#include "common.hpp"
#include "launch.hpp"

namespace qlora {

// ---------------------------------------------------------------------------
// host side

// ---- diagnostics: HIP events around the main kernel launches (events are
// pooled, so a timed launch costs two event records and no event creation)
namespace {
bool g_timing = false;
std::vector<TimedLaunch> g_timed;
std::vector<hipEvent_t> g_event_pool;

bool pooled_event(hipEvent_t &e) {
  if (!g_event_pool.empty()) {
    e = g_event_pool.back();
    g_event_pool.pop_back();
    return true;
  }
  return hipEventCreate(&e) == hipSuccess;
}
}  // namespace

bool timing_begin(hipStream_t st, TimedLaunch &t, int kind) {
  if (!g_timing) return false;
  if (!pooled_event(t.start)) return false;
  if (!pooled_event(t.stop)) {
    g_event_pool.push_back(t.start);
    return false;
  }
  t.kind = kind;
  (void)hipEventRecord(t.start, st);
  return true;
}

void timing_end(hipStream_t st, TimedLaunch &t) {
  (void)hipEventRecord(t.stop, st);
  g_timed.push_back(t);
}

void kernel_timing_enable(bool on) { g_timing = on; }

bool kernel_timing_read(int64_t *launches, double *ms) {
  for (int k = 0; k < kTimedKinds; ++k) {
    launches[k] = 0;
    ms[k] = 0.0;
  }
  bool ok = true;
  for (auto &t : g_timed) {
    float e = 0.f;
    if (hipEventSynchronize(t.stop) != hipSuccess || hipEventElapsedTime(&e, t.start, t.stop) != hipSuccess)
      ok = false;
    launches[t.kind] += 1;
    ms[t.kind] += e;
    g_event_pool.push_back(t.start);
    g_event_pool.push_back(t.stop);
  }
  g_timed.clear();
  return ok;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

LinearPlan plan_linear(int64_t T, int64_t N, int64_t K, int r, bool dropout) {
  LinearPlan p;
  p.T = T;
  p.N = N;
  p.K = K;
  p.r = r;
  p.dropout = dropout;
  // the four adapter-side products (see lora.hip): M x Nc outputs, contraction Kc
  const int64_t shapes[4][3] = {{T, r, K}, {T, r, N}, {r, K, T}, {N, r, T}};
  size_t part = 0;
  for (const auto &sh : shapes) part = std::max(part, lora_part_floats(sh[0], sh[1], sh[2]));
  // grad_A and grad_B are formed together
  part = std::max(part, lora_part_floats(r, K, T) + lora_part_floats(N, r, T));
  if (gemv_bwd_applies(T, N, K, 1))
    part = std::max(part, gemv_part_floats(T, N, K, r));
  else if (gemv_fwd_applies(T, N, K))  // the forward on the few-token kernels, the backward on the GEMMs
    part = std::max(part, gemv_fwd_part_floats(T, N, K, r));
  size_t off = 0;
  p.off_status = off;  // status word (never written by the linear calls)
  off = 256;
  p.off_u = off;
  off += align256((size_t)T * r * 2);
  p.off_v = off;
  off += align256((size_t)T * r * 2);
  p.off_part = off;
  off += align256(part * 4);
  // split contraction of the fused GEMMs (few tokens or a narrow output): fp32 partial tiles of the
  // forward (y) or of grad_x, whichever needs more
  p.off_qpart = off;
  if (!gemv_bwd_applies(T, N, K, 1))
    off += align256(std::max(qgemm_split_floats(T, N, K), qgemm_split_floats(T, K, N)) * 4);
  // dropout: keep words [ceil(T/32)][K] and the dropped-out input [T x K] bf16
  p.off_keep = p.off_xd = 0;
  if (dropout) {
    p.off_keep = off;
    off += align256(dropout_keep_words(T, K) * 4);
    p.off_xd = off;
    off += align256((size_t)T * K * 2);
  }
  p.total = off;
  return p;
}

// The adapter input of a call: x itself, or with dropout the masked copy the
// mask kernel writes into the workspace (with its keep words).
struct AdapterInput {
  const uint16_t *xa;
  const uint32_t *keep;
  float inv_keep;
  hipError_t err;
};

static AdapterInput adapter_input(const LinearPlan &p, const uint16_t *x, char *ws, const Dropout &d,
                                  hipStream_t st) {
  if (!d.on) return AdapterInput{x, nullptr, 1.0f, hipSuccess};
  uint32_t *keep = (uint32_t *)(ws + p.off_keep);
  uint16_t *xd = (uint16_t *)(ws + p.off_xd);
  const hipError_t e = launch_dropout_mask(x, p.T, p.K, d.thresh, d.seed, keep, xd, st);
  return AdapterInput{xd, keep, d.inv_keep, e};
}

hipError_t launch_linear_fwd(const LinearPlan &p, const uint16_t *x, const QWeight &w, const uint16_t *A,
                             const uint16_t *B, float scale, uint16_t *y, uint16_t *u_out, char *ws,
                             const Codebook &cb, hipStream_t st, const Dropout &d) {
  uint16_t *u = u_out ? u_out : (uint16_t *)(ws + p.off_u);
  float *part = (float *)(ws + p.off_part);
  const AdapterInput ai = adapter_input(p, x, ws, d, st);
  if (ai.err != hipSuccess) return ai.err;
  if (gemv_fwd_applies(p.T, p.N, p.K))
    return launch_gemv_fwd(p.T, x, ai.xa, w, A, B, p.r, scale, ai.inv_keep, y, u, part, cb, st);
  // u = bf16((1 / (1 - p)) xa A^T): the factor is exactly 1 without dropout
  hipError_t e = launch_lora(LoraKind::kU, ai.xa, p.K, A, p.K, p.T, p.r, p.K, ai.inv_keep, u, part, st);
  if (e != hipSuccess) return e;
  TimedLaunch tl;
  const bool timed = timing_begin(st, tl, kTimedQgemmFwd);
  e = launch_qgemm(false, x, p.T, p.N, p.K, w, u, B, p.r, scale, y, cb, st, nullptr, (float *)(ws + p.off_qpart));
  if (timed) timing_end(st, tl);
  return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_linear_bwd(const LinearPlan &p, const uint16_t *dy, const uint16_t *x, const QWeight &w,
                             const uint16_t *A, const uint16_t *B, float scale, const uint16_t *u,
                             uint16_t *grad_x, float *grad_A, float *grad_B, char *ws, const Codebook &cb,
                             hipStream_t st, const Dropout &d) {
  float *part = (float *)(ws + p.off_part);
  uint16_t *v = (uint16_t *)(ws + p.off_v);
  const AdapterInput ai = adapter_input(p, x, ws, d, st);  // the forward's mask, regenerated
  if (ai.err != hipSuccess) return ai.err;
  // grad_A and the adapter term of grad_x carry s / (1 - p); grad_B = s dy^T u
  const float scale_ax = scale * ai.inv_keep;
  hipError_t e;
  if (gemv_bwd_applies(p.T, p.N, p.K, 1)) {
    if (!u) {  // recompute u = (1 / (1 - p)) xa A^T
      uint16_t *uw = (uint16_t *)(ws + p.off_u);
      e = launch_gemv_fwd(p.T, x, ai.xa, w, A, B, p.r, scale, ai.inv_keep, nullptr, uw, part, cb, st);
      if (e != hipSuccess) return e;
      u = uw;
    }
    return launch_gemv_bwd(p.T, dy, ai.xa, w, A, B, p.r, scale, scale_ax, ai.keep, u, grad_x, grad_A, grad_B, part,
                           cb, st);
  }
  if (!u) {  // recompute u = (1 / (1 - p)) xa A^T
    uint16_t *uw = (uint16_t *)(ws + p.off_u);
    e = launch_lora(LoraKind::kU, ai.xa, p.K, A, p.K, p.T, p.r, p.K, ai.inv_keep, uw, part, st);
    if (e != hipSuccess) return e;
    u = uw;
  }
  // v = dy B
  e = launch_lora(LoraKind::kV, dy, p.N, B, p.r, p.T, p.r, p.N, 1.0f, v, part, st);
  if (e != hipSuccess) return e;
  if (grad_x) {  // grad_x = dy W_hat + keep (.) (s / (1 - p)) v A
    TimedLaunch tl;
    const bool timed = timing_begin(st, tl, kTimedQgemmDx);
    e = launch_qgemm(true, dy, p.T, p.K, p.N, w, v, A, p.r, scale_ax, grad_x, cb, st, ai.keep,
                     (float *)(ws + p.off_qpart));
    if (timed) timing_end(st, tl);
    if (e != hipSuccess) return e;
  }
  // grad_A = (s / (1 - p)) v^T xa [r x K] and grad_B = s dy^T u [N x r], one launch (and one
  // reduction) for both
  return launch_lora_grads(v, ai.xa, dy, u, p.T, p.N, p.K, p.r, scale_ax, scale, grad_A, grad_B, part,
                           lora_part_floats(p.r, p.K, p.T), st);
}

// ---------------------------------------------------------------------------
// Projection sets: linears that read the same input (q/k/v, gate/up).

SetPlan plan_linear_set(int64_t T, int count, const int64_t *N, int64_t K, int r) {
  SetPlan p;
  p.T = T;
  p.K = K;
  p.r = r;
  p.count = count;
  for (int i = 0; i < kMaxSetMembers; ++i) p.N[i] = i < count ? N[i] : 0;
  const size_t uv = align256((size_t)T * count * r * 2);
  size_t off = 256;
  p.off_u = off;
  off += uv;
  p.off_v = off;
  off += uv;
  p.off_part = off;
  int64_t ntot = 0;
  for (int i = 0; i < count; ++i) ntot += N[i];
  p.fwd_few = gemv_fwd_applies(T, ntot, K);
  p.bwd_few = gemv_bwd_applies(T, ntot, K, count);
  const bool fwd_few = p.fwd_few, bwd_few = p.bwd_few;
  size_t part = 0;
  if (fwd_few) {  // the few-token forward: the set pass's span partials or the largest member's
    part = gemv_set_fwd_part_floats(T, N, count, K, r);
    for (int i = 0; i < count; ++i) part = std::max(part, gemv_fwd_part_floats(T, N[i], K, r));
  }
  if (bwd_few) {  // the few-token backward pass
    part = std::max(part, gemv_set_part_floats(T, N, count, K, r));
    for (int i = 0; i < count; ++i) part = std::max(part, gemv_part_floats(T, N[i], K, r));
  }
  if (!fwd_few || !bwd_few)  // the adapter products of the direction(s) on the fused GEMM
    part = std::max(part, lora_set_part_floats(T, count, N, K, r));
  off += align256(part * 4);
  p.off_um = off;
  if (fwd_few || bwd_few) off += align256((size_t)T * r * 2);  // one [T x r] u block
  // grad_x of a set whose members share n_out may split its contraction (each
  // split contracts the same range of every member), and so may the forward
  // when every member's n_out is whole 128-column tiles (or the set has one
  // member): their fp32 partial tiles
  p.off_qpart = 0;
  bool same_n = !bwd_few, tiles_n = !fwd_few;
  int64_t n_all = 0;
  for (int i = 0; i < count; ++i) {
    same_n = same_n && N[i] == N[0];
    tiles_n = tiles_n && (count == 1 || N[i] % 128 == 0);
    n_all += N[i];
  }
  size_t qsplit = std::max(same_n ? qgemm_split_floats(T, K, N[0]) : 0,
                           tiles_n ? qgemm_split_floats(T, n_all, K) : 0);
  // at a few tokens a set may run member by member on the few-token tiles
  if (tiles_n)
    for (int i = 0; i < count; ++i) qsplit = std::max(qsplit, qgemm_split_floats(T, N[i], K));
  if (!bwd_few && count > 1) qsplit = std::max(qsplit, qgemm_set_dx_member_floats(T, count, N, K));
  if (qsplit) {
    p.off_qpart = off;
    off += align256(qsplit * 4);
  }
  p.total = off;
  return p;
}

// Few-token sets.  The forward (T <= kGemvFwdMaxT) runs as one pass over the
// members' concatenated rows when every member but the last has a multiple of
// 64 rows, else member by member (u moves between the set's [T x count r]
// layout and one [T x r] block); the backward (gemv_bwd_applies) is one pass
// over every member's rows, which sums grad_x over the members in its fp32
// partials.
static hipError_t set_fwd_few(const SetPlan &p, const uint16_t *x, const QWeight *w, const uint16_t *A_set,
                              const uint16_t *const *B, float scale, uint16_t *const *y, uint16_t *u, char *ws,
                              const Codebook &cb, hipStream_t st) {
  float *part = (float *)(ws + p.off_part);
  if (gemv_set_fusable(p.N, p.count))
    return launch_gemv_fwd_set(p.T, x, w, p.count, A_set, B, p.r, scale, y, u, part, cb, st);
  uint16_t *um = (uint16_t *)(ws + p.off_um);
  const int64_t rt = (int64_t)p.count * p.r;
  for (int i = 0; i < p.count; ++i) {
    hipError_t e = launch_gemv_fwd(p.T, x, x, w[i], A_set + (int64_t)i * p.r * p.K, B[i], p.r, scale, 1.0f, y[i], um,
                                   part, cb, st);
    if (e == hipSuccess) e = launch_copy_rows(um, p.r, u + (int64_t)i * p.r, rt, p.T, p.r, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static hipError_t set_bwd_few(const SetPlan &p, const uint16_t *const *dy, const uint16_t *x, const QWeight *w,
                              const uint16_t *A_set, const uint16_t *const *B, float scale, const uint16_t *u,
                              uint16_t *grad_x, float *grad_A_set, float *const *grad_B, char *ws, const Codebook &cb,
                              hipStream_t st) {
  float *part = (float *)(ws + p.off_part);
  if (!u) {  // recompute u_set member by member (u only), through one [T x r] block
    uint16_t *um = (uint16_t *)(ws + p.off_um), *us = (uint16_t *)(ws + p.off_u);
    const int64_t rt = (int64_t)p.count * p.r;
    for (int i = 0; i < p.count; ++i) {
      hipError_t e = launch_gemv_fwd(p.T, x, x, w[i], A_set + (int64_t)i * p.r * p.K, B[i], p.r, scale, 1.0f, nullptr, um,
                                     part, cb, st);
      if (e == hipSuccess) e = launch_copy_rows(um, p.r, us + (int64_t)i * p.r, rt, p.T, p.r, st);
      if (e != hipSuccess) return e;
    }
    u = us;
  }
  return launch_gemv_bwd_set(p.T, dy, x, w, p.count, A_set, B, p.r, scale, u, grad_x, grad_A_set, grad_B, part, cb, st);
}

hipError_t launch_linear_set_fwd(const SetPlan &p, const uint16_t *x, const QWeight *w, const uint16_t *A_set,
                                 const uint16_t *const *B, float scale, uint16_t *const *y, uint16_t *u_out, char *ws,
                                 const Codebook &cb, hipStream_t st) {
  uint16_t *u = u_out ? u_out : (uint16_t *)(ws + p.off_u);
  if (p.fwd_few) return set_fwd_few(p, x, w, A_set, B, scale, y, u, ws, cb, st);
  float *part = (float *)(ws + p.off_part);
  const int64_t rt = (int64_t)p.count * p.r;
  // u_set = x A_set^T: one product for every member's u
  hipError_t e = launch_lora(LoraKind::kU, x, p.K, A_set, p.K, p.T, rt, p.K, 1.0f, u, part, st);
  if (e != hipSuccess) return e;
  QgemmSet s{};
  s.count = p.count;
  s.ld_la = rt;
  for (int i = 0; i < p.count; ++i) {
    s.m[i].w = w[i];
    s.m[i].lb = B[i];
    s.m[i].out = y[i];
  }
  TimedLaunch tl;
  const bool timed = timing_begin(st, tl, kTimedQgemmFwd);
  e = launch_qgemm_set(false, s, p.T, x, u, nullptr, p.r, scale, nullptr, cb, st, nullptr,
                       p.off_qpart ? (float *)(ws + p.off_qpart) : nullptr);
  if (timed) timing_end(st, tl);
  return e;
}

hipError_t launch_linear_set_bwd(const SetPlan &p, const uint16_t *const *dy, const uint16_t *x, const QWeight *w,
                                 const uint16_t *A_set, const uint16_t *const *B, float scale, const uint16_t *u,
                                 uint16_t *grad_x, float *grad_A_set, float *const *grad_B, char *ws,
                                 const Codebook &cb, hipStream_t st) {
  if (p.bwd_few)
    return set_bwd_few(p, dy, x, w, A_set, B, scale, u, grad_x, grad_A_set, grad_B, ws, cb, st);
  float *part = (float *)(ws + p.off_part);
  uint16_t *v = (uint16_t *)(ws + p.off_v);
  const int64_t rt = (int64_t)p.count * p.r;
  hipError_t e;
  if (!u) {  // recompute u_set = x A_set^T
    uint16_t *uw = (uint16_t *)(ws + p.off_u);
    e = launch_lora(LoraKind::kU, x, p.K, A_set, p.K, p.T, rt, p.K, 1.0f, uw, part, st);
    if (e != hipSuccess) return e;
    u = uw;
  }
  // v_set: member i's columns = dy_i B_i
  e = launch_lora_set_v(dy, B, p.N, p.count, p.T, p.r, v, part, st);
  if (e != hipSuccess) return e;
  if (grad_x) {  // grad_x = sum_i dy_i W_hat_i + s v_set A_set: one GEMM contracting over every member
    QgemmSet s{};
    s.count = p.count;
    s.ld_la = rt;
    for (int i = 0; i < p.count; ++i) {
      s.m[i].w = w[i];
      s.m[i].act = dy[i];
    }
    TimedLaunch tl;
    const bool timed = timing_begin(st, tl, kTimedQgemmDx);
    e = launch_qgemm_set(true, s, p.T, nullptr, v, A_set, (int)rt, scale, grad_x, cb, st, nullptr,
                         p.off_qpart ? (float *)(ws + p.off_qpart) : nullptr);
    if (timed) timing_end(st, tl);
    if (e != hipSuccess) return e;
  }
  return launch_lora_set_grads(v, x, dy, u, p.N, p.count, p.T, p.K, p.r, scale, grad_A_set, grad_B, part, st);
}

}  // namespace qlora
