// QLoRA linear layer kernels for gfx950: dequant-fused bf16 MFMA GEMMs for
// the forward product and grad_x, and the LoRA side products.
//
// Method ("qlora" encyclopedia entry, tonho.wtf, section "a ideia"): the
// frozen 4-bit weight is dequantized to BFloat16 every time it enters a
// matrix product and is never kept in 16 bits; the gradient flows through it
// into the 16-bit adapters only.  Adapter algebra from the nexusinovation
// tutorial, section "LoRA: O Padrão Ouro de Eficiência": W' = W + s.B.A.
//
//   y      = x W_hat^T + s (x A^T) B^T        qgemm.hip (forward form) + nt_splitk for u
//   grad_x = dy W_hat + s (dy B) A            qgemm.hip (transposed form) + nt_splitk for v
//   grad_A = s (dy B)^T x                     tn_split + reduce_splits
//   grad_B = s dy^T (x A^T)                   tn_split + reduce_splits
//
// MFMA lane layouts used (v_mfma_f32_32x32x16_bf16, 64 lanes, l = lane):
//   A operand: lane l holds A[i = l%32][k = 8(l/32) .. 8(l/32)+7]
//   B operand: lane l holds B[k = 8(l/32) .. +7][j = l%32]
//   D:         lane l, register q holds D[8(q/4) + 4(l/32) + q%4][l%32]

#include <vector>

#include "common.hpp"
#include "launch.hpp"

namespace qlora {

// 8 consecutive bf16 of one row at columns [c, c + 8); zero at columns >= ncols.
__device__ __forceinline__ u32x4 load8(const uint16_t *row, int64_t c, int64_t ncols, bool vec) {
  if (vec && c + 8 <= ncols) return *(const u32x4 *)(row + c);
  u32x4 v = {0u, 0u, 0u, 0u};
  for (int i = 0; i < 8; ++i)
    if (c + i < ncols) v[i >> 1] |= (uint32_t)row[c + i] << (16 * (i & 1));
  return v;
}

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// part[s][m][j] = sum over k in chunk s of P[m][k] Q[j][k]   (P [M x Kc], Q [R x Kc])
// Workgroup tile 64 x 64 (4 waves of 32 x 32); operands straight from global
// memory in MFMA layout.
__global__ __launch_bounds__(256) void nt_splitk(const uint16_t *__restrict__ P, const uint16_t *__restrict__ Q,
                                                 int64_t M, int64_t R, int64_t Kc, int64_t kchunk,
                                                 float *__restrict__ part) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, lhi = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * 64, j0 = (int64_t)blockIdx.y * 64, s = blockIdx.z;
  const int64_t kb = s * kchunk, ke = min(Kc, kb + kchunk);
  const int64_t row = m0 + wm * 32 + l32, jr = j0 + wn * 32 + l32;
  const bool vec = (Kc % 8) == 0;
  f32x16 acc;
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.f;
  for (int64_t k = kb; k < ke; k += 64) {
    u32x4 a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t kc = k + 16 * u + 8 * lhi;
      a[u] = (row < M) ? load8(P + row * Kc, kc, ke, vec) : u32x4{0u, 0u, 0u, 0u};
      b[u] = (jr < R) ? load8(Q + jr * Kc, kc, ke, vec) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = mfma32(a[u], b[u], acc);
  }
  const int64_t jo = j0 + wn * 32 + l32;
  if (jo < R) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t m = m0 + wm * 32 + 8 * (q >> 2) + 4 * lhi + (q & 3);
      if (m < M) part[(s * M + m) * R + jo] = acc[q];
    }
  }
}

// ---------------------------------------------------------------------------
// part[s][m][n] = sum over t in chunk s of P[t][m] Q[t][n]   (P [T x Mp], Q [T x Np])
// 32-token slices of P and Q are transposed through LDS so that the token
// index becomes the MFMA contraction.
constexpr int TLD = 40;
__global__ __launch_bounds__(256) void tn_split(const uint16_t *__restrict__ P, const uint16_t *__restrict__ Q,
                                                int64_t T, int64_t Mp, int64_t Np, int64_t tchunk,
                                                float *__restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t sp[64 * TLD];
  __shared__ __attribute__((aligned(16))) uint16_t sq[64 * TLD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, lhi = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * 64, n0 = (int64_t)blockIdx.y * 64, s = blockIdx.z;
  const int64_t tb = s * tchunk, te = min(T, tb + tchunk);
  const int tl = tid >> 3, c8 = 8 * (tid & 7);
  const bool vp = (Mp % 8) == 0, vq = (Np % 8) == 0;
  f32x16 acc;
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.f;
  for (int64_t t = tb; t < te; t += 32) {
    const int64_t trow = t + tl;
    const u32x4 pv = (trow < te) ? load8(P + trow * Mp, m0 + c8, Mp, vp) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 qv = (trow < te) ? load8(Q + trow * Np, n0 + c8, Np, vq) : u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sp[(c8 + i) * TLD + tl] = (uint16_t)(pv[i >> 1] >> (16 * (i & 1)));
      sq[(c8 + i) * TLD + tl] = (uint16_t)(qv[i >> 1] >> (16 * (i & 1)));
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4 a = *(const u32x4 *)&sp[(wm * 32 + l32) * TLD + kk * 16 + 8 * lhi];
      const u32x4 b = *(const u32x4 *)&sq[(wn * 32 + l32) * TLD + kk * 16 + 8 * lhi];
      acc = mfma32(a, b, acc);
    }
  }
  const int64_t no = n0 + wn * 32 + l32;
  if (no < Np) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t m = m0 + wm * 32 + 8 * (q >> 2) + 4 * lhi + (q & 3);
      if (m < Mp) part[(s * Mp + m) * Np + no] = acc[q];
    }
  }
}

// out[i] = scale * sum_s part[s][i], in a fixed order (deterministic).
template <bool kBf16Out>
__global__ __launch_bounds__(256) void reduce_splits(const float *__restrict__ part, int S, int64_t count,
                                                     float scale, void *__restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
    float acc = 0.f;
    for (int s = 0; s < S; ++s) acc += part[s * count + i];
    acc *= scale;
    if (kBf16Out) {
      __bf16 h = (__bf16)acc;
      ((uint16_t *)out)[i] = __builtin_bit_cast(uint16_t, h);
    } else {
      ((float *)out)[i] = acc;
    }
  }
}

// out [C x R] = in [R x C]^T (bf16), 32 x 32 tiles through LDS.
__global__ __launch_bounds__(256) void transpose_bf16(const uint16_t *__restrict__ in, int64_t R, int64_t C,
                                                      uint16_t *__restrict__ out) {
  __shared__ uint16_t t[32][33];
  const int64_t r0 = (int64_t)blockIdx.y * 32, c0 = (int64_t)blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int k = ty; k < 32; k += 8)
    if (r0 + k < R && c0 + tx < C) t[k][tx] = in[(r0 + k) * C + c0 + tx];
  __syncthreads();
  for (int k = ty; k < 32; k += 8)
    if (c0 + k < C && r0 + tx < R) out[(c0 + k) * R + r0 + tx] = t[tx][k];
}

__global__ void set_word(uint32_t *p, uint32_t v) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *p = v;
}

// ---------------------------------------------------------------------------
// host side

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- diagnostics: HIP events around the fused GEMM launches
namespace {
struct TimedLaunch {
  hipEvent_t start, stop;
  bool dx;
};
bool g_timing = false;
std::vector<TimedLaunch> g_timed;

bool timing_begin(hipStream_t st, TimedLaunch &t, bool dx) {
  if (!g_timing) return false;
  if (hipEventCreate(&t.start) != hipSuccess) return false;
  if (hipEventCreate(&t.stop) != hipSuccess) {
    (void)hipEventDestroy(t.start);
    return false;
  }
  t.dx = dx;
  (void)hipEventRecord(t.start, st);
  return true;
}

void timing_end(hipStream_t st, TimedLaunch &t) {
  (void)hipEventRecord(t.stop, st);
  g_timed.push_back(t);
}
}  // namespace

void gemm_timing_enable(bool on) { g_timing = on; }

bool gemm_timing_read(int64_t *fwd_n, double *fwd_ms, int64_t *dx_n, double *dx_ms) {
  int64_t n[2] = {0, 0};
  double ms[2] = {0.0, 0.0};
  bool ok = true;
  for (auto &t : g_timed) {
    float e = 0.f;
    if (hipEventSynchronize(t.stop) != hipSuccess || hipEventElapsedTime(&e, t.start, t.stop) != hipSuccess)
      ok = false;
    n[t.dx] += 1;
    ms[t.dx] += e;
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  g_timed.clear();
  if (fwd_n) *fwd_n = n[0];
  if (fwd_ms) *fwd_ms = ms[0];
  if (dx_n) *dx_n = n[1];
  if (dx_ms) *dx_ms = ms[1];
  return ok;
}
static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Number of splits of a reduction of length `len` (in units of `unit`) so that
// tiles * splits is about 512 workgroups.
static int choose_splits(int64_t tiles, int64_t len, int64_t unit) {
  int64_t maxs = cdiv(len, unit);
  int64_t s = cdiv(512, tiles);
  if (s > maxs) s = maxs;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  // make every split non-empty with a chunk that is a whole number of units
  const int64_t chunk = cdiv(cdiv(len, s), unit) * unit;
  return (int)cdiv(len, chunk);
}

static int64_t chunk_of(int64_t len, int s, int64_t unit) { return cdiv(cdiv(len, s), unit) * unit; }

LinearPlan plan_linear(int64_t T, int64_t N, int64_t K, int r) {
  LinearPlan p;
  p.T = T;
  p.N = N;
  p.K = K;
  p.r = r;
  const int64_t tr = cdiv(T, 64) * cdiv(r, 64);
  p.s_u = choose_splits(tr, K, 64);
  p.s_v = choose_splits(tr, N, 64);
  p.s_ga = choose_splits(cdiv(r, 64) * cdiv(K, 64), T, 32);
  p.s_gb = choose_splits(cdiv(N, 64) * cdiv(r, 64), T, 32);
  size_t off = 0;
  p.off_status = off;
  off += 256;
  p.off_u = off;
  off += align256((size_t)T * r * 2);
  p.off_v = off;
  off += align256((size_t)T * r * 2);
  p.off_bt = off;
  off += align256((size_t)N * r * 2);
  p.off_at = off;
  off += align256((size_t)K * r * 2);
  p.off_part = off;
  size_t part = (size_t)p.s_u * T * r;
  part = std::max(part, (size_t)p.s_v * T * r);
  part = std::max(part, (size_t)p.s_ga * r * K);
  part = std::max(part, (size_t)p.s_gb * N * r);
  off += align256(part * 4);
  p.total = off;
  return p;
}

static void launch_reduce(const float *part, int S, int64_t count, float scale, void *out, bool bf16,
                          hipStream_t st) {
  int64_t g = cdiv(count, 256);
  if (g > 4096) g = 4096;
  if (bf16)
    reduce_splits<true><<<(unsigned)g, 256, 0, st>>>(part, S, count, scale, out);
  else
    reduce_splits<false><<<(unsigned)g, 256, 0, st>>>(part, S, count, scale, out);
}

// u = x A^T (bf16 [T x r]) via split-K partials.
static void launch_u(const LinearPlan &p, const uint16_t *x, const uint16_t *A, uint16_t *u, float *part,
                     hipStream_t st) {
  const int64_t kchunk = chunk_of(p.K, p.s_u, 64);
  dim3 g((unsigned)cdiv(p.T, 64), (unsigned)cdiv(p.r, 64), (unsigned)p.s_u);
  nt_splitk<<<g, 256, 0, st>>>(x, A, p.T, p.r, p.K, kchunk, part);
  launch_reduce(part, p.s_u, p.T * p.r, 1.0f, u, true, st);
}

hipError_t launch_linear_fwd(const LinearPlan &p, const uint16_t *x, const QWeight &w, const uint16_t *A,
                             const uint16_t *B, float scale, uint16_t *y, uint16_t *u_out, char *ws,
                             const Codebook &cb, hipStream_t st) {
  uint16_t *u = u_out ? u_out : (uint16_t *)(ws + p.off_u);
  float *part = (float *)(ws + p.off_part);
  set_word<<<1, 64, 0, st>>>((uint32_t *)(ws + p.off_status), 0u);
  launch_u(p, x, A, u, part, st);
  TimedLaunch tl;
  const bool timed = timing_begin(st, tl, false);
  const hipError_t e = launch_qgemm(false, x, p.T, p.N, p.K, w, u, B, p.r, scale, y, cb, st);
  if (timed) timing_end(st, tl);
  return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_linear_bwd(const LinearPlan &p, const uint16_t *dy, const uint16_t *x, const QWeight &w,
                             const uint16_t *A, const uint16_t *B, float scale, const uint16_t *u,
                             uint16_t *grad_x, float *grad_A, float *grad_B, char *ws, const Codebook &cb,
                             hipStream_t st) {
  float *part = (float *)(ws + p.off_part);
  uint16_t *v = (uint16_t *)(ws + p.off_v);
  uint16_t *bt = (uint16_t *)(ws + p.off_bt);
  set_word<<<1, 64, 0, st>>>((uint32_t *)(ws + p.off_status), 0u);
  if (!u) {
    uint16_t *uw = (uint16_t *)(ws + p.off_u);
    launch_u(p, x, A, uw, part, st);
    u = uw;
  }
  // v = dy B = dy (B^T)^T
  transpose_bf16<<<dim3((unsigned)cdiv(p.r, 32), (unsigned)cdiv(p.N, 32)), 256, 0, st>>>(B, p.N, p.r, bt);
  {
    const int64_t kchunk = chunk_of(p.N, p.s_v, 64);
    dim3 g((unsigned)cdiv(p.T, 64), (unsigned)cdiv(p.r, 64), (unsigned)p.s_v);
    nt_splitk<<<g, 256, 0, st>>>(dy, bt, p.T, p.r, p.N, kchunk, part);
    launch_reduce(part, p.s_v, p.T * p.r, 1.0f, v, true, st);
  }
  if (grad_x) {
    TimedLaunch tl;
    const bool timed = timing_begin(st, tl, true);
    const hipError_t e = launch_qgemm(true, dy, p.T, p.K, p.N, w, v, A, p.r, scale, grad_x, cb, st);
    if (timed) timing_end(st, tl);
    if (e != hipSuccess) return e;
  }
  {  // grad_A = s v^T x   [r x K]
    const int64_t tchunk = chunk_of(p.T, p.s_ga, 32);
    dim3 g((unsigned)cdiv(p.r, 64), (unsigned)cdiv(p.K, 64), (unsigned)p.s_ga);
    tn_split<<<g, 256, 0, st>>>(v, x, p.T, p.r, p.K, tchunk, part);
    launch_reduce(part, p.s_ga, (int64_t)p.r * p.K, scale, grad_A, false, st);
  }
  {  // grad_B = s dy^T u   [N x r]
    const int64_t tchunk = chunk_of(p.T, p.s_gb, 32);
    dim3 g((unsigned)cdiv(p.N, 64), (unsigned)cdiv(p.r, 64), (unsigned)p.s_gb);
    tn_split<<<g, 256, 0, st>>>(dy, u, p.T, p.N, p.r, tchunk, part);
    launch_reduce(part, p.s_gb, p.N * (int64_t)p.r, scale, grad_B, false, st);
  }
  return hipGetLastError();
}

}  // namespace qlora
