// AdamW update of the LoRA adapters, one pass over a flat fp32 buffer.
//
// Only the adapters train; for each trained value the optimizer holds two
// moments ("LoRA vs. QLoRA vs. Full Fine-Tuning", section "Quanta VRAM cada
// método precisa?"), and those states may sit in host memory that the update
// reads in place ("qlora" entry, section "como funciona": paged optimizers).
// The update is AdamW (Loshchilov and Hutter, decoupled weight decay) with
// fp32 moments and an fp32 master copy; every operation is one fp32 operation
// with one rounding, in this order (no contraction: the library is built with
// -ffp-contract=off, and division and square root are correctly rounded):
//
//   m <- b1 m + c_m g          v <- b2 v + c_v (g g)
//   d  = sqrt(v) / bc2_sqrt + eps
//   p <- p decay;   p <- p - step_size (m / d);   p_bf16 = bf16_rne(p)
//
// The step-dependent scalars arrive precomputed (host, fp64, rounded once).
//
// The pass is HBM-bound: 16 bytes read and 12 + 2 written per element when
// the states are in device memory.  Each thread takes kVec groups of four
// consecutive elements, one 16-byte access per array per group, all loads
// issued before any arithmetic; consecutive lanes take consecutive groups so
// a wave touches 1 KiB contiguous runs of every array.  Every access is
// non-temporal: each byte is touched once, so nothing is kept in the caches
// (measured: 5.6 TB/s against 5.35 TB/s with ordinary accesses, and 5.69 TB/s
// for a kernel with the same eight streams and no arithmetic).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "launch.hpp"

namespace qlora {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;                                   // float4 groups per thread
constexpr int64_t kTileElems = (int64_t)kThreads * kVec * 4;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float adamw_one(float &p, float g, float &m, float &v, const AdamwScalars &s) {
  const float mn = s.b1 * m + s.c_m * g;
  const float gg = g * g;
  const float vn = s.b2 * v + s.c_v * gg;
  const float d = __builtin_sqrtf(vn) / s.bc2_sqrt + s.eps;
  float pn = p * s.decay;
  const float r = mn / d;
  pn = pn - s.step_size * r;
  m = mn;
  v = vn;
  p = pn;
  return pn;
}

// Full tiles only: every element of [tile * kTileElems, +kTileElems) exists.
__global__ __launch_bounds__(kThreads) void adamw_full(float *__restrict__ param, uint16_t *__restrict__ pbf,
                                                      const float *__restrict__ grad, float *__restrict__ m1,
                                                      float *__restrict__ m2, AdamwScalars s) {
  const int64_t base = (int64_t)blockIdx.x * kTileElems;
  f32x4 p[kVec], g[kVec], m[kVec], v[kVec];
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const int64_t e = base + ((int64_t)j * kThreads + threadIdx.x) * 4;
    p[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(param + e));
    g[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(grad + e));
    m[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(m1 + e));
    v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(m2 + e));
  }
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const int64_t e = base + ((int64_t)j * kThreads + threadIdx.x) * 4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float pc = p[j][c], mc = m[j][c], vc = v[j][c];
      adamw_one(pc, g[j][c], mc, vc, s);
      p[j][c] = pc;
      m[j][c] = mc;
      v[j][c] = vc;
    }
    const u32x2v b = {pack_bf16x2(p[j][0], p[j][1]), pack_bf16x2(p[j][2], p[j][3])};
    __builtin_nontemporal_store(p[j], reinterpret_cast<f32x4 *>(param + e));
    __builtin_nontemporal_store(m[j], reinterpret_cast<f32x4 *>(m1 + e));
    __builtin_nontemporal_store(v[j], reinterpret_cast<f32x4 *>(m2 + e));
    __builtin_nontemporal_store(b, reinterpret_cast<u32x2v *>(pbf + e));
  }
}

// The ragged end: elements [first, n), one per thread, scalar accesses.
__global__ __launch_bounds__(kThreads) void adamw_tail(float *__restrict__ param, uint16_t *__restrict__ pbf,
                                                      const float *__restrict__ grad, float *__restrict__ m1,
                                                      float *__restrict__ m2, int64_t first, int64_t n,
                                                      AdamwScalars s) {
  const int64_t e = first + (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (e >= n) return;
  float p = param[e], m = m1[e], v = m2[e];
  adamw_one(p, grad[e], m, v, s);
  param[e] = p;
  m1[e] = m;
  m2[e] = v;
  pbf[e] = (uint16_t)(pack_bf16x2(p, 0.0f) & 0xFFFFu);
}

}  // namespace

hipError_t launch_adamw(float *param, uint16_t *param_bf16, const float *grad, float *exp_avg, float *exp_avg_sq,
                        int64_t n, const AdamwScalars &s, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t tiles = n / kTileElems;
  const int64_t first = tiles * kTileElems;
  TimedLaunch tl;
  const bool timed = tiles > 0 && timing_begin(st, tl, kTimedAdamw);
  if (tiles > 0)
    hipLaunchKernelGGL(adamw_full, dim3((unsigned)tiles), dim3(kThreads), 0, st, param, param_bf16, grad, exp_avg,
                       exp_avg_sq, s);
  if (timed) timing_end(st, tl);
  if (first < n) {
    const int64_t rest = n - first;
    hipLaunchKernelGGL(adamw_tail, dim3((unsigned)((rest + kThreads - 1) / kThreads)), dim3(kThreads), 0, st, param,
                       param_bf16, grad, exp_avg, exp_avg_sq, first, n, s);
  }
  return hipGetLastError();
}

}  // namespace qlora
