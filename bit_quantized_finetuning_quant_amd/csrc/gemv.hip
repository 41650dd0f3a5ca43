// Few-token (T <= 2) QLoRA linear layer for gfx950: reading the 4-bit weight
// from HBM is the bound, so each weight is decoded once and used for all T
// tokens with vector ALU dot products.
//
// Method ("qlora" encyclopedia entry, tonho.wtf, section "a ideia"): the weight
// is dequantized to BFloat16 as it is used; gradients reach only the LoRA
// adapters.  W' = W + s.B.A (nexusinovation tutorial, section "LoRA: O Padrão
// Ouro de Eficiência").  Decoded values are bit-identical to the dequantizer:
// w_hat = bf16_rne(fl32(CB[code] * c1hat)).
//
//   gemv_u            u = x A^T                      (one workgroup per adapter row)
//   gemv_fwd          y = x W_hat^T + s u B^T        (a wave per weight row, a lane per NF4 block)
//   gemv_v            v = dy B and grad_B = s dy^T u (one workgroup per 8 adapter columns)
//   gemv_bwd_partial  partial grad_x = dy W_hat      (a workgroup per 64-column block slab and
//                                                     row chunk, a thread per weight row)
//   gemv_bwd_finish   grad_x = sum of chunk partials + s v A, grad_A = s v^T x

#include "common.hpp"
#include "launch.hpp"

namespace qlora {

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float bf(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t to_bf16(float v) {
  __bf16 h = (__bf16)v;
  return __builtin_bit_cast(uint16_t, h);
}

// Decode the 64 elements of one NF4 block (32 code bytes) into 32 bf16 pairs.
__device__ __forceinline__ void decode_block(const u32x4 (&c)[2], float ch, const float *lut, uint32_t (&w)[32]) {
  float lv[64];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int j = 0; j < 8; ++j) lv[32 * h + 8 * v + j] = lut[(c[h][v] >> (4 * j)) & 15u];
#pragma unroll
  for (int p = 0; p < 32; ++p) w[p] = pack_bf16x2(decode_product(lv[2 * p], ch), decode_product(lv[2 * p + 1], ch));
}

struct BlockLoad {
  u32x4 c[2];
  uint32_t q;
  float s2;
};

__device__ __forceinline__ void load_block(const QWeight &w, int64_t n, int64_t b, int64_t kblk_row, BlockLoad &L) {
  const uint8_t *src = w.codes + n * (w.n_in / 2) + b * 32;
  L.c[0] = *(const u32x4 *)src;
  L.c[1] = *(const u32x4 *)(src + 16);
  const int64_t blk = n * kblk_row + b;
  L.q = w.fp8[blk];
  L.s2 = w.s2[blk >> 8];
}

// ---------------------------------------------------------------------------
template <int T>
__global__ __launch_bounds__(256) void gemv_u(const uint16_t *__restrict__ x, int64_t K,
                                              const uint16_t *__restrict__ A, int r, uint16_t *__restrict__ u) {
  __shared__ float red[4][T];
  const int j = blockIdx.x, tid = threadIdx.x;
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.f;
  for (int64_t k = 8 * (int64_t)tid; k < K; k += 8 * 256) {
    const u32x4 a = *(const u32x4 *)(A + (int64_t)j * K + k);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const u32x4 xv = *(const u32x4 *)(x + t * K + k);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t] = dot2(a[e], xv[e], acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const float s = wave_sum(acc[t]);
    if ((tid & 63) == 0) red[tid >> 6][t] = s;
  }
  __syncthreads();
  if (tid < T) u[tid * r + j] = to_bf16(red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid]);
}

// ---------------------------------------------------------------------------
// y: each wave owns weight rows; lane l owns NF4 blocks l, l + 64, ... of a
// row.  x is staged in LDS; the next row's codes are fetched while the
// current row is decoded.
template <int T>
__global__ __launch_bounds__(256) void gemv_fwd(const uint16_t *__restrict__ x, QWeight w,
                                                const uint16_t *__restrict__ u, const uint16_t *__restrict__ B,
                                                int r, float scale, uint16_t *__restrict__ y, int64_t rows_per_wg,
                                                Codebook cb) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [T][K]
  __shared__ float lut[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t K = w.n_in, N = w.n_out, kblk_row = K / kBlock;
  if (tid < 16) lut[tid] = cb.v[tid];
  for (int64_t i = 8 * (int64_t)tid; i < T * K; i += 8 * 256) *(u32x4 *)&xs[i] = *(const u32x4 *)(x + i);
  __syncthreads();
  const float mu = *w.mu;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg, r1 = min(N, r0 + rows_per_wg);
  for (int64_t n = r0 + wave; n < r1; n += 4) {
    float acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.f;
    BlockLoad L;
    if (lane < kblk_row) load_block(w, n, lane, kblk_row, L);
    for (int64_t b = lane; b < kblk_row; b += 64) {
      BlockLoad cur = L;
      if (b + 64 < kblk_row) load_block(w, n, b + 64, kblk_row, L);
      uint32_t wv[32];
      decode_block(cur.c, decode_constant(cur.q, cur.s2, mu), lut, wv);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const u32x4 *xp = (const u32x4 *)&xs[t * K + 64 * b];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const u32x4 xv = xp[v];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t] = dot2(wv[4 * v + e], xv[e], acc[t]);
        }
      }
    }
    // LoRA term: lane j adds scale * u[t][j] * B[n][j] (j = lane, lane + 64, ...)
    for (int j = lane; j < r; j += 64) {
      const float bnj = bf(B[n * r + j]);
#pragma unroll
      for (int t = 0; t < T; ++t) acc[t] += scale * bf(u[t * r + j]) * bnj;
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float s = wave_sum(acc[t]);
      if (lane == 0) y[t * N + n] = to_bf16(s);
    }
  }
}

// v = dy B (fp32, [T x r]) and grad_B = s dy^T u: workgroup g owns adapter
// columns [8 g, 8 g + 8); thread t walks weight rows t, t + 256, ...
template <int T>
__global__ __launch_bounds__(256) void gemv_v(const uint16_t *__restrict__ dy, int64_t N,
                                              const uint16_t *__restrict__ B, const uint16_t *__restrict__ u, int r,
                                              float scale, float *__restrict__ v, float *__restrict__ grad_B) {
  __shared__ float red[256][T * 8 + 1];
  const int tid = threadIdx.x;
  const int j0 = 8 * blockIdx.x;
  float uj[T][8];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) uj[t][e] = (j0 + e < r) ? bf(u[t * r + j0 + e]) : 0.f;
  float acc[T][8];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;
  const bool vec = (r % 8) == 0;
  for (int64_t n = tid; n < N; n += 256) {
    float b[8];
    if (vec) {
      const u32x4 bv = *(const u32x4 *)(B + n * r + j0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        b[2 * e] = bf16_lo(bv[e]);
        b[2 * e + 1] = bf16_hi(bv[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = (j0 + e < r) ? bf(B[n * r + j0 + e]) : 0.f;
    }
    float d[T];
#pragma unroll
    for (int t = 0; t < T; ++t) d[t] = bf(dy[t * N + n]);
    float gb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      gb[e] = 0.f;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        acc[t][e] = __builtin_fmaf(d[t], b[e], acc[t][e]);
        gb[e] = __builtin_fmaf(d[t], uj[t][e], gb[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (j0 + e < r) grad_B[n * r + j0 + e] = scale * gb[e];
  }
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tid][t * 8 + e] = acc[t][e];
  __syncthreads();
  if (tid < T * 8) {
    float s = 0.f;
    for (int i = 0; i < 256; ++i) s += red[i][tid];  // fixed order
    const int t = tid / 8, e = tid % 8;
    if (j0 + e < r) v[t * r + j0 + e] = s;
  }
}

// ---------------------------------------------------------------------------
// Backward, pass 1: partial grad_x = dy W_hat.  Workgroup (slab, chunk) owns
// the 64 columns of NF4 block `slab` of every row and the weight rows of
// `chunk`; thread t takes rows r0 + t, r0 + t + 256, ... (two rows of loads in
// flight), accumulating 64 column sums per token.  The 256 threads' sums are
// added in thread order through LDS and written as this chunk's partial.
template <int T>
__global__ __launch_bounds__(256) void gemv_bwd_partial(const uint16_t *__restrict__ dy, QWeight w,
                                                        int64_t rows_per_chunk, float *__restrict__ gx_part,
                                                        Codebook cb) {
  extern __shared__ __attribute__((aligned(16))) float red[];  // [T * 64][256 + 1]
  __shared__ float lut[16];
  const int tid = threadIdx.x;
  const int64_t K = w.n_in, N = w.n_out, kblk_row = K / kBlock;
  const int64_t slab = blockIdx.x, chunk = blockIdx.y;
  if (tid < 16) lut[tid] = cb.v[tid];
  __syncthreads();
  const float mu = *w.mu;
  const int64_t r0 = chunk * rows_per_chunk, r1 = min(N, r0 + rows_per_chunk);
  float acc[T][64];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int e = 0; e < 64; ++e) acc[t][e] = 0.f;
  BlockLoad L;
  if (r0 + tid < r1) load_block(w, r0 + tid, slab, kblk_row, L);
  for (int64_t n = r0 + tid; n < r1; n += 256) {
    BlockLoad cur = L;
    if (n + 256 < r1) load_block(w, n + 256, slab, kblk_row, L);
    float d[T];
#pragma unroll
    for (int t = 0; t < T; ++t) d[t] = bf(dy[t * N + n]);
    uint32_t wv[32];
    decode_block(cur.c, decode_constant(cur.q, cur.s2, mu), lut, wv);
#pragma unroll
    for (int p = 0; p < 32; ++p)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        acc[t][2 * p] = __builtin_fmaf(bf16_lo(wv[p]), d[t], acc[t][2 * p]);
        acc[t][2 * p + 1] = __builtin_fmaf(bf16_hi(wv[p]), d[t], acc[t][2 * p + 1]);
      }
  }
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int e = 0; e < 64; ++e) red[(t * 64 + e) * 257 + tid] = acc[t][e];
  __syncthreads();
  if (tid < T * 64) {
    float s = 0.f;
    for (int i = 0; i < 256; ++i) s += red[tid * 257 + i];  // thread order
    const int t = tid / 64, e = tid % 64;
    gx_part[(chunk * T + t) * K + 64 * slab + e] = s;
  }
}

// Backward, pass 2: one thread per column of grad_x.
template <int T>
__global__ __launch_bounds__(256) void gemv_bwd_finish(const float *__restrict__ gx_part, int64_t chunks,
                                                       const float *__restrict__ v, const uint16_t *__restrict__ x,
                                                       const uint16_t *__restrict__ A, int r, int64_t K, float scale,
                                                       uint16_t *__restrict__ grad_x, float *__restrict__ grad_A) {
  __shared__ float vs[T][256];
  const int tid = threadIdx.x;
  for (int idx = tid; idx < T * r; idx += 256) vs[idx / r][idx % r] = v[idx];
  __syncthreads();
  const int64_t col = (int64_t)blockIdx.x * 256 + tid;
  if (col >= K) return;
  float g[T];
#pragma unroll
  for (int t = 0; t < T; ++t) g[t] = 0.f;
  for (int64_t c = 0; c < chunks; ++c)
#pragma unroll
    for (int t = 0; t < T; ++t) g[t] += gx_part[(c * T + t) * K + col];
  float xv[T];
#pragma unroll
  for (int t = 0; t < T; ++t) xv[t] = bf(x[t * K + col]);
  for (int j = 0; j < r; ++j) {
    const float a = bf(A[(int64_t)j * K + col]);
    float ga = 0.f;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      g[t] = __builtin_fmaf(scale * vs[t][j], a, g[t]);
      ga = __builtin_fmaf(vs[t][j], xv[t], ga);
    }
    grad_A[(int64_t)j * K + col] = scale * ga;
  }
#pragma unroll
  for (int t = 0; t < T; ++t) grad_x[t * K + col] = to_bf16(g[t]);
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

bool gemv_applies(int64_t T, int64_t K) { return T <= kGemvMaxT && (size_t)T * K * 2 <= 96 * 1024; }

// Row chunks of the transposed pass: about 256 workgroups over (blocks x chunks).
int64_t gemv_chunks(int64_t N, int64_t K) {
  const int64_t slabs = K / kBlock;
  int64_t chunks = cdiv(256, slabs);
  if (chunks > cdiv(N, 256)) chunks = cdiv(N, 256);
  return chunks < 1 ? 1 : chunks;
}

static void raise_lds_limit(const void *fn, size_t bytes) {
  if (bytes > 64 * 1024) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_gemv_u(int64_t T, const uint16_t *x, int64_t K, const uint16_t *A, int r, uint16_t *u,
                         hipStream_t st) {
  if (T == 1)
    gemv_u<1><<<r, 256, 0, st>>>(x, K, A, r, u);
  else
    gemv_u<2><<<r, 256, 0, st>>>(x, K, A, r, u);
  return hipGetLastError();
}

hipError_t launch_gemv_fwd(int64_t T, const uint16_t *x, const QWeight &w, const uint16_t *A, const uint16_t *B,
                           int r, float scale, uint16_t *y, uint16_t *u, const Codebook &cb, hipStream_t st) {
  const int64_t N = w.n_out, K = w.n_in;
  const int64_t rows_per_wg = 16;
  const unsigned g = (unsigned)cdiv(N, rows_per_wg);
  const size_t lds = (size_t)T * K * 2;
  if (T == 1) {
    raise_lds_limit((const void *)gemv_fwd<1>, lds);
    gemv_u<1><<<r, 256, 0, st>>>(x, K, A, r, u);
    gemv_fwd<1><<<g, 256, lds, st>>>(x, w, u, B, r, scale, y, rows_per_wg, cb);
  } else {
    raise_lds_limit((const void *)gemv_fwd<2>, lds);
    gemv_u<2><<<r, 256, 0, st>>>(x, K, A, r, u);
    gemv_fwd<2><<<g, 256, lds, st>>>(x, w, u, B, r, scale, y, rows_per_wg, cb);
  }
  return hipGetLastError();
}

hipError_t launch_gemv_bwd(int64_t T, const uint16_t *dy, const uint16_t *x, const QWeight &w, const uint16_t *A,
                           const uint16_t *B, int r, float scale, const uint16_t *u, uint16_t *grad_x,
                           float *grad_A, float *grad_B, float *gx_part, float *v, const Codebook &cb,
                           hipStream_t st) {
  const int64_t N = w.n_out, K = w.n_in;
  const int64_t slabs = K / kBlock;
  const int64_t chunks = gemv_chunks(N, K);
  const int64_t rows_per_chunk = cdiv(N, chunks);
  dim3 g1((unsigned)slabs, (unsigned)chunks);
  const size_t lds = (size_t)T * 64 * 257 * 4;
  const unsigned gv = (unsigned)cdiv(r, 8);
  const unsigned g2 = (unsigned)cdiv(K, 256);
  if (T == 1) {
    raise_lds_limit((const void *)gemv_bwd_partial<1>, lds);
    gemv_v<1><<<gv, 256, 0, st>>>(dy, N, B, u, r, scale, v, grad_B);
    gemv_bwd_partial<1><<<g1, 256, lds, st>>>(dy, w, rows_per_chunk, gx_part, cb);
    gemv_bwd_finish<1><<<g2, 256, 0, st>>>(gx_part, chunks, v, x, A, r, K, scale, grad_x, grad_A);
  } else {
    raise_lds_limit((const void *)gemv_bwd_partial<2>, lds);
    gemv_v<2><<<gv, 256, 0, st>>>(dy, N, B, u, r, scale, v, grad_B);
    gemv_bwd_partial<2><<<g1, 256, lds, st>>>(dy, w, rows_per_chunk, gx_part, cb);
    gemv_bwd_finish<2><<<g2, 256, 0, st>>>(gx_part, chunks, v, x, A, r, K, scale, grad_x, grad_A);
  }
  return hipGetLastError();
}

}  // namespace qlora
