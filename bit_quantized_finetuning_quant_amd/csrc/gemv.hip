// Few-token (T <= 4) QLoRA linear layer for gfx950.  With so few tokens the
// work per weight element is a handful of flops, so reading the 4-bit weight
// from HBM is the bound: every weight byte is read once, decoded once and used
// for all T tokens with vector ALU dot products.
//
// Method ("qlora" encyclopedia entry, tonho.wtf, section "a ideia"): the weight
// is dequantized to BFloat16 as it is used; gradients reach only the LoRA
// adapters.  W' = W + s.B.A (nexusinovation tutorial, section "LoRA: O Padrão
// Ouro de Eficiência").  Decoded values are bit-identical to the dequantizer:
// w_hat = bf16_rne(fl32(CB[code] * c1hat)).
//
// Layout of the work.  A row of the weight is split into 16-byte units of 32
// codes (half an NF4 block).
//
//   gemv_fwd_main    workgroup = (span of 32 units, 64 rows): x W_hat^T on
//                    v_mfma_f32_16x16x32_bf16 with the tokens padded to 16; a
//                    lane decodes one unit per step straight into the B operand.
//                    Extra workgroups do the same for the rows of A (partial u).
//   gemv_fwd_finish  y = sum of span partials + s u B^T, u = bf16(sum of partials)
//   gemv_bwd_main    workgroup = (span of 64 units, row chunk): a lane owns one
//                    unit column and walks groups of eight rows, pairing rows in
//                    v_dot2 against dy; the eight waves' column sums are added
//                    through LDS in a fixed tree.  Extra workgroups own rows of
//                    B: grad_B = s dy^T u and a partial v = dy B.
//   gemv_bwd_finish  per 64 columns: grad_x = sum of chunk partials + s v A,
//                    grad_A = s v^T x
// Every sum runs in a fixed order, so results do not depend on scheduling.

#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace qlora {

namespace {

constexpr int kSpanUnits = 64;   // backward: units per span (one per lane)
constexpr int kRowsPerWave = 8;  // backward: rows of one group
constexpr int kBwdWaves = 8;     // waves of a backward workgroup
constexpr int kBRows = 64;       // rows of B staged at a time by an adapter workgroup
constexpr int kFwdUnits = 32;    // forward: units per span
constexpr int kFwdSteps = kFwdUnits / 4;
constexpr int kFwdRows = 64;                    // forward: rows per workgroup (16 per wave)
constexpr int kXStride = kFwdUnits * 32 + 8;    // bf16 per token row of the LDS x tile

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float bf(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t to_bf16(float v) {
  __bf16 h = (__bf16)v;
  return __builtin_bit_cast(uint16_t, h);
}

__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// One unit (32 codes) of one row with the constants of its NF4 block.
struct UnitLoad {
  u32x4 c;
  uint32_t q;
  float s2;
};

__device__ __forceinline__ void load_unit(const QWeight &w, int64_t n, int64_t unit, int64_t kblk_row, UnitLoad &L) {
  L.c = *(const u32x4 *)(w.codes + n * (w.n_in / 2) + 16 * unit);
  const int64_t blk = n * kblk_row + (unit >> 1);
  L.q = w.fp8[blk];
  L.s2 = w.s2[blk >> 8];
}

// Codebook levels of the 32 codes of a unit.  Each byte of the masked words
// (c << 2) & 0x3C3C3C3C and (c >> 2) & 0x3C3C3C3C is four times a code (even
// and odd elements), i.e. the byte offset of its level in `lut`.
__device__ __forceinline__ void unit_levels(const u32x4 &c, const float *lut, float (&lv)[32]) {
  const char *base = (const char *)lut;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    uint32_t ev = (c[v] << 2) & 0x3C3C3C3Cu, od = (c[v] >> 2) & 0x3C3C3C3Cu;
    // opaque to the optimizer, which would otherwise rebuild a shift and a mask per code
    asm("" : "+v"(ev), "+v"(od));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lv[8 * v + 2 * k] = *(const float *)(base + __builtin_amdgcn_ubfe(ev, 8 * k, 8));
      lv[8 * v + 2 * k + 1] = *(const float *)(base + __builtin_amdgcn_ubfe(od, 8 * k, 8));
    }
  }
}

// 32 codes -> 16 bf16 pairs; pair p holds elements 2p (low half) and 2p + 1.
__device__ __forceinline__ void decode_unit(const u32x4 &c, float ch, const float *lut, uint32_t (&w)[16]) {
  float lv[32];
  unit_levels(c, lut, lv);
#pragma unroll
  for (int p = 0; p < 16; ++p) w[p] = pack_bf16x2(decode_product(lv[2 * p], ch), decode_product(lv[2 * p + 1], ch));
}

__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Forward, pass 1.  v_mfma_f32_16x16x32_bf16 lane layout: A lane l holds
// A[l % 16][8 (l / 16) + 0..7], B lane l holds B[8 (l / 16) + 0..7][l % 16] and
// D register i of lane l is D[4 (l / 16) + i][l % 16].  Here D[t][n] =
// sum_k x[t][k] W_hat[n][k] for a tile of 16 weight rows: lane (n = l % 16,
// g = l / 16) decodes unit 4 s + g of row n at step s, whose 32 values are the
// B operands of four MFMAs; the A operands are the same 32 columns of x for
// token min(l % 16, T - 1) (tokens are padded to 16; rows t >= T of D are
// never stored).
//
// Workgroup (span, row block): x[:, span columns] is staged in LDS (zero past
// n_in, so clamped units add nothing); wave w takes rows 64 block + 16 w +
// 0..15 of the weight, or of A for the workgroups past the weight's (partial
// u).
struct FwdTile {
  UnitLoad L[kFwdSteps];
};

__device__ __forceinline__ void fwd_load(const QWeight &w, int64_t n, int64_t unit0, int64_t U, int64_t kblk_row,
                                         FwdTile &f) {
#pragma unroll
  for (int st = 0; st < kFwdSteps; ++st) load_unit(w, n, min(unit0 + 4 * st, U - 1), kblk_row, f.L[st]);
}

__device__ __forceinline__ f32x4 fwd_tile(const FwdTile &f, float mu, const float *lut, const uint16_t *xrow) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < kFwdSteps; ++st) {
    uint32_t wv[16];
    decode_unit(f.L[st].c, decode_constant(f.L[st].q, f.L[st].s2, mu), lut, wv);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 xa = *(const u32x4 *)(xrow + 128 * st + 8 * j);
      acc = mfma16(xa, u32x4{wv[4 * j], wv[4 * j + 1], wv[4 * j + 2], wv[4 * j + 3]}, acc);
    }
  }
  return acc;
}

__device__ __forceinline__ void fwd_store(const f32x4 &acc, float *dst, int64_t rows, int64_t row, int T, int g) {
  if (row < rows) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * g + i < T) dst[(int64_t)(4 * g + i) * rows + row] = acc[i];
  }
}

__global__ __launch_bounds__(256) void gemv_fwd_main(const uint16_t *__restrict__ x, int T, QWeight w,
                                                     const uint16_t *__restrict__ A, int r, float *__restrict__ y_part,
                                                     float *__restrict__ u_part, int64_t spans, int64_t wblocks,
                                                     Codebook cb) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [T][kXStride]
  __shared__ float lut[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < 16) lut[tid] = cb.v[tid];
  const int64_t K = w.n_in, N = w.n_out, U = K / 32, kblk_row = K / kBlock;
  const bool a_rows = (int64_t)blockIdx.x >= wblocks;
  const int64_t blk = a_rows ? (int64_t)blockIdx.x - wblocks : (int64_t)blockIdx.x;
  const int64_t span = blk % spans, p = blk / spans;
  const int64_t col0 = span * kFwdUnits * 32;
  constexpr int kChunks = kFwdUnits * 4;  // 16-byte chunks of a token row of the tile
  for (int i = tid; i < T * kChunks; i += 256) {
    const int t = i / kChunks, c8 = (i % kChunks) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (col0 + c8 < K) v = *(const u32x4 *)(x + (int64_t)t * K + col0 + c8);
    *(u32x4 *)(xs + t * kXStride + c8) = v;
  }
  __syncthreads();
  const int rl = lane & 15, g = lane >> 4;
  const uint16_t *xrow = xs + min(rl, T - 1) * kXStride + 32 * g;
  const int64_t unit0 = span * kFwdUnits + g;
  if (a_rows) {
    const int64_t nrow0 = p * kFwdRows + wave * 16;
    if (nrow0 >= r) return;
    const int64_t n = min(nrow0 + rl, (int64_t)r - 1);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 av[kFwdSteps / 2][4];
#pragma unroll
      for (int st = 0; st < kFwdSteps / 2; ++st) {
        const int64_t unit = min(unit0 + 4 * (st + h * kFwdSteps / 2), U - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) av[st][j] = *(const u32x4 *)(A + n * K + 32 * unit + 8 * j);
      }
#pragma unroll
      for (int st = 0; st < kFwdSteps / 2; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 xa = *(const u32x4 *)(xrow + 128 * (st + h * kFwdSteps / 2) + 8 * j);
          acc = mfma16(xa, av[st][j], acc);
        }
    }
    fwd_store(acc, u_part + span * T * r, r, nrow0 + rl, T, g);
    return;
  }
  const int64_t row0 = p * kFwdRows + wave * 16;
  if (row0 >= N) return;
  FwdTile f;
  fwd_load(w, min(row0 + rl, N - 1), unit0, U, kblk_row, f);
  fwd_store(fwd_tile(f, *w.mu, lut, xrow), y_part + span * T * N, N, row0 + rl, T, g);
}

// Forward, pass 2: a workgroup per 64 output rows (N may be 0: u only).
// Quarter q = tid / 64 sums s u B^T over the 8-column chunks q, q + 4, ... of
// row 64 blockIdx.x + tid % 64 (eight loads in flight); quarter 0 adds the
// four quarters in order to the span partials.
template <int T>
__global__ __launch_bounds__(256) void gemv_fwd_finish(const float *__restrict__ y_part,
                                                       const float *__restrict__ u_part, int64_t spans,
                                                       const uint16_t *__restrict__ B, int r, float scale, int64_t N,
                                                       uint16_t *__restrict__ y, uint16_t *__restrict__ u_out) {
  __shared__ float us[T * 256];
  __shared__ float red[4][T][64];
  const int tid = threadIdx.x;
  for (int e = tid; e < T * r; e += 256) {
    float s = 0.f;
#pragma unroll 8
    for (int64_t sp = 0; sp < spans; ++sp) s += u_part[sp * T * r + e];
    const uint16_t h = to_bf16(s);
    us[e] = bf(h);
    if (blockIdx.x == 0) u_out[e] = h;
  }
  if (N == 0) return;
  __syncthreads();
  const int q = __builtin_amdgcn_readfirstlane(tid >> 6), c = tid & 63;
  const int64_t n = (int64_t)blockIdx.x * 64 + c;
  const uint16_t *brow = B + (n < N ? n : N - 1) * r;
  float lora[T];
#pragma unroll
  for (int t = 0; t < T; ++t) lora[t] = 0.f;
  if ((r & 7) == 0) {
    const int nch = r / 8;
    for (int c0 = q; c0 < nch; c0 += 32) {
      u32x4 b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) b[i] = *(const u32x4 *)(brow + 8 * min(c0 + 4 * i, nch - 1));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ch = c0 + 4 * i;
        if (ch < nch) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int t = 0; t < T; ++t) {
              lora[t] = __builtin_fmaf(us[t * r + 8 * ch + 2 * e], bf16_lo(b[i][e]), lora[t]);
              lora[t] = __builtin_fmaf(us[t * r + 8 * ch + 2 * e + 1], bf16_hi(b[i][e]), lora[t]);
            }
        }
      }
    }
  } else {
    for (int j0 = q; j0 < r; j0 += 32) {
      float b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) b[i] = bf(brow[min(j0 + 4 * i, r - 1)]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = j0 + 4 * i;
        if (j < r) {
#pragma unroll
          for (int t = 0; t < T; ++t) lora[t] = __builtin_fmaf(us[t * r + j], b[i], lora[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t) red[q][t][c] = lora[t];
  __syncthreads();
  if (q == 0 && n < N) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float s = 0.f;
#pragma unroll 8
      for (int64_t sp = 0; sp < spans; ++sp) s += y_part[(sp * T + t) * N + n];
      y[t * N + n] = to_bf16(s + scale * (red[0][t][c] + red[1][t][c] + red[2][t][c] + red[3][t][c]));
    }
  }
}

// ---------------------------------------------------------------------------
// Eight rows of one unit column with dy of those rows (zero past N).
template <int T>
struct BwdGroup {
  UnitLoad L[kRowsPerWave];
  float d[kRowsPerWave][T];
};

template <int T>
__device__ __forceinline__ void bwd_load(const QWeight &w, const uint16_t *dy, int64_t n0, int64_t unit,
                                         int64_t kblk_row, BwdGroup<T> &g) {
  const int64_t N = w.n_out;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int64_t n = n0 + i;
    load_unit(w, min(n, N - 1), unit, kblk_row, g.L[i]);
#pragma unroll
    for (int t = 0; t < T; ++t) g.d[i][t] = n < N ? bf(dy[t * N + n]) : 0.f;
  }
}

// Rows i and i + 1 share a bf16 pair: element e of both rows against
// (dy[t][n0 + i], dy[t][n0 + i + 1]) in one dot2.
template <int T>
__device__ __forceinline__ void bwd_group(const BwdGroup<T> &g, float mu, const float *lut, float (&acc)[T][32]) {
#pragma unroll
  for (int i = 0; i < kRowsPerWave; i += 2) {
    float l0[32], l1[32];
    unit_levels(g.L[i].c, lut, l0);
    unit_levels(g.L[i + 1].c, lut, l1);
    const float c0 = decode_constant(g.L[i].q, g.L[i].s2, mu), c1 = decode_constant(g.L[i + 1].q, g.L[i + 1].s2, mu);
    uint32_t dp[T];
#pragma unroll
    for (int t = 0; t < T; ++t) dp[t] = pack_bf16x2(g.d[i][t], g.d[i + 1][t]);
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const uint32_t wp = pack_bf16x2(decode_product(l0[e], c0), decode_product(l1[e], c1));
#pragma unroll
      for (int t = 0; t < T; ++t) acc[t][e] = dot2(wp, dp[t], acc[t][e]);
    }
  }
}

// Backward, pass 1.  Workgroups below nf4_wgs: span = id % spans, chunk =
// id / spans; wave w takes `groups` groups of eight rows starting at row
// chunk * 8 groups * 8 + w * groups * 8 and accumulates 32 column sums per
// token.  The eight waves' sums are added through LDS in a fixed tree
// (4 + 4, 2 + 2, 1 + 1) and wave 0 writes the chunk's partial.  Later
// workgroups each own `bsub` blocks of 64 rows of B: grad_B rows and a partial
// v = dy B over their rows.
template <int T>
__device__ __forceinline__ void bwd_main_body(const uint16_t *__restrict__ dy, QWeight w,
                                              const uint16_t *__restrict__ B, const uint16_t *__restrict__ u, int r,
                                              float scale, float *__restrict__ gx_part, float *__restrict__ v_part,
                                              float *__restrict__ grad_B, int64_t spans, int64_t nf4_wgs, int groups,
                                              int bsub, const Codebook &cb, float *smem, float *lut) {
  static_assert(T <= 4, "adapter partials hold at most two entries per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = w.n_in, N = w.n_out;
  if ((int64_t)blockIdx.x >= nf4_wgs) {
    // adapter rows [bid * bsub * 64, ...) of B, 64 at a time (r <= 256)
    const int64_t bid = (int64_t)blockIdx.x - nf4_wgs;
    float *us = smem;                          // [T][r]
    float *ds = us + T * 256;                  // [T][64]
    uint16_t *bt = (uint16_t *)(ds + T * 64);  // [64][r]
    float *vt = (float *)(bt + kBRows * 256);  // [S][E]
    const int E = T * r, S = E >= 512 ? 1 : 512 / E;
    for (int e = tid; e < T * r; e += 512) us[e] = bf(u[e]);
    float vacc[2] = {0.f, 0.f};  // entries idx = tid and tid + 512 of the [S][E] slices
    for (int sb = 0; sb < bsub; ++sb) {
      const int64_t n0 = (bid * bsub + sb) * kBRows;
      if (n0 >= N) break;
      const int rows = (int)min((int64_t)kBRows, N - n0);
      __syncthreads();  // the previous block's tile is no longer read
      for (int e = tid; e < T * kBRows; e += 512) {
        const int t = e / kBRows, i = e % kBRows;
        ds[e] = i < rows ? bf(dy[t * N + n0 + i]) : 0.f;
      }
      const uint16_t *bsrc = B + n0 * r;
      const int elems = rows * r;
      for (int e0 = tid; e0 < elems; e0 += 512 * 8) {
        uint16_t b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) b[i] = bsrc[min(e0 + 512 * i, elems - 1)];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (e0 + 512 * i < elems) bt[e0 + 512 * i] = b[i];
      }
      __syncthreads();
      for (int e = tid; e < elems; e += 512) {
        const int i = e / r, j = e % r;
        float g = 0.f;
#pragma unroll
        for (int t = 0; t < T; ++t) g = __builtin_fmaf(ds[t * kBRows + i], us[t * r + j], g);
        grad_B[n0 * r + e] = scale * g;
      }
      // slice sl of the threads takes rows sl, sl + S, ... of this block
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int idx = tid + 512 * k;
        if (idx < E * S) {
          const int e = idx % E, sl = idx / E, t = e / r, j = e % r;
          float s = vacc[k];
          for (int i = sl; i < rows; i += S) s = __builtin_fmaf(ds[t * kBRows + i], bf(bt[i * r + j]), s);
          vacc[k] = s;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (tid + 512 * k < E * S) vt[tid + 512 * k] = vacc[k];
    __syncthreads();
    for (int e = tid; e < E; e += 512) {
      float s = 0.f;
      for (int sl = 0; sl < S; ++sl) s += vt[sl * E + e];
      v_part[bid * E + e] = s;
    }
    return;
  }

  if (tid < 16) lut[tid] = cb.v[tid];
  __syncthreads();
  const int64_t U = K / 32, kblk_row = K / kBlock;
  const int64_t span = blockIdx.x % spans, chunk = blockIdx.x / spans;
  const int64_t unit = span * kSpanUnits + lane;
  const bool valid = unit < U;
  const int64_t uc = valid ? unit : U - 1;
  const int64_t n_base = (chunk * kBwdWaves + wave) * (int64_t)groups * kRowsPerWave;
  const float mu = *w.mu;
  float acc[T][32];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int e = 0; e < 32; ++e) acc[t][e] = 0.f;
  for (int64_t n0 = n_base; n0 < min(N, n_base + (int64_t)groups * kRowsPerWave); n0 += kRowsPerWave) {
    BwdGroup<T> g0;
    bwd_load(w, dy, n0, uc, kblk_row, g0);
    bwd_group(g0, mu, lut, acc);
  }
  // fixed tree over the eight waves; smem holds [4][T * 32][64]
#pragma unroll
  for (int half = 4; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int e = 0; e < 32; ++e) smem[((wave - half) * T * 32 + t * 32 + e) * 64 + lane] = acc[t][e];
    }
    __syncthreads();
    if (wave < half) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int e = 0; e < 32; ++e) acc[t][e] += smem[(wave * T * 32 + t * 32 + e) * 64 + lane];
    }
    __syncthreads();
  }
  if (wave == 0 && valid) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float *dst = gx_part + (chunk * T + t) * K + 32 * unit;
#pragma unroll
      for (int v = 0; v < 8; ++v)
        *(f32x4 *)(dst + 4 * v) = f32x4{acc[t][4 * v], acc[t][4 * v + 1], acc[t][4 * v + 2], acc[t][4 * v + 3]};
    }
  }
}

// One token fits in 128 registers, which keeps two workgroups on every CU.
__global__ __launch_bounds__(512, 4) void gemv_bwd_main_t1(const uint16_t *__restrict__ dy, QWeight w,
                                                           const uint16_t *__restrict__ B,
                                                           const uint16_t *__restrict__ u, int r, float scale,
                                                           float *__restrict__ gx_part, float *__restrict__ v_part,
                                                           float *__restrict__ grad_B, int64_t spans, int64_t nf4_wgs,
                                                           int groups, int bsub, Codebook cb) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ float lut[16];
  bwd_main_body<1>(dy, w, B, u, r, scale, gx_part, v_part, grad_B, spans, nf4_wgs, groups, bsub, cb, smem, lut);
}

template <int T>
__global__ __launch_bounds__(512) void gemv_bwd_main(const uint16_t *__restrict__ dy, QWeight w,
                                                     const uint16_t *__restrict__ B, const uint16_t *__restrict__ u,
                                                     int r, float scale, float *__restrict__ gx_part,
                                                     float *__restrict__ v_part, float *__restrict__ grad_B,
                                                     int64_t spans, int64_t nf4_wgs, int groups, int bsub,
                                                     Codebook cb) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ float lut[16];
  bwd_main_body<T>(dy, w, B, u, r, scale, gx_part, v_part, grad_B, spans, nf4_wgs, groups, bsub, cb, smem, lut);
}

// Backward, pass 2: a workgroup per 64 columns; thread (jg, c) = (tid / 64,
// tid % 64) takes adapter rows j = jg, jg + 4, ... and chunk partials
// jg, jg + 4, ...; the four groups are added in order through LDS.
template <int T>
__global__ __launch_bounds__(256) void gemv_bwd_finish(const float *__restrict__ gx_part, int64_t chunks,
                                                       const float *__restrict__ v_part, int64_t vparts,
                                                       const uint16_t *__restrict__ x, const uint16_t *__restrict__ A,
                                                       int r, int64_t K, float scale, uint16_t *__restrict__ grad_x,
                                                       float *__restrict__ grad_A) {
  __shared__ float tmp[1024];
  __shared__ float vs[T * 256];
  __shared__ float red[4][T][64];
  const int tid = threadIdx.x;
  // v = sum of the adapter workgroups' partials: slice sl of the threads sums
  // partials sl, sl + S, ...; the S slices are then added in order
  const int E = T * r;
  const int S = E >= 256 ? 1 : 256 / E;
  for (int idx = tid; idx < E * S; idx += 256) {
    const int e = idx % E, sl = idx / E;
    float s = 0.f;
    for (int64_t p0 = sl; p0 < vparts; p0 += 8 * S) {
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pv[i] = v_part[min(p0 + i * S, vparts - 1) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) s += p0 + i * S < vparts ? pv[i] : 0.f;
    }
    tmp[idx] = s;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    float s = 0.f;
    for (int sl = 0; sl < S; ++sl) s += tmp[sl * E + e];
    vs[e] = s;
  }
  __syncthreads();
  const int jg = __builtin_amdgcn_readfirstlane(tid >> 6), c = tid & 63;
  const int64_t col = (int64_t)blockIdx.x * 64 + c;
  const bool valid = col < K;
  const int64_t cc = valid ? col : K - 1;
  float xv[T], g[T], lora[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    xv[t] = bf(x[t * K + cc]);
    g[t] = 0.f;
    lora[t] = 0.f;
  }
  for (int j0 = jg; j0 < r; j0 += 32) {
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = bf(A[(int64_t)min(j0 + 4 * i, r - 1) * K + cc]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = j0 + 4 * i;
      if (j < r) {
        float ga = 0.f;
#pragma unroll
        for (int t = 0; t < T; ++t) {
          lora[t] = __builtin_fmaf(vs[t * r + j], a[i], lora[t]);
          ga = __builtin_fmaf(vs[t * r + j], xv[t], ga);
        }
        if (valid) grad_A[(int64_t)j * K + col] = scale * ga;
      }
    }
  }
  if (grad_x) {
    for (int64_t c0 = jg; c0 < chunks; c0 += 32) {
      float gv[8][T];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int t = 0; t < T; ++t) gv[i][t] = gx_part[(min(c0 + 4 * i, chunks - 1) * T + t) * K + cc];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int t = 0; t < T; ++t) g[t] += c0 + 4 * i < chunks ? gv[i][t] : 0.f;
    }
#pragma unroll
    for (int t = 0; t < T; ++t) red[jg][t][c] = g[t] + scale * lora[t];
    __syncthreads();
    if (jg == 0 && valid) {
#pragma unroll
      for (int t = 0; t < T; ++t)
        grad_x[t * K + col] = to_bf16(red[0][t][c] + red[1][t][c] + red[2][t][c] + red[3][t][c]);
    }
  }
}

// Work split of one call.  The backward takes enough rows per wave that the
// chunk partials stay small next to the weight, and no more than keeps about
// 2048 waves in flight.
struct GemvGeometry {
  int64_t fspans, fblocks, ablocks;       // forward: spans, weight and A workgroups
  int64_t bspans, groups, chunks;         // backward weight pass
  int64_t bsub, bparts;                   // backward adapter workgroups
};

GemvGeometry geometry(int64_t N, int64_t K, int r) {
  GemvGeometry g;
  g.fspans = cdiv(K / 32, kFwdUnits);
  g.fblocks = g.fspans * cdiv(N, kFwdRows);
  g.ablocks = g.fspans * cdiv(r, kFwdRows);
  g.bspans = cdiv(K / 32, kSpanUnits);
  const int64_t rows_per_wave = g.bspans * N / 2048;
  g.groups = std::max<int64_t>(1, std::min<int64_t>(4, rows_per_wave / kRowsPerWave));
  g.chunks = cdiv(N, kBwdWaves * g.groups * kRowsPerWave);
  const int64_t blocks = cdiv(N, kBRows);
  g.bsub = std::max<int64_t>(1, blocks / 64);
  g.bparts = cdiv(blocks, g.bsub);
  return g;
}

size_t bwd_lds_bytes(int T) {
  const size_t tree = (size_t)4 * T * 32 * 64 * 4;
  const size_t adapter = (size_t)T * 256 * 4 + (size_t)T * 64 * 4 + (size_t)kBRows * 256 * 2 + 1024 * 4;
  return std::max(tree, adapter);
}

template <int T>
hipError_t gemv_fwd_impl(const uint16_t *x, const QWeight &w, const uint16_t *A, const uint16_t *B, int r,
                         float scale, uint16_t *y, uint16_t *u, float *part, const Codebook &cb, hipStream_t st) {
  const int64_t N = w.n_out;
  const GemvGeometry g = geometry(N, w.n_in, r);
  const bool rows = y != nullptr;
  const int64_t fblocks = rows ? g.fblocks : 0;
  float *y_part = part, *u_part = part + g.fspans * T * N;
  const size_t lds = (size_t)T * kXStride * 2;
  TimedLaunch tl;
  const bool timed = rows && timing_begin(st, tl, kTimedGemvFwd);
  gemv_fwd_main<<<(unsigned)(fblocks + g.ablocks), 256, lds, st>>>(x, T, w, A, r, y_part, u_part, g.fspans, fblocks,
                                                                   cb);
  if (timed) timing_end(st, tl);
  const int64_t out_rows = rows ? N : 0;
  const unsigned fg = (unsigned)std::max<int64_t>(1, cdiv(out_rows, 64));
  gemv_fwd_finish<T><<<fg, 256, 0, st>>>(y_part, u_part, g.fspans, B, r, scale, out_rows, y, u);
  return hipGetLastError();
}

template <int T>
hipError_t gemv_bwd_impl(const uint16_t *dy, const uint16_t *x, const QWeight &w, const uint16_t *A,
                         const uint16_t *B, int r, float scale, const uint16_t *u, uint16_t *grad_x, float *grad_A,
                         float *grad_B, float *part, const Codebook &cb, hipStream_t st) {
  const int64_t N = w.n_out, K = w.n_in;
  const GemvGeometry g = geometry(N, K, r);
  const int64_t nf4_wgs = grad_x ? g.bspans * g.chunks : 0;
  float *gx_part = part, *v_part = part + g.chunks * T * K;
  const size_t lds = bwd_lds_bytes(T);
  const void *fn = T == 1 ? (const void *)gemv_bwd_main_t1 : (const void *)gemv_bwd_main<T>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const unsigned grid = (unsigned)(nf4_wgs + g.bparts);
  TimedLaunch tl;
  const bool timed = grad_x && timing_begin(st, tl, kTimedGemvBwd);
  if (T == 1)
    gemv_bwd_main_t1<<<grid, 512, lds, st>>>(dy, w, B, u, r, scale, gx_part, v_part, grad_B, g.bspans, nf4_wgs,
                                             (int)g.groups, (int)g.bsub, cb);
  else
    gemv_bwd_main<T><<<grid, 512, lds, st>>>(dy, w, B, u, r, scale, gx_part, v_part, grad_B, g.bspans, nf4_wgs,
                                             (int)g.groups, (int)g.bsub, cb);
  if (timed) timing_end(st, tl);
  gemv_bwd_finish<T><<<(unsigned)cdiv(K, 64), 256, 0, st>>>(gx_part, g.chunks, v_part, g.bparts, x, A, r, K, scale,
                                                            grad_x, grad_A);
  return hipGetLastError();
}

}  // namespace

bool gemv_applies(int64_t T, int64_t K) { return T >= 1 && T <= kGemvMaxT && K % 64 == 0; }

size_t gemv_part_floats(int64_t T, int64_t N, int64_t K, int r) {
  const GemvGeometry g = geometry(N, K, r);
  const size_t fwd = (size_t)(g.fspans * T * (N + r));
  const size_t bwd = (size_t)(g.chunks * T * K + g.bparts * T * r);
  return std::max(fwd, bwd);
}

hipError_t launch_gemv_fwd(int64_t T, const uint16_t *x, const QWeight &w, const uint16_t *A, const uint16_t *B,
                           int r, float scale, uint16_t *y, uint16_t *u, float *part, const Codebook &cb,
                           hipStream_t st) {
  switch (T) {
    case 1: return gemv_fwd_impl<1>(x, w, A, B, r, scale, y, u, part, cb, st);
    case 2: return gemv_fwd_impl<2>(x, w, A, B, r, scale, y, u, part, cb, st);
    case 3: return gemv_fwd_impl<3>(x, w, A, B, r, scale, y, u, part, cb, st);
    case 4: return gemv_fwd_impl<4>(x, w, A, B, r, scale, y, u, part, cb, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv_bwd(int64_t T, const uint16_t *dy, const uint16_t *x, const QWeight &w, const uint16_t *A,
                           const uint16_t *B, int r, float scale, const uint16_t *u, uint16_t *grad_x,
                           float *grad_A, float *grad_B, float *part, const Codebook &cb, hipStream_t st) {
  switch (T) {
    case 1: return gemv_bwd_impl<1>(dy, x, w, A, B, r, scale, u, grad_x, grad_A, grad_B, part, cb, st);
    case 2: return gemv_bwd_impl<2>(dy, x, w, A, B, r, scale, u, grad_x, grad_A, grad_B, part, cb, st);
    case 3: return gemv_bwd_impl<3>(dy, x, w, A, B, r, scale, u, grad_x, grad_A, grad_B, part, cb, st);
    case 4: return gemv_bwd_impl<4>(dy, x, w, A, B, r, scale, u, grad_x, grad_A, grad_B, part, cb, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qlora
