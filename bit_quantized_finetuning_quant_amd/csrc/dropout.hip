// LoRA dropout mask for the adapter input x [T x K] (bf16).
//
// The training recipe sets a dropout probability on the adapters ("Tutorial
// fine-tuning LLM LoRA/QLoRA", section "Código Completo", step "4.
// Configuração LoRA").  Dropout acts on the adapter input only, with the
// kept values scaled by 1 / (1 - p) (applied by the consumers of the mask),
// and the backward reuses the mask.  The mask comes from Philox4x64-10
// (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC 2011): element e = t K + k takes 32-bit word e mod 8 of the block for
// counter (e div 8, 0, 0, 0) and key (seed, 0) -- the four 64-bit outputs in
// order, low half first -- and is kept iff that word is >= thresh.
//
// One launch writes both forms the consumers read:
//   keep  uint32 [ceil(T/32)][K]: bit b of word [tb][k] is the keep bit of
//         (32 tb + b, k) (0 past T).  A consumer wave of the grad_x GEMM
//         holds, per 32 x 32 sub-tile, 16 accumulators of one column and rows
//         of one 32-row block, so one word serves all of them.
//   xd    bf16 [T x K]: x where kept, +0 where dropped (exact), the input of
//         the adapter products u = xd A^T and grad_A = v^T xd.
// A workgroup (1-D grid, row block major) covers 32 rows x 256 columns: each thread runs four block
// functions (8 consecutive columns of one row each), writes 16 bytes of xd
// per block and its 8 keep bits to LDS; then thread c packs column c's 32
// bits into one word.

#include "common.hpp"
#include "launch.hpp"

namespace qlora {
namespace {

constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull, kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull, kPhiloxW1 = 0xBB67AE8584CAA73Bull;

// hi:lo = m * c (128 bits) from four 32 x 32 -> 64 products, each a v_mad_u64_u32 with the
// running partial sum as its addend (no sum overflows 64 bits).
__device__ __forceinline__ void mulhilo64(uint64_t m, uint64_t c, uint64_t &hi, uint64_t &lo) {
  const uint32_t ml = (uint32_t)m, mh = (uint32_t)(m >> 32), cl = (uint32_t)c, ch = (uint32_t)(c >> 32);
  const uint64_t p0 = (uint64_t)ml * cl;
  const uint64_t t = (uint64_t)ml * ch + (p0 >> 32);
  const uint64_t u = (uint64_t)mh * cl + (uint32_t)t;
  lo = (u << 32) | (uint32_t)p0;
  hi = (uint64_t)mh * ch + ((t >> 32) + (u >> 32));
}

__device__ __forceinline__ void philox4x64_10(uint64_t c0, uint64_t k0, uint64_t k1, uint64_t (&o)[4]) {
  uint64_t c1 = 0, c2 = 0, c3 = 0;
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    uint64_t hi0, lo0, hi1, lo1;
    mulhilo64(kPhiloxM0, c0, hi0, lo0);
    mulhilo64(kPhiloxM1, c2, hi1, lo1);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  o[0] = c0;
  o[1] = c1;
  o[2] = c2;
  o[3] = c3;
}

constexpr int kMaskRows = 32, kMaskCols = 256;

__global__ __launch_bounds__(256) void dropout_mask(const uint16_t *__restrict__ x, int64_t T, int64_t K,
                                                    uint32_t thresh, uint64_t seed, uint32_t *__restrict__ keep,
                                                    uint16_t *__restrict__ xd, int64_t col_tiles) {
  __shared__ uint8_t kb[kMaskRows][kMaskCols];
  const int tid = threadIdx.x;
  const int64_t tb = (int64_t)blockIdx.x / col_tiles, col0 = ((int64_t)blockIdx.x % col_tiles) * kMaskCols;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i;
    const int rr = id >> 5, cc = id & 31;
    const int64_t t = tb * kMaskRows + rr, k0 = col0 + 8 * cc;
    uint32_t bits = 0u;
    if (t < T && k0 < K) {  // K % 8 == 0: the 8 columns are all in range
      const int64_t e0 = t * K + k0;
      uint64_t o[4];
      philox4x64_10((uint64_t)(e0 >> 3), seed, 0ull, o);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t word = (uint32_t)(o[j >> 1] >> (32 * (j & 1)));
        bits |= (word >= thresh ? 1u : 0u) << j;
      }
      u32x4 v = *(const u32x4 *)(x + e0);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t m = ((bits >> (2 * h)) & 1u ? 0x0000FFFFu : 0u) | ((bits >> (2 * h + 1)) & 1u ? 0xFFFF0000u : 0u);
        v[h] &= m;
      }
      *(u32x4 *)(xd + e0) = v;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) kb[rr][8 * cc + j] = (uint8_t)((bits >> j) & 1u);
  }
  __syncthreads();
  const int64_t col = col0 + tid;
  if (col < K) {
    uint32_t wv = 0u;
#pragma unroll
    for (int rr = 0; rr < kMaskRows; ++rr) wv |= (uint32_t)kb[rr][tid] << rr;
    keep[tb * K + col] = wv;
  }
}

}  // namespace

size_t dropout_keep_words(int64_t T, int64_t K) { return (size_t)((T + kMaskRows - 1) / kMaskRows) * (size_t)K; }

hipError_t launch_dropout_mask(const uint16_t *x, int64_t T, int64_t K, uint32_t thresh, uint64_t seed,
                               uint32_t *keep, uint16_t *xd, hipStream_t st) {
  if (T <= 0 || K <= 0) return hipSuccess;
  const int64_t col_tiles = (K + kMaskCols - 1) / kMaskCols, row_blocks = (T + kMaskRows - 1) / kMaskRows;
  dropout_mask<<<(unsigned)(col_tiles * row_blocks), 256, 0, st>>>(x, T, K, thresh, seed, keep, xd, col_tiles);
  return hipGetLastError();
}

}  // namespace qlora
