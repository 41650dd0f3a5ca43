// Few-token QLoRA linear layer for gfx950 (forward T <= 32, backward T <= 4).
// With so few tokens the work per weight element is a handful of flops, so
// reading the 4-bit weight from HBM is the bound: every weight byte is read
// once, decoded once and used for all T tokens (the forward's matrix tiles pad
// the tokens to 16, one or two tiles; the backward's vector ALU dot products
// cost per token).
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
//   gemv_fwd_main    workgroup = (span of 8 or 32 units, 64 rows): x W_hat^T on
//                    v_mfma_f32_16x16x32_bf16 with the tokens padded to 16 (one
//                    or two token tiles); a lane decodes one unit per step
//                    straight into the B operand of every token tile.
//                    The first workgroups do the same for the rows of A
//                    (partial u).
//   gemv_fwd_finish  y = sum of span partials + s u B^T, u = bf16(sum of partials)
//   gemv_bwd_main    workgroup = (span of 64 units, row chunk): a lane owns one
//                    unit column and walks groups of four rows, pairing rows in
//                    v_dot2 against dy; the eight waves' column sums are added
//                    through LDS in a fixed tree.  The first workgroups own rows
//                    of B: grad_B = s dy^T u and a partial v = dy B.
//   gemv_bwd_finish  per 64 columns: grad_x = sum of chunk partials + s v A,
//                    grad_A = s v^T x
// Every sum runs in a fixed order, so results do not depend on scheduling.

#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace qlora {

namespace {

constexpr int kSpanUnits = 64;   // backward: units per span (one per lane)
constexpr int kRowsPerWave = 4;  // backward: rows of one group
constexpr int kBwdWaves = 8;     // waves of a backward workgroup
constexpr int kBwdThreads = kBwdWaves * 64;
// backward: waves the row split aims for; from 2 tokens the dot products per weight double and
// fewer, longer row chunks (half the chunk partials to add) pay
constexpr int64_t kBwdTargetWavesT1 = 2048, kBwdTargetWaves = 1024;
constexpr int kBRows = 64;       // rows of B staged at a time by an adapter workgroup
constexpr int kFwdRows = 64;     // forward: rows per workgroup (16 per wave)
// Forward span (units per workgroup): short spans give small weights enough
// waves to hide the load latency; large weights have waves to spare and take
// long spans, which keep the span partials and per-workgroup set-up few.
constexpr int kFwdUnitsSmall = 8, kFwdUnitsLarge = 32;
constexpr int64_t kFwdShortSpanWaves = 8192;  // short spans while they give at most this many waves
// Above 16 tokens (two to four tiles of 16 per decoded unit) the forward pays only while its x tile
// leaves room for several workgroups per CU: with the long spans of large weights 32 tokens take
// 66 KB of LDS per workgroup and run slower than the fused GEMM's few-token tiles (22016 x 8192:
// 157.7 -> 171.5 us per fwd+bwd, against 61 -> 50 us at 4096^2 and 17 tokens).
constexpr size_t kFwdMultiTileMaxLds = 40 * 1024;
template <int kUnits>
struct FwdShape {
  static constexpr int kSteps = kUnits / 4;
  static constexpr int kXStride = kUnits * 32 + 8;  // bf16 per token row of the LDS x tile
  static constexpr int kASlice = kSteps < 4 ? kSteps : 4;
  static_assert(kSteps % kASlice == 0, "A rows are read in whole slices");
};

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

// One unit (32 codes) of one row with the constants of its NF4 block.  With
// fp32 block constants (no double quantization) the unit carries q = 0x38
// (e4m3 1.0) and s2 = c1, and the decode runs with mu = 0: fl32(fl32(1 * c1)
// + 0) = c1 exactly, so one decode serves both storage forms.
constexpr uint32_t kE4m3One = 0x38u;
struct UnitLoad {
  u32x4 c;
  uint32_t q;
  float s2;
};

__device__ __forceinline__ void load_unit(const QWeight &w, int64_t n, int64_t unit, int64_t kblk_row, UnitLoad &L) {
  L.c = *(const u32x4 *)(w.codes + n * (w.n_in / 2) + 16 * unit);
  const int64_t blk = n * kblk_row + (unit >> 1);
  if (w.dq) {
    L.q = w.fp8[blk];
    L.s2 = w.s2[blk >> 8];
  } else {
    L.q = kE4m3One;
    L.s2 = w.s2[blk];
  }
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
// 0..15 of A (the first workgroups: partial u) or of the weight.  Each wave
// issues the loads of its rows before x is staged, so the two overlap.
template <int kSteps>
struct FwdTile {
  UnitLoad L[kSteps];
};

// The weights of one forward pass: up to kMaxSetMembers linears that share x, their rows
// concatenated (a single linear is a set of one).  Member m's rows start at 64-row block block0[m]
// (every member but the last has a multiple of 64 rows); block0[m] is past every block for
// m >= count.  y[m] and B[m] are its output and right factor.
struct GemvFwdSet {
  int count;
  QWeight w[kMaxSetMembers];
  int64_t block0[kMaxSetMembers + 1];
  const uint16_t *B[kMaxSetMembers];
  uint16_t *y[kMaxSetMembers];
};

__device__ __forceinline__ int fwd_member(const GemvFwdSet &s, int64_t p) {
  return (p >= s.block0[1] ? 1 : 0) + (p >= s.block0[2] ? 1 : 0) + (p >= s.block0[3] ? 1 : 0);
}

template <int kSteps>
__device__ __forceinline__ void fwd_load(const QWeight &w, int64_t n, int64_t unit0, int64_t U, int64_t kblk_row,
                                         FwdTile<kSteps> &f) {
#pragma unroll
  for (int st = 0; st < kSteps; ++st) load_unit(w, n, min(unit0 + 4 * st, U - 1), kblk_row, f.L[st]);
}

// kTT tiles of 16 tokens (xrow[h]: this lane's token row of tile h) share
// each decoded unit.
template <int kSteps, int kTT>
__device__ __forceinline__ void fwd_tile(const FwdTile<kSteps> &f, float mu, const float *lut,
                                         const uint16_t *const (&xrow)[kTT], f32x4 (&acc)[kTT]) {
#pragma unroll
  for (int h = 0; h < kTT; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    uint32_t wv[16];
    decode_unit(f.L[st].c, decode_constant(f.L[st].q, f.L[st].s2, mu), lut, wv);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 wj = u32x4{wv[4 * j], wv[4 * j + 1], wv[4 * j + 2], wv[4 * j + 3]};
#pragma unroll
      for (int h = 0; h < kTT; ++h) acc[h] = mfma16(*(const u32x4 *)(xrow[h] + 128 * st + 8 * j), wj, acc[h]);
    }
  }
}

// Rows of A: the same tile with bf16 values read directly, in slices of at
// most four steps (16 registers a step).
template <int kASlice>
__device__ __forceinline__ void a_load(const uint16_t *A, int64_t K, int64_t n, int64_t unit0, int64_t U, int h,
                                       u32x4 (&av)[kASlice][4]) {
#pragma unroll
  for (int st = 0; st < kASlice; ++st) {
    const int64_t unit = min(unit0 + 4 * (st + h * kASlice), U - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) av[st][j] = *(const u32x4 *)(A + n * K + 32 * unit + 8 * j);
  }
}

__device__ __forceinline__ void fwd_store(const f32x4 &acc, float *dst, int64_t rows, int64_t row, int T, int g,
                                          int h) {
  if (row < rows) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * h + 4 * g + i;
      if (t < T) dst[(int64_t)t * rows + row] = acc[i];
    }
  }
}

template <int kUnits, int kTT>
__global__ __launch_bounds__(256) void gemv_fwd_main(const uint16_t *__restrict__ x,
                                                     const uint16_t *__restrict__ xa, int T, GemvFwdSet set,
                                                     int64_t Ntot, const uint16_t *__restrict__ A, int r,
                                                     float *__restrict__ y_part, float *__restrict__ u_part,
                                                     int64_t spans, int64_t ablocks, Codebook cb) {
  typedef FwdShape<kUnits> S;
  constexpr int kSteps = S::kSteps, kXStride = S::kXStride, kASlice = S::kASlice;
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [T][kXStride]
  __shared__ float lut[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = set.w[0].n_in, U = K / 32, kblk_row = K / kBlock;
  const bool a_rows = (int64_t)blockIdx.x < ablocks;
  const int64_t blk = a_rows ? (int64_t)blockIdx.x : (int64_t)blockIdx.x - ablocks;
  const int64_t span = blk % spans, pg = blk / spans;
  // the member of this row block, and the block within it
  const int m = a_rows ? 0 : fwd_member(set, pg);
  const QWeight w = set.w[m];
  const int64_t p = a_rows ? pg : pg - set.block0[m], N = w.n_out;
  const int64_t col0 = span * kUnits * 32;
  const int rl = lane & 15, g = lane >> 4;
  const int64_t unit0 = span * kUnits + g;
  const int64_t row0 = p * kFwdRows + wave * 16, rows = a_rows ? r : N;
  const bool active = row0 < rows;
  const int64_t n = min(row0 + rl, rows - 1);
  FwdTile<kSteps> f;
  u32x4 av[kASlice][4];
  if (active) {
    if (a_rows)
      a_load<kASlice>(A, K, n, unit0, U, 0, av);
    else
      fwd_load(w, n, unit0, U, kblk_row, f);
  }
  if (tid < 16) lut[tid] = cb.v[tid];
  constexpr int kChunks = kUnits * 4;  // 16-byte chunks of a token row of the tile
  const uint16_t *xsrc = a_rows ? xa : x;  // the adapter rows read the adapter input
  for (int i = tid; i < T * kChunks; i += 256) {
    const int t = i / kChunks, c8 = (i % kChunks) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (col0 + c8 < K) v = *(const u32x4 *)(xsrc + (int64_t)t * K + col0 + c8);
    *(u32x4 *)(xs + t * kXStride + c8) = v;
  }
  __syncthreads();
  if (!active) return;
  const uint16_t *xrow[kTT];
#pragma unroll
  for (int h = 0; h < kTT; ++h) xrow[h] = xs + min(16 * h + rl, T - 1) * kXStride + 32 * g;
  f32x4 acc[kTT];
  if (a_rows) {
#pragma unroll
    for (int h = 0; h < kTT; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sl = 0; sl < kSteps / kASlice; ++sl) {
      if (sl > 0) a_load<kASlice>(A, K, n, unit0, U, sl, av);
#pragma unroll
      for (int st = 0; st < kASlice; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int h = 0; h < kTT; ++h)
            acc[h] = mfma16(*(const u32x4 *)(xrow[h] + 128 * (st + sl * kASlice) + 8 * j), av[st][j], acc[h]);
    }
#pragma unroll
    for (int h = 0; h < kTT; ++h) fwd_store(acc[h], u_part + span * T * r, r, row0 + rl, T, g, h);
    return;
  }
  fwd_tile(f, w.dq ? *w.mu : 0.f, lut, xrow, acc);
  // concatenated row index, row stride Ntot
#pragma unroll
  for (int h = 0; h < kTT; ++h)
    fwd_store(acc[h], y_part + span * T * Ntot + set.block0[m] * kFwdRows, Ntot, row0 + rl, T, g, h);
}

// Sum of `count` fp32 values p[0], p[stride], ... in index order, fetched
// kFinBatch at a time with every load of a batch issued before the adds.
constexpr int kFinBatch = 16;

__device__ __forceinline__ float strided_sum(const float *p, int64_t stride, int64_t count) {
  float s = 0.f;
  for (int64_t i0 = 0; i0 < count; i0 += kFinBatch) {
    float v[kFinBatch];
#pragma unroll
    for (int i = 0; i < kFinBatch; ++i) v[i] = p[min(i0 + i, count - 1) * stride];
#pragma unroll
    for (int i = 0; i < kFinBatch; ++i) s += i0 + i < count ? v[i] : 0.f;
  }
  return s;
}

// Forward, pass 2: a workgroup per 64 output rows (N may be 0: u only) and
// per group of TG tokens (blockIdx.y: tokens TG blockIdx.y .. + TG - 1 of T;
// one group for T <= 4, groups of 4 above).  u = bf16(sum of the span partials
// of u): with E = TG r entries, slice sl of S = 256 / E thread groups sums
// spans sl, sl + S, ... and the slices are added in order.  Thread (q, c) =
// (tid / 64, tid % 64) owns row n = 64 blockIdx.x + c and its quarter q of the
// rest: span partials q, q + 4, ... and the 8-wide rank chunks q, q + 4, ... of
// s u B^T; the four quarters are added in order.  Every load that does not
// need u is issued before u is reduced, so that one memory round trip covers
// them.  Tokens of the last group past T read token T - 1 and are never stored.
template <int TG>
__global__ __launch_bounds__(256) void gemv_fwd_finish(const float *__restrict__ y_part,
                                                       const float *__restrict__ u_part, int64_t spans,
                                                       GemvFwdSet set, int r, int ld_u, float scale,
                                                       float u_scale, int64_t Ntot, int T,
                                                       uint16_t *__restrict__ u_out) {
  __shared__ float us[TG * 256];
  __shared__ float tmp[1024];  // E S <= max(E, 256) entries, E = TG r <= 1024
  __shared__ float red[4][TG][64];
  const int tid = threadIdx.x;
  const int q = __builtin_amdgcn_readfirstlane(tid >> 6), c = tid & 63;
  const int t0 = TG * (int)blockIdx.y;
  auto tok = [&](int t) { return min(t0 + t, T - 1); };  // token of group position t (clamped)
  // this workgroup's member (Ntot = 0: u only, member 0) and its 64 rows
  const int m = Ntot > 0 ? fwd_member(set, blockIdx.x) : 0;
  const int64_t pl = (int64_t)blockIdx.x - set.block0[m];
  const int64_t N = Ntot > 0 ? set.w[m].n_out : 0;
  const uint16_t *__restrict__ B = set.B[m];
  uint16_t *__restrict__ y = set.y[m];
  const int64_t n = pl * 64 + c;
  const int64_t nc = n < N ? n : (N > 0 ? N - 1 : 0);
  const int64_t gc = set.block0[m] * 64 + nc;  // row in the concatenated partials
  const bool vec = (r & 7) == 0;
  const int nch = r / 8;
  const uint16_t *brow = B + nc * r;
  // first batch of this thread's partials and B chunks
  constexpr int kYB = kFinBatch / 2;
  float yp[kYB][TG];
  u32x4 b[8];
  if (N > 0) {
#pragma unroll
    for (int i = 0; i < kYB; ++i)
#pragma unroll
      for (int t = 0; t < TG; ++t) yp[i][t] = y_part[(min((int64_t)(q + 4 * i), spans - 1) * T + tok(t)) * Ntot + gc];
    if (vec) {
#pragma unroll
      for (int i = 0; i < 8; ++i) b[i] = *(const u32x4 *)(brow + 8 * min(q + 4 * i, nch - 1));
    }
  }
  const int E = TG * r, S = E >= 256 ? 1 : 256 / E;
  const int64_t per = (spans + S - 1) / S;
  // the member's u columns m r .. m r + r - 1 of the [span][t][ld_u] partials
  const int64_t ustride = (int64_t)T * ld_u;
  for (int idx = tid; idx < E * S; idx += 256) {
    const int e = idx % E, sl = idx / E;
    const int64_t cnt = max((int64_t)0, min(per, (spans - sl + S - 1) / S));
    tmp[idx] = strided_sum(u_part + sl * ustride + (int64_t)tok(e / r) * ld_u + m * r + e % r, (int64_t)S * ustride, cnt);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    float s = 0.f;
    for (int sl = 0; sl < S; ++sl) s += tmp[sl * E + e];
    const uint16_t h = to_bf16(s * u_scale);
    us[e] = bf(h);
    if (pl == 0 && t0 + e / r < T) u_out[(t0 + e / r) * ld_u + m * r + e % r] = h;
  }
  if (N == 0) return;
  __syncthreads();
  float ys[TG], lora[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) ys[t] = lora[t] = 0.f;
  for (int64_t s0 = q;; s0 += 4 * kYB) {
#pragma unroll
    for (int i = 0; i < kYB; ++i)
#pragma unroll
      for (int t = 0; t < TG; ++t) ys[t] += s0 + 4 * i < spans ? yp[i][t] : 0.f;
    if (s0 + 4 * kYB >= spans) break;
#pragma unroll
    for (int i = 0; i < kYB; ++i)
#pragma unroll
      for (int t = 0; t < TG; ++t) yp[i][t] = y_part[(min(s0 + 4 * kYB + 4 * i, spans - 1) * T + tok(t)) * Ntot + gc];
  }
  if (vec) {
    for (int c0 = q;; c0 += 32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ch = c0 + 4 * i;
        if (ch < nch) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int t = 0; t < TG; ++t) {
              lora[t] = __builtin_fmaf(us[t * r + 8 * ch + 2 * e], bf16_lo(b[i][e]), lora[t]);
              lora[t] = __builtin_fmaf(us[t * r + 8 * ch + 2 * e + 1], bf16_hi(b[i][e]), lora[t]);
            }
        }
      }
      if (c0 + 32 >= nch) break;
#pragma unroll
      for (int i = 0; i < 8; ++i) b[i] = *(const u32x4 *)(brow + 8 * min(c0 + 32 + 4 * i, nch - 1));
    }
  } else {
    for (int j0 = q; j0 < r; j0 += 32) {
      float bs[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) bs[i] = bf(brow[min(j0 + 4 * i, r - 1)]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = j0 + 4 * i;
        if (j < r) {
#pragma unroll
          for (int t = 0; t < TG; ++t) lora[t] = __builtin_fmaf(us[t * r + j], bs[i], lora[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TG; ++t) red[q][t][c] = ys[t] + scale * lora[t];
  __syncthreads();
  if (q == 0 && n < N) {
#pragma unroll
    for (int t = 0; t < TG; ++t)
      if (t0 + t < T) y[(t0 + t) * N + n] = to_bf16(red[0][t][c] + red[1][t][c] + red[2][t][c] + red[3][t][c]);
  }
}

// ---------------------------------------------------------------------------
// kRowsPerWave rows of one unit column with dy of those rows (zero past N).
template <int T>
struct BwdGroup {
  UnitLoad L[kRowsPerWave];
  float d[kRowsPerWave][T];
};

// The weights of one backward pass: up to kMaxSetMembers linears that share x, each with its dy,
// B and grad_B (a single linear is a set of one).  Member m owns weight chunks chunk0[m] ..
// chunk0[m + 1] - 1 and adapter workgroups part0[m] .. part0[m + 1] - 1; entries past the last
// member are past every chunk and workgroup.
struct GemvBwdSet {
  int count;
  QWeight w[kMaxSetMembers];
  const uint16_t *dy[kMaxSetMembers];
  const uint16_t *B[kMaxSetMembers];
  float *grad_B[kMaxSetMembers];
  int64_t chunk0[kMaxSetMembers + 1];
  int64_t part0[kMaxSetMembers + 1];
};

__device__ __forceinline__ int bwd_member(const int64_t (&first)[kMaxSetMembers + 1], int64_t i) {
  return (i >= first[1] ? 1 : 0) + (i >= first[2] ? 1 : 0) + (i >= first[3] ? 1 : 0);
}

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

// Backward, pass 1.  The first `awgs` workgroups each own `bsub` blocks of 64
// rows of B: grad_B rows and a partial v = dy B over their rows.  The others,
// id = blockIdx.x - awgs: span = id % spans, chunk = id / spans; wave w takes
// `groups` groups of kRowsPerWave rows starting at row
// (chunk * kBwdWaves + w) * groups * kRowsPerWave and accumulates 32 column
// sums per token.  The waves' sums are added through LDS in a fixed tree
// (halves added pairwise) and wave 0 writes the chunk's partial.
template <int T, bool Multi>
__device__ __forceinline__ void bwd_main_body(const GemvBwdSet &set, const uint16_t *__restrict__ u, int ld_u, int r,
                                              float scale, float *__restrict__ gx_part, float *__restrict__ v_part,
                                              int64_t spans, int64_t awgs, int groups, int bsub, const Codebook &cb,
                                              float *smem, float *lut) {
  static_assert(T <= 4, "adapter partials hold at most two entries per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = set.w[0].n_in;
  if ((int64_t)blockIdx.x < awgs) {
    // adapter rows [b * bsub * 64, ...) of the member's B, 64 at a time (r <= 256); b is the
    // workgroup's index within its member, bid its index among all adapter workgroups
    const int64_t bid = blockIdx.x;
    const int m = Multi ? bwd_member(set.part0, bid) : 0;
    const int64_t b = bid - set.part0[m], N = set.w[m].n_out;
    const uint16_t *__restrict__ dy = set.dy[m];
    const uint16_t *__restrict__ B = set.B[m];
    float *__restrict__ grad_B = set.grad_B[m];
    float *us = smem;                          // [T][r]
    float *ds = us + T * 256;                  // [T][64]
    uint16_t *bt = (uint16_t *)(ds + T * 64);  // [64][r]
    float *vt = (float *)(bt + kBRows * 256);  // [S][E]
    const int E = T * r, S = E >= kBwdThreads ? 1 : kBwdThreads / E;
    for (int e = tid; e < T * r; e += kBwdThreads) us[e] = bf(u[(e / r) * ld_u + m * r + e % r]);
    constexpr int kV = (1024 + kBwdThreads - 1) / kBwdThreads;  // E * S <= max(E, threads) <= 1024
    float vacc[kV];  // entries idx = tid + kBwdThreads k of the [S][E] slices
#pragma unroll
    for (int k = 0; k < kV; ++k) vacc[k] = 0.f;
    for (int sb = 0; sb < bsub; ++sb) {
      const int64_t n0 = (b * bsub + sb) * kBRows;
      if (n0 >= N) break;
      const int rows = (int)min((int64_t)kBRows, N - n0);
      __syncthreads();  // the previous block's tile is no longer read
      for (int e = tid; e < T * kBRows; e += kBwdThreads) {
        const int t = e / kBRows, i = e % kBRows;
        ds[e] = i < rows ? bf(dy[t * N + n0 + i]) : 0.f;
      }
      const uint16_t *bsrc = B + n0 * r;
      const int elems = rows * r;
      for (int e0 = tid; e0 < elems; e0 += kBwdThreads * 8) {
        uint16_t b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) b[i] = bsrc[min(e0 + kBwdThreads * i, elems - 1)];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (e0 + kBwdThreads * i < elems) bt[e0 + kBwdThreads * i] = b[i];
      }
      __syncthreads();
      for (int e = tid; e < elems; e += kBwdThreads) {
        const int i = e / r, j = e % r;
        float g = 0.f;
#pragma unroll
        for (int t = 0; t < T; ++t) g = __builtin_fmaf(ds[t * kBRows + i], us[t * r + j], g);
        grad_B[n0 * r + e] = scale * g;
      }
      // slice sl of the threads takes rows sl, sl + S, ... of this block
#pragma unroll
      for (int k = 0; k < kV; ++k) {
        const int idx = tid + kBwdThreads * k;
        if (idx < E * S) {
          const int e = idx % E, sl = idx / E, t = e / r, j = e % r;
          float s = vacc[k];
          for (int i = sl; i < rows; i += S) s = __builtin_fmaf(ds[t * kBRows + i], bf(bt[i * r + j]), s);
          vacc[k] = s;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kV; ++k)
      if (tid + kBwdThreads * k < E * S) vt[tid + kBwdThreads * k] = vacc[k];
    __syncthreads();
    for (int e = tid; e < E; e += kBwdThreads) {
      float s = 0.f;
      for (int sl = 0; sl < S; ++sl) s += vt[sl * E + e];
      v_part[bid * E + e] = s;
    }
    return;
  }

  if (tid < 16) lut[tid] = cb.v[tid];
  __syncthreads();
  const int64_t U = K / 32, kblk_row = K / kBlock;
  const int64_t id = (int64_t)blockIdx.x - awgs;
  const int64_t span = id % spans, chunk = id / spans;  // chunk among all members'
  const int m = Multi ? bwd_member(set.chunk0, chunk) : 0;
  const QWeight w = set.w[m];
  const uint16_t *__restrict__ dy = set.dy[m];
  const int64_t N = w.n_out;
  const int64_t unit = span * kSpanUnits + lane;
  const bool valid = unit < U;
  const int64_t uc = valid ? unit : U - 1;
  const int64_t n_base = ((chunk - set.chunk0[m]) * kBwdWaves + wave) * (int64_t)groups * kRowsPerWave;
  const float mu = w.dq ? *w.mu : 0.f;
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
  // fixed tree over the waves; smem holds [kBwdWaves / 2][T * 32][64]
#pragma unroll
  for (int half = kBwdWaves / 2; half >= 1; half >>= 1) {
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

// One token fits in 128 registers, which keeps two workgroups on every CU.  Multi: more than one
// member (a single linear reads member 0 without the lookup).
template <bool Multi>
__global__ __launch_bounds__(kBwdThreads, 4) void gemv_bwd_main_t1(GemvBwdSet set, const uint16_t *__restrict__ u,
                                                           int ld_u, int r, float scale,
                                                           float *__restrict__ gx_part, float *__restrict__ v_part,
                                                           int64_t spans, int64_t awgs, int groups, int bsub,
                                                           Codebook cb) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ float lut[16];
  bwd_main_body<1, Multi>(set, u, ld_u, r, scale, gx_part, v_part, spans, awgs, groups, bsub, cb, smem, lut);
}

template <int T, bool Multi>
__global__ __launch_bounds__(kBwdThreads) void gemv_bwd_main(GemvBwdSet set, const uint16_t *__restrict__ u, int ld_u,
                                                     int r, float scale, float *__restrict__ gx_part,
                                                     float *__restrict__ v_part, int64_t spans, int64_t awgs,
                                                     int groups, int bsub, Codebook cb) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ float lut[16];
  bwd_main_body<T, Multi>(set, u, ld_u, r, scale, gx_part, v_part, spans, awgs, groups, bsub, cb, smem, lut);
}

// Backward, pass 2: a workgroup per 64 columns; thread (jg, c) = (tid / 64,
// tid % 64) takes adapter rows j = jg, jg + 4, ... and chunk partials
// jg, jg + 4, ...; the four groups are added in order through LDS.  v is the
// sum of the adapter workgroups' partials, sliced like u in the forward pass.
// Every load that does not need v (the first kFinBatch rows of A and chunk
// partials of each thread, x) is issued before v is reduced.
template <int T>
__global__ __launch_bounds__(256) void gemv_bwd_finish(const float *__restrict__ gx_part, int64_t chunks,
                                                       const float *__restrict__ v_part, GemvBwdSet set,
                                                       const uint16_t *__restrict__ x, const uint16_t *__restrict__ A,
                                                       int r, int64_t K, float scale, const uint32_t *__restrict__ keep,
                                                       uint16_t *__restrict__ grad_x, float *__restrict__ grad_A) {
  // r is a member's rank; A and grad_A have rt = count r rows (member m: rows m r ..), and v
  // [T x rt] is member m's adapter partials summed in its columns
  const int rt = set.count * r;
  __shared__ float tmp[1024];
  __shared__ float vs[T * 256 * kMaxSetMembers];
  __shared__ float red[4][T][64];
  const int tid = threadIdx.x;
  const int jg = __builtin_amdgcn_readfirstlane(tid >> 6), c = tid & 63;
  const int64_t col = (int64_t)blockIdx.x * 64 + c;
  const bool valid = col < K;
  const int64_t cc = valid ? col : K - 1;
  float xv[T], a[kFinBatch], gv[kFinBatch][T];
#pragma unroll
  for (int t = 0; t < T; ++t) xv[t] = bf(x[t * K + cc]);
#pragma unroll
  for (int i = 0; i < kFinBatch; ++i) a[i] = bf(A[(int64_t)min(jg + 4 * i, rt - 1) * K + cc]);
  if (grad_x) {
#pragma unroll
    for (int i = 0; i < kFinBatch; ++i)
#pragma unroll
      for (int t = 0; t < T; ++t) gv[i][t] = gx_part[(min((int64_t)(jg + 4 * i), chunks - 1) * T + t) * K + cc];
  }
  const int E = T * r, S = E >= 256 ? 1 : 256 / E;
  for (int mm = 0; mm < set.count; ++mm) {
    const int64_t p0 = set.part0[mm], vparts = set.part0[mm + 1] - p0;
    const int64_t per = (vparts + S - 1) / S;
    for (int idx = tid; idx < E * S; idx += 256) {
      const int e = idx % E, sl = idx / E;
      const int64_t cnt = max((int64_t)0, min(per, (vparts - sl + S - 1) / S));
      tmp[idx] = strided_sum(v_part + (p0 + sl) * (int64_t)E + e, (int64_t)S * E, cnt);
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
      float s = 0.f;
      for (int sl = 0; sl < S; ++sl) s += tmp[sl * E + e];
      vs[(e / r) * rt + mm * r + e % r] = s;
    }
    __syncthreads();
  }
  float g[T], lora[T];
#pragma unroll
  for (int t = 0; t < T; ++t) g[t] = lora[t] = 0.f;
  for (int j0 = jg;; j0 += 4 * kFinBatch) {
#pragma unroll
    for (int i = 0; i < kFinBatch; ++i) {
      const int j = j0 + 4 * i;
      if (j < rt) {
        float ga = 0.f;
#pragma unroll
        for (int t = 0; t < T; ++t) {
          lora[t] = __builtin_fmaf(vs[t * rt + j], a[i], lora[t]);
          ga = __builtin_fmaf(vs[t * rt + j], xv[t], ga);
        }
        if (valid) grad_A[(int64_t)j * K + col] = scale * ga;
      }
    }
    if (j0 + 4 * kFinBatch >= rt) break;
#pragma unroll
    for (int i = 0; i < kFinBatch; ++i) a[i] = bf(A[(int64_t)min(j0 + 4 * kFinBatch + 4 * i, rt - 1) * K + cc]);
  }
  if (grad_x) {
    for (int64_t c0 = jg;; c0 += 4 * kFinBatch) {
#pragma unroll
      for (int i = 0; i < kFinBatch; ++i)
#pragma unroll
        for (int t = 0; t < T; ++t) g[t] += c0 + 4 * i < chunks ? gv[i][t] : 0.f;
      if (c0 + 4 * kFinBatch >= chunks) break;
#pragma unroll
      for (int i = 0; i < kFinBatch; ++i)
#pragma unroll
        for (int t = 0; t < T; ++t)
          gv[i][t] = gx_part[(min(c0 + 4 * kFinBatch + 4 * i, chunks - 1) * T + t) * K + cc];
    }
    // dropout: the adapter term of row t is kept where bit t of the column's word is set
    const uint32_t kw = keep ? keep[cc] : 0xFFFFFFFFu;
#pragma unroll
    for (int t = 0; t < T; ++t) red[jg][t][c] = g[t] + (((kw >> t) & 1u) ? scale * lora[t] : 0.f);
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
// kBwdTargetWaves (one token: kBwdTargetWavesT1) waves in flight.
struct GemvGeometry {
  int64_t funits, fspans, fblocks, ablocks;  // forward: span units, spans, weight and A workgroups
  int64_t bspans, groups, chunks;         // backward weight pass
  int64_t bsub, bparts;                   // backward adapter workgroups
};

GemvGeometry geometry(int64_t T, int64_t N, int64_t K, int r) {
  GemvGeometry g;
  const int64_t short_span_waves = cdiv(K / 32, kFwdUnitsSmall) * cdiv(N, 16);
  g.funits = short_span_waves <= kFwdShortSpanWaves ? kFwdUnitsSmall : kFwdUnitsLarge;
  g.fspans = cdiv(K / 32, g.funits);
  g.fblocks = g.fspans * cdiv(N, kFwdRows);
  g.ablocks = g.fspans * cdiv(r, kFwdRows);
  g.bspans = cdiv(K / 32, kSpanUnits);
  const int64_t rows_per_wave = g.bspans * N / (T == 1 ? kBwdTargetWavesT1 : kBwdTargetWaves);
  g.groups = std::max<int64_t>(1, std::min<int64_t>(4, rows_per_wave / kRowsPerWave));
  g.chunks = cdiv(N, kBwdWaves * g.groups * kRowsPerWave);
  const int64_t blocks = cdiv(N, kBRows);
  g.bsub = std::max<int64_t>(1, blocks / 64);
  g.bparts = cdiv(blocks, g.bsub);
  return g;
}

size_t bwd_lds_bytes(int T) {
  const size_t tree = (size_t)(kBwdWaves / 2) * T * 32 * 64 * 4;
  const size_t adapter = (size_t)T * 256 * 4 + (size_t)T * 64 * 4 + (size_t)kBRows * 256 * 2 + 1024 * 4;
  return std::max(tree, adapter);
}

constexpr int64_t kNoBlock = INT64_MAX / 4;  // block0 past every block

// The forward of a set: Ntot concatenated rows (rows == false: u only, from A [r_total x K]); u
// [T x r_total] holds every member's u (member m: columns m r ..).
template <int T>
hipError_t gemv_fwd_run(const uint16_t *x, const uint16_t *xa, const GemvFwdSet &set, int64_t Ntot, bool rows,
                        const uint16_t *A, int r, int r_total, float scale, float u_scale, uint16_t *u, float *part,
                        const Codebook &cb, hipStream_t st) {
  const GemvGeometry g = geometry(T, Ntot, set.w[0].n_in, r_total);
  const int64_t fblocks = rows ? g.fblocks : 0;
  float *y_part = part, *u_part = part + g.fspans * T * Ntot;
  const size_t lds = (size_t)T * (g.funits * 32 + 8) * 2;
  const unsigned grid = (unsigned)(fblocks + g.ablocks);
  constexpr int kTT = (T + 15) / 16;  // tiles of 16 tokens
  // the x tile is at most 40 KB above 16 tokens (gemv_fwd_applies), within the default LDS limit
  if (lds > kFwdMultiTileMaxLds && T > 16) return hipErrorInvalidValue;
  TimedLaunch tl;
  const bool timed = rows && timing_begin(st, tl, kTimedGemvFwd);
  if (g.funits == kFwdUnitsSmall) {
    gemv_fwd_main<kFwdUnitsSmall, kTT><<<grid, 256, lds, st>>>(x, xa, T, set, Ntot, A, r_total, y_part, u_part,
                                                               g.fspans, g.ablocks, cb);
  } else {
    // long spans hold at most 19 tokens in 40 KB
    if constexpr (kTT <= 2)
      gemv_fwd_main<kFwdUnitsLarge, kTT><<<grid, 256, lds, st>>>(x, xa, T, set, Ntot, A, r_total, y_part, u_part,
                                                                 g.fspans, g.ablocks, cb);
    else
      return hipErrorInvalidValue;
  }
  if (timed) timing_end(st, tl);
  const int64_t out_rows = rows ? Ntot : 0;
  const unsigned fg = (unsigned)std::max<int64_t>(1, cdiv(out_rows, 64));
  constexpr int TG = T <= 4 ? T : 4;  // tokens per finishing workgroup
  gemv_fwd_finish<TG><<<dim3(fg, (unsigned)((T + TG - 1) / TG)), 256, 0, st>>>(y_part, u_part, g.fspans, set, r, r_total,
                                                                               scale, u_scale, out_rows, (int)T, u);
  return hipGetLastError();
}

template <int T>
hipError_t gemv_fwd_impl(const uint16_t *x, const uint16_t *xa, const QWeight &w, const uint16_t *A, const uint16_t *B,
                         int r, float scale, float u_scale, uint16_t *y, uint16_t *u, float *part, const Codebook &cb,
                         hipStream_t st) {
  GemvFwdSet set{};
  set.count = 1;
  set.w[0] = w;
  set.B[0] = B;
  set.y[0] = y;
  set.block0[0] = 0;
  for (int i = 1; i <= kMaxSetMembers; ++i) set.block0[i] = kNoBlock;
  for (int i = 1; i < kMaxSetMembers; ++i) set.w[i] = w;
  return gemv_fwd_run<T>(x, xa, set, w.n_out, y != nullptr, A, r, r, scale, u_scale, u, part, cb, st);
}

template <int T>
hipError_t gemv_fwd_set_impl(const uint16_t *x, const QWeight *w, int count, const uint16_t *A_set,
                             const uint16_t *const *B, int r, float scale, uint16_t *const *y, uint16_t *u_set,
                             float *part, const Codebook &cb, hipStream_t st) {
  GemvFwdSet set{};
  set.count = count;
  int64_t blocks = 0, Ntot = 0;
  for (int i = 0; i < kMaxSetMembers; ++i) {
    set.w[i] = w[i < count ? i : 0];
    set.B[i] = i < count ? B[i] : B[0];
    set.y[i] = i < count ? y[i] : y[0];
    set.block0[i] = i < count ? blocks : kNoBlock;
    if (i < count) {
      blocks += cdiv(w[i].n_out, kFwdRows);
      Ntot += w[i].n_out;
    }
  }
  set.block0[kMaxSetMembers] = kNoBlock;
  return gemv_fwd_run<T>(x, x, set, Ntot, true, A_set, r, count * r, scale, 1.0f, u_set, part, cb, st);
}

// Work split of a backward set: the geometry of the concatenated rows decides the rows per wave
// and the adapter blocks per workgroup; each member then takes whole chunks and adapter
// workgroups of its own.
struct BwdSplit {
  GemvGeometry g;
  int64_t chunks, parts;
};

static BwdSplit bwd_split(int64_t T, GemvBwdSet &set, int64_t K, int r) {
  int64_t ntot = 0;
  for (int i = 0; i < set.count; ++i) ntot += set.w[i].n_out;
  BwdSplit b;
  b.g = geometry(T, ntot, K, r);
  const int64_t chunk_rows = (int64_t)kBwdWaves * b.g.groups * kRowsPerWave;
  b.chunks = 0;
  b.parts = 0;
  for (int i = 0; i <= kMaxSetMembers; ++i) {
    set.chunk0[i] = i <= set.count ? b.chunks : kNoBlock;
    set.part0[i] = i <= set.count ? b.parts : kNoBlock;
    if (i < set.count) {
      b.chunks += cdiv(set.w[i].n_out, chunk_rows);
      b.parts += cdiv(cdiv(set.w[i].n_out, kBRows), b.g.bsub);
    }
  }
  // lookups compare against entries 1 .. 3: a member past the last never matches
  for (int i = set.count + 1; i <= kMaxSetMembers; ++i) set.chunk0[i] = set.part0[i] = kNoBlock;
  return b;
}

template <int T, bool Multi>
hipError_t gemv_bwd_run(GemvBwdSet &set, const uint16_t *xa, const uint16_t *A, int r, float scale, float scale_ax,
                        const uint32_t *keep, const uint16_t *u, int ld_u, uint16_t *grad_x, float *grad_A,
                        float *part, const Codebook &cb, hipStream_t st) {
  const int64_t K = set.w[0].n_in;
  const BwdSplit b = bwd_split(T, set, K, r);
  const int64_t nf4_wgs = grad_x ? b.g.bspans * b.chunks : 0;
  float *gx_part = part, *v_part = part + b.chunks * T * K;
  const size_t lds = bwd_lds_bytes(T);
  const void *fn = T == 1 ? (const void *)gemv_bwd_main_t1<Multi> : (const void *)gemv_bwd_main<T, Multi>;
  // the attribute is set once per device, token count and variant (the size depends on T only), so
  // calls under stream capture make no attribute call
  static bool lds_set[64][kGemvMaxT + 1] = {};
  int dev = 0;
  if (lds > 64 * 1024) {
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!lds_set[dev][T]) {
      const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      lds_set[dev][T] = true;
    }
  }
  const unsigned grid = (unsigned)(nf4_wgs + b.parts);  // adapter workgroups first
  TimedLaunch tl;
  const bool timed = grad_x && timing_begin(st, tl, kTimedGemvBwd);
  if (T == 1)
    gemv_bwd_main_t1<Multi><<<grid, kBwdThreads, lds, st>>>(set, u, ld_u, r, scale, gx_part, v_part, b.g.bspans, b.parts,
                                                     (int)b.g.groups, (int)b.g.bsub, cb);
  else
    gemv_bwd_main<T, Multi><<<grid, kBwdThreads, lds, st>>>(set, u, ld_u, r, scale, gx_part, v_part, b.g.bspans, b.parts,
                                                     (int)b.g.groups, (int)b.g.bsub, cb);
  if (timed) timing_end(st, tl);
  gemv_bwd_finish<T><<<(unsigned)cdiv(K, 64), 256, 0, st>>>(gx_part, b.chunks, v_part, set, xa, A, r, K, scale_ax,
                                                            keep, grad_x, grad_A);
  return hipGetLastError();
}

template <int T>
hipError_t gemv_bwd_impl(const uint16_t *dy, const uint16_t *xa, const QWeight &w, const uint16_t *A,
                         const uint16_t *B, int r, float scale, float scale_ax, const uint32_t *keep, const uint16_t *u,
                         uint16_t *grad_x, float *grad_A, float *grad_B, float *part, const Codebook &cb,
                         hipStream_t st) {
  GemvBwdSet set{};
  set.count = 1;
  for (int i = 0; i < kMaxSetMembers; ++i) {
    set.w[i] = w;
    set.dy[i] = dy;
    set.B[i] = B;
    set.grad_B[i] = grad_B;
  }
  return gemv_bwd_run<T, false>(set, xa, A, r, scale, scale_ax, keep, u, r, grad_x, grad_A, part, cb, st);
}

template <int T>
hipError_t gemv_bwd_set_impl(const uint16_t *const *dy, const uint16_t *x, const QWeight *w, int count,
                             const uint16_t *A_set, const uint16_t *const *B, int r, float scale, const uint16_t *u_set,
                             uint16_t *grad_x, float *grad_A_set, float *const *grad_B, float *part,
                             const Codebook &cb, hipStream_t st) {
  GemvBwdSet set{};
  set.count = count;
  for (int i = 0; i < kMaxSetMembers; ++i) {
    const int k = i < count ? i : 0;
    set.w[i] = w[k];
    set.dy[i] = dy[k];
    set.B[i] = B[k];
    set.grad_B[i] = grad_B[k];
  }
  return count > 1 ? gemv_bwd_run<T, true>(set, x, A_set, r, scale, scale, nullptr, u_set, count * r, grad_x,
                                            grad_A_set, part, cb, st)
                   : gemv_bwd_run<T, false>(set, x, A_set, r, scale, scale, nullptr, u_set, count * r, grad_x,
                                            grad_A_set, part, cb, st);
}

}  // namespace

// A single linear's backward runs here up to 2 tokens, and up to 4 when the weight is small: with
// the row split of two and more tokens the few-token pass beats the fused GEMM's backward at 4096^2
// (3 tokens 45.2 -> 39.2 us per fwd+bwd, 4 tokens 46.6 -> 42.9) but not at 22016 x 8192 (4 tokens
// 124 -> 135 us).  A projection set's one pass over all its members' rows runs up to 4 tokens, and
// up to 3 once the members hold more than 128 M weights in all (q/k/v of 3 x 8192^2, backward alone
// at 4 tokens: 119.6 us here against 108.6 on the fused GEMM; gate/up of 2 x 11008 x 4096 even).
constexpr int64_t kGemvLargeSet = (int64_t)128 << 20;

bool gemv_bwd_applies(int64_t T, int64_t N, int64_t K, int count) {
  int64_t max_t = count > 1 || N * K <= kGemvSmallWeight ? kGemvMaxT : kGemvLinearBwdMaxT;
  if (count > 1 && N * K > kGemvLargeSet) max_t = 3;
  return T >= 1 && T <= max_t && K % 64 == 0;
}
bool gemv_fwd_applies(int64_t T, int64_t N, int64_t K) {
  if (T < 1 || T > kGemvFwdMaxT || K % 64 != 0) return false;
  if (T <= 16) return true;
  const GemvGeometry g = geometry(T, N, K, 0);
  return (size_t)T * (g.funits * 32 + 8) * 2 <= kFwdMultiTileMaxLds;
}

bool gemv_set_fusable(const int64_t *N, int count) {
  for (int i = 0; i + 1 < count; ++i)
    if (N[i] % kFwdRows != 0) return false;
  return true;
}

hipError_t launch_gemv_fwd_set(int64_t T, const uint16_t *x, const QWeight *w, int count, const uint16_t *A_set,
                               const uint16_t *const *B, int r, float scale, uint16_t *const *y, uint16_t *u_set,
                               float *part, const Codebook &cb, hipStream_t st) {
  switch (T) {
    case 1: return gemv_fwd_set_impl<1>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 2: return gemv_fwd_set_impl<2>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 3: return gemv_fwd_set_impl<3>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 4: return gemv_fwd_set_impl<4>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 5: return gemv_fwd_set_impl<5>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 6: return gemv_fwd_set_impl<6>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 7: return gemv_fwd_set_impl<7>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 8: return gemv_fwd_set_impl<8>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 9: return gemv_fwd_set_impl<9>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 10: return gemv_fwd_set_impl<10>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 11: return gemv_fwd_set_impl<11>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 12: return gemv_fwd_set_impl<12>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 13: return gemv_fwd_set_impl<13>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 14: return gemv_fwd_set_impl<14>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 15: return gemv_fwd_set_impl<15>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 16: return gemv_fwd_set_impl<16>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 17: return gemv_fwd_set_impl<17>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 18: return gemv_fwd_set_impl<18>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 19: return gemv_fwd_set_impl<19>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 20: return gemv_fwd_set_impl<20>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 21: return gemv_fwd_set_impl<21>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 22: return gemv_fwd_set_impl<22>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 23: return gemv_fwd_set_impl<23>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 24: return gemv_fwd_set_impl<24>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 25: return gemv_fwd_set_impl<25>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 26: return gemv_fwd_set_impl<26>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 27: return gemv_fwd_set_impl<27>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 28: return gemv_fwd_set_impl<28>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 29: return gemv_fwd_set_impl<29>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 30: return gemv_fwd_set_impl<30>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 31: return gemv_fwd_set_impl<31>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 32: return gemv_fwd_set_impl<32>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 33: return gemv_fwd_set_impl<33>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 34: return gemv_fwd_set_impl<34>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 35: return gemv_fwd_set_impl<35>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 36: return gemv_fwd_set_impl<36>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 37: return gemv_fwd_set_impl<37>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 38: return gemv_fwd_set_impl<38>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 39: return gemv_fwd_set_impl<39>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 40: return gemv_fwd_set_impl<40>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 41: return gemv_fwd_set_impl<41>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 42: return gemv_fwd_set_impl<42>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 43: return gemv_fwd_set_impl<43>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 44: return gemv_fwd_set_impl<44>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 45: return gemv_fwd_set_impl<45>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 46: return gemv_fwd_set_impl<46>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 47: return gemv_fwd_set_impl<47>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 48: return gemv_fwd_set_impl<48>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 49: return gemv_fwd_set_impl<49>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 50: return gemv_fwd_set_impl<50>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 51: return gemv_fwd_set_impl<51>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 52: return gemv_fwd_set_impl<52>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 53: return gemv_fwd_set_impl<53>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 54: return gemv_fwd_set_impl<54>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 55: return gemv_fwd_set_impl<55>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 56: return gemv_fwd_set_impl<56>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 57: return gemv_fwd_set_impl<57>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 58: return gemv_fwd_set_impl<58>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 59: return gemv_fwd_set_impl<59>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 60: return gemv_fwd_set_impl<60>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 61: return gemv_fwd_set_impl<61>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 62: return gemv_fwd_set_impl<62>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 63: return gemv_fwd_set_impl<63>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    case 64: return gemv_fwd_set_impl<64>(x, w, count, A_set, B, r, scale, y, u_set, part, cb, st);
    default: return hipErrorInvalidValue;
  }
}

size_t gemv_set_part_floats(int64_t T, const int64_t *N, int count, int64_t K, int r) {
  GemvBwdSet set{};
  set.count = count;
  for (int i = 0; i < count; ++i) set.w[i].n_out = N[i];
  const BwdSplit b = bwd_split(T, set, K, r);
  const size_t bwd = (size_t)(b.chunks * T * K + b.parts * T * r);
  return std::max(gemv_set_fwd_part_floats(T, N, count, K, r), bwd);
}

size_t gemv_set_fwd_part_floats(int64_t T, const int64_t *N, int count, int64_t K, int r) {
  int64_t ntot = 0;
  for (int i = 0; i < count; ++i) ntot += N[i];
  const GemvGeometry gf = geometry(T, ntot, K, count * r);
  return (size_t)(gf.fspans * T * (ntot + (int64_t)count * r));
}

hipError_t launch_gemv_bwd_set(int64_t T, const uint16_t *const *dy, const uint16_t *x, const QWeight *w, int count,
                               const uint16_t *A_set, const uint16_t *const *B, int r, float scale,
                               const uint16_t *u_set, uint16_t *grad_x, float *grad_A_set, float *const *grad_B,
                               float *part, const Codebook &cb, hipStream_t st) {
  switch (T) {
    case 1: return gemv_bwd_set_impl<1>(dy, x, w, count, A_set, B, r, scale, u_set, grad_x, grad_A_set, grad_B, part, cb, st);
    case 2: return gemv_bwd_set_impl<2>(dy, x, w, count, A_set, B, r, scale, u_set, grad_x, grad_A_set, grad_B, part, cb, st);
    case 3: return gemv_bwd_set_impl<3>(dy, x, w, count, A_set, B, r, scale, u_set, grad_x, grad_A_set, grad_B, part, cb, st);
    case 4: return gemv_bwd_set_impl<4>(dy, x, w, count, A_set, B, r, scale, u_set, grad_x, grad_A_set, grad_B, part, cb, st);
    default: return hipErrorInvalidValue;
  }
}

size_t gemv_part_floats(int64_t T, int64_t N, int64_t K, int r) {
  const GemvGeometry g = geometry(T, N, K, r);
  const size_t bwd = (size_t)(g.chunks * T * K + g.bparts * T * r);
  return std::max(gemv_fwd_part_floats(T, N, K, r), bwd);
}

size_t gemv_fwd_part_floats(int64_t T, int64_t N, int64_t K, int r) {
  const GemvGeometry g = geometry(T, N, K, r);
  return (size_t)(g.fspans * T * (N + r));
}

hipError_t launch_gemv_fwd(int64_t T, const uint16_t *x, const uint16_t *xa, const QWeight &w, const uint16_t *A,
                           const uint16_t *B, int r, float scale, float u_scale, uint16_t *y, uint16_t *u,
                           float *part, const Codebook &cb, hipStream_t st) {
  switch (T) {
    case 1: return gemv_fwd_impl<1>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 2: return gemv_fwd_impl<2>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 3: return gemv_fwd_impl<3>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 4: return gemv_fwd_impl<4>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 5: return gemv_fwd_impl<5>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 6: return gemv_fwd_impl<6>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 7: return gemv_fwd_impl<7>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 8: return gemv_fwd_impl<8>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 9: return gemv_fwd_impl<9>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 10: return gemv_fwd_impl<10>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 11: return gemv_fwd_impl<11>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 12: return gemv_fwd_impl<12>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 13: return gemv_fwd_impl<13>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 14: return gemv_fwd_impl<14>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 15: return gemv_fwd_impl<15>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 16: return gemv_fwd_impl<16>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 17: return gemv_fwd_impl<17>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 18: return gemv_fwd_impl<18>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 19: return gemv_fwd_impl<19>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 20: return gemv_fwd_impl<20>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 21: return gemv_fwd_impl<21>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 22: return gemv_fwd_impl<22>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 23: return gemv_fwd_impl<23>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 24: return gemv_fwd_impl<24>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 25: return gemv_fwd_impl<25>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 26: return gemv_fwd_impl<26>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 27: return gemv_fwd_impl<27>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 28: return gemv_fwd_impl<28>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 29: return gemv_fwd_impl<29>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 30: return gemv_fwd_impl<30>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 31: return gemv_fwd_impl<31>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 32: return gemv_fwd_impl<32>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 33: return gemv_fwd_impl<33>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 34: return gemv_fwd_impl<34>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 35: return gemv_fwd_impl<35>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 36: return gemv_fwd_impl<36>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 37: return gemv_fwd_impl<37>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 38: return gemv_fwd_impl<38>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 39: return gemv_fwd_impl<39>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 40: return gemv_fwd_impl<40>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 41: return gemv_fwd_impl<41>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 42: return gemv_fwd_impl<42>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 43: return gemv_fwd_impl<43>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 44: return gemv_fwd_impl<44>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 45: return gemv_fwd_impl<45>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 46: return gemv_fwd_impl<46>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 47: return gemv_fwd_impl<47>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 48: return gemv_fwd_impl<48>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 49: return gemv_fwd_impl<49>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 50: return gemv_fwd_impl<50>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 51: return gemv_fwd_impl<51>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 52: return gemv_fwd_impl<52>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 53: return gemv_fwd_impl<53>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 54: return gemv_fwd_impl<54>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 55: return gemv_fwd_impl<55>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 56: return gemv_fwd_impl<56>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 57: return gemv_fwd_impl<57>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 58: return gemv_fwd_impl<58>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 59: return gemv_fwd_impl<59>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 60: return gemv_fwd_impl<60>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 61: return gemv_fwd_impl<61>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 62: return gemv_fwd_impl<62>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 63: return gemv_fwd_impl<63>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    case 64: return gemv_fwd_impl<64>(x, xa, w, A, B, r, scale, u_scale, y, u, part, cb, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv_bwd(int64_t T, const uint16_t *dy, const uint16_t *xa, const QWeight &w, const uint16_t *A,
                           const uint16_t *B, int r, float scale, float scale_ax, const uint32_t *keep,
                           const uint16_t *u, uint16_t *grad_x, float *grad_A, float *grad_B, float *part,
                           const Codebook &cb, hipStream_t st) {
  switch (T) {
    case 1: return gemv_bwd_impl<1>(dy, xa, w, A, B, r, scale, scale_ax, keep, u, grad_x, grad_A, grad_B, part, cb, st);
    case 2: return gemv_bwd_impl<2>(dy, xa, w, A, B, r, scale, scale_ax, keep, u, grad_x, grad_A, grad_B, part, cb, st);
    case 3: return gemv_bwd_impl<3>(dy, xa, w, A, B, r, scale, scale_ax, keep, u, grad_x, grad_A, grad_B, part, cb, st);
    case 4: return gemv_bwd_impl<4>(dy, xa, w, A, B, r, scale, scale_ax, keep, u, grad_x, grad_A, grad_B, part, cb, st);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Few-token projection sets whose forward runs member by member: u moves
// between the set's [T x count r] layout and one [T x r] block.

namespace {

__global__ __launch_bounds__(256) void copy_rows_u16(const uint16_t *__restrict__ src, int64_t ld_src,
                                                     uint16_t *__restrict__ dst, int64_t ld_dst, int64_t rows,
                                                     int64_t cols) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows * cols; i += (int64_t)gridDim.x * 256)
    dst[(i / cols) * ld_dst + i % cols] = src[(i / cols) * ld_src + i % cols];
}

}  // namespace

hipError_t launch_copy_rows(const uint16_t *src, int64_t ld_src, uint16_t *dst, int64_t ld_dst, int64_t rows,
                            int64_t cols, hipStream_t st) {
  const int64_t n = rows * cols;
  if (n <= 0) return hipSuccess;
  copy_rows_u16<<<(unsigned)std::min<int64_t>(cdiv(n, 256), 1024), 256, 0, st>>>(src, ld_src, dst, ld_dst, rows,
                                                                                    cols);
  return hipGetLastError();
}

}  // namespace qlora
