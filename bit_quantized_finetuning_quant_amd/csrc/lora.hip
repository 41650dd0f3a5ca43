// The adapter-side products of the QLoRA linear layer (gfx950), one kernel
// family for all four of them.
//
// Adapter algebra: W' = W + s.B.A with A [r x n_in], B [n_out x r] (the LoRA
// formula of the nexusinovation tutorial, section "LoRA: O Padrão Ouro de
// Eficiência"); only the adapters receive gradients ("qlora" encyclopedia
// entry, tonho.wtf, section "a ideia").
//
//   u      = x A^T        [T x r]      A op: x (rows)          B op: A (rows)
//   v      = dy B         [T x r]      A op: dy (rows)         B op: B (columns)
//   grad_A = s v^T x      [r x n_in]   A op: v (columns)       B op: x (columns)
//   grad_B = s dy^T u     [n_out x r]  A op: dy (columns)      B op: u (columns)
//
// C[M x Nc] = scale * sum_k Aop(m, k) Bop(k, n), where an operand is either
// "row" (its contraction index is contiguous: Aop(m, k) = P[m ld + k]) or
// "column" (the contraction index strides: Aop(m, k) = P[k ld + m]).  Tiles of
// both operands are staged in LDS in their natural layout; "column" operands
// reach the MFMA through LDS transpose reads (ds_read_b64_tr_b16).  The
// contraction is split over the grid's z dimension; every split writes an
// fp32 partial tile and a second kernel adds the partials in split order (so
// the result is deterministic) and writes the scaled output.

#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace qlora {

namespace {

constexpr int LT = 64;   // output tile (M and N) and contraction step
constexpr int LLD = 72;  // LDS row length (bf16), padded

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld8(const uint16_t *row, int64_t c, int64_t ncols, bool vec) {
  if (vec && c + 8 <= ncols) return *(const u32x4 *)(row + c);
  u32x4 v = {0u, 0u, 0u, 0u};
  for (int i = 0; i < 8; ++i)
    if (c + i < ncols) v[i >> 1] |= (uint32_t)row[c + i] << (16 * (i & 1));
  return v;
}

// Tile rows [r0, r0 + 64) x columns [c0, c0 + 64) of a row-major [nrows x ld]
// bf16 matrix (columns >= ncols and rows >= nrows read as zero); thread t
// fetches columns 8 (t%8) .. +7 of rows t/8 and t/8 + 32, so that each wave's
// load covers 8 whole 128-byte rows (a load that covers half of each of 16
// lines moves about half as many bytes per cycle from L2).  kFull: the tile is
// known to be in range and 16-byte aligned, so the loads are unconditional.
struct TileRegs {
  u32x4 v[2];
};

template <bool kFull>
__device__ __forceinline__ void load_tile(const uint16_t *src, int64_t ld, int64_t nrows, int64_t ncols,
                                          int64_t r0, int64_t c0, bool vec, int tid, TileRegs &t) {
  const int64_t row = r0 + (tid >> 3);
  const int64_t col = c0 + 8 * (tid & 7);
  if (kFull) {
    const uint16_t *p = src + row * ld + col;
    t.v[0] = *(const u32x4 *)p;
    t.v[1] = *(const u32x4 *)(p + 32 * ld);
    return;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
    t.v[h] = (row + 32 * h < nrows) ? ld8(src + (row + 32 * h) * ld, col, ncols, vec) : u32x4{0u, 0u, 0u, 0u};
}

__device__ __forceinline__ void store_tile(const TileRegs &t, uint16_t *lds, int tid) {
#pragma unroll
  for (int h = 0; h < 2; ++h) *(u32x4 *)&lds[((tid >> 3) + 32 * h) * LLD + 8 * (tid & 7)] = t.v[h];
}

// MFMA operand fragment for output rows/cols [base, base + 32), contraction
// sub-step kk (16 wide).  kTrans = false: the LDS tile is [out][contraction];
// kTrans = true: the LDS tile is [contraction][out] and is read transposed
// (in each 16-lane group, source lane s points at contraction row
// 16 kk + 8 (g/2) + s/4 (and +4) and output column 16 (g%2) + 4 (s%4); lane l
// then holds 4 consecutive contraction rows of output column l%32).
template <bool kTrans>
__device__ __forceinline__ u32x4 frag(const uint16_t *lds, int base, int kk, int lane) {
  if (!kTrans) return *(const u32x4 *)&lds[(base + (lane & 31)) * LLD + 16 * kk + 8 * (lane >> 5)];
  const int s = lane & 15, g = lane >> 4;
  const int row = 16 * kk + 8 * (g >> 1) + (s >> 2);
  const int col = base + 16 * (g & 1) + 4 * (s & 3);
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3))) *)(lds_void_t *)&lds[row * LLD + col]);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3))) *)(lds_void_t *)&lds[(row + 4) * LLD + col]);
  const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
  return u32x4{l2.x, l2.y, h2.x, h2.y};
}

// Contraction steps fetched at once: 4 (a group of 256) or, when a split is
// exactly 512 long and the launch fits one round of workgroups, all 8 of it,
// so that the whole split arrives in one round trip (128 KB per workgroup in
// flight, 147 KB of LDS).

template <bool kAT, bool kBT, bool kBf16Out, bool kFull, int kGroupSteps>
__device__ __forceinline__ void lora_body(const uint16_t *__restrict__ P, int64_t ldp,
                                          const uint16_t *__restrict__ Q, int64_t ldq, int64_t M, int64_t Nc,
                                          int64_t kb, int64_t ke, int64_t m0, int64_t n0, uint16_t (*sA)[LT * LLD],
                                          uint16_t (*sB)[LT * LLD], f32x16 &acc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // 16-byte loads need 16-byte aligned rows: the row stride and the base (a
  // member's columns of a set's u may start mid-row)
  const bool vp = (ldp % 8) == 0 && ((uintptr_t)P & 15u) == 0, vq = (ldq % 8) == 0 && ((uintptr_t)Q & 15u) == 0;
  // Operand tiles in natural layout: a row operand as [out rows][contraction],
  // a column operand as [contraction rows][out columns].  A group of
  // contraction steps is fetched at once; the next group's loads reuse the
  // registers as soon as the current group is in LDS, so they overlap with its
  // MFMAs.
  TileRegs ta[kGroupSteps], tb[kGroupSteps];
  auto fetch = [&](int64_t g0) {
#pragma unroll
    for (int st = 0; st < kGroupSteps; ++st) {
      const int64_t k0 = g0 + LT * st;
      if (!kAT)
        load_tile<kFull>(P, ldp, M, ke, m0, k0, vp, tid, ta[st]);
      else
        load_tile<kFull>(P, ldp, ke, M, k0, m0, vp, tid, ta[st]);
      if (!kBT)
        load_tile<kFull>(Q, ldq, Nc, ke, n0, k0, vq, tid, tb[st]);
      else
        load_tile<kFull>(Q, ldq, ke, Nc, k0, n0, vq, tid, tb[st]);
    }
  };
  fetch(kb);
  for (int64_t g0 = kb; g0 < ke; g0 += LT * kGroupSteps) {
#pragma unroll
    for (int st = 0; st < kGroupSteps; ++st) {
      store_tile(ta[st], sA[st], tid);
      store_tile(tb[st], sB[st], tid);
    }
    __syncthreads();
    // next group while this one multiplies (a uniform branch: the registers
    // are next needed by the LDS store above, which waits for them anyway)
    if (g0 + LT * kGroupSteps < ke) fetch(g0 + LT * kGroupSteps);
#pragma unroll
    for (int st = 0; st < kGroupSteps; ++st)
#pragma unroll
      for (int kk = 0; kk < LT / 16; ++kk) {
        const u32x4 a = frag<kAT>(sA[st], wm * 32, kk, lane);
        const u32x4 b = frag<kBT>(sB[st], wn * 32, kk, lane);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), acc, 0, 0, 0);
      }
    __syncthreads();
  }
}

template <bool kBf16Out>
__device__ __forceinline__ void emit_out(void *out, int64_t idx, float v) {
  if (kBf16Out) {
    __bf16 h = (__bf16)v;
    ((uint16_t *)out)[idx] = __builtin_bit_cast(uint16_t, h);
  } else {
    ((float *)out)[idx] = v;
  }
}

// One adapter product of a launch: C[M x Nc] = scale * Aop Bop over a
// contraction of Kc, split in chunks of `chunk` (S splits); tiles are numbered
// column-major (tile = n-tile * tiles_m + m-tile).
struct LoraProblem {
  const uint16_t *P;
  int64_t ldp;
  const uint16_t *Q;
  int64_t ldq;
  int64_t M, Nc, Kc, chunk, tiles_m;
  int S;
  float scale;  // applied here when S == 1, else by the reduction
  void *out;
  int64_t ldo;  // row stride of out (Nc unless the product fills columns of a wider matrix)
  float *part;
};

template <bool kAT, bool kBT, bool kBf16Out, int kGroupSteps>
__device__ __forceinline__ void lora_tile(const LoraProblem &pr, int64_t tile, int s, uint16_t (*sA)[LT * LLD],
                                          uint16_t (*sB)[LT * LLD]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (tile % pr.tiles_m) * LT, n0 = (tile / pr.tiles_m) * LT;
  const int64_t kb = (int64_t)s * pr.chunk, ke = min(pr.Kc, kb + pr.chunk);

  f32x16 acc;
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.f;
  // full: both operand tiles in range and aligned, and the chunk is whole groups
  const bool full = (m0 + LT <= pr.M) && (n0 + LT <= pr.Nc) && ((ke - kb) % (LT * kGroupSteps) == 0) &&
                    (pr.ldp % 8 == 0) && (pr.ldq % 8 == 0) && (((uintptr_t)pr.P & 15u) == 0) &&
                    (((uintptr_t)pr.Q & 15u) == 0);
  if (full)
    lora_body<kAT, kBT, kBf16Out, true, kGroupSteps>(pr.P, pr.ldp, pr.Q, pr.ldq, pr.M, pr.Nc, kb, ke, m0, n0, sA, sB,
                                                      acc);
  else
    lora_body<kAT, kBT, kBf16Out, false, kGroupSteps>(pr.P, pr.ldp, pr.Q, pr.ldq, pr.M, pr.Nc, kb, ke, m0, n0, sA,
                                                       sB, acc);

  // result element q of this lane: tile row wm*32 + 8(q/4) + 4(lane/32) + q%4, column wn*32 + lane%32
  const int col = wn * 32 + (lane & 31);
  if (pr.S == 1) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t gm = m0 + wm * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3), gn = n0 + col;
      if (gm < pr.M && gn < pr.Nc) emit_out<kBf16Out>(pr.out, gm * pr.ldo + gn, acc[q] * pr.scale);
    }
    return;
  }
  // partial tile, row-major 64 x 64, at part[((tile * S) + s) * 4096]
  float *mine = pr.part + (tile * pr.S + s) * (LT * LT);
#pragma unroll
  for (int q = 0; q < 16; ++q) mine[(wm * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)) * LT + col] = acc[q];
}

// One or two products of the same operand forms in one launch: workgroups
// below `first` take problem a (tile-major, splits innermost), the rest
// problem b.
template <bool kAT, bool kBT, bool kBf16Out, int kGroupSteps>
__global__ __launch_bounds__(256) void lora_gemm(LoraProblem a, LoraProblem b, int64_t first) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[kGroupSteps][LT * LLD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kGroupSteps][LT * LLD];
  const int64_t id = blockIdx.x;
  const bool in_a = id < first;
  const LoraProblem &pr = in_a ? a : b;
  const int64_t j = in_a ? id : id - first;
  lora_tile<kAT, kBT, kBf16Out, kGroupSteps>(pr, j / pr.S, (int)(j % pr.S), sA, sB);
}

// out = scale * (sum over splits, in split order) of the partial tiles; one
// thread per 4 consecutive columns of a tile row.  Quads below `first` belong
// to problem a, the rest to problem b.
template <bool kBf16Out>
__device__ __forceinline__ void reduce_quad(const LoraProblem &pr, int64_t qd) {
  const int64_t tile = qd / (LT * LT / 4);
  const int local = (int)(qd % (LT * LT / 4)) * 4;
  const int64_t gm = (tile % pr.tiles_m) * LT + local / LT;
  const int64_t gn = (tile / pr.tiles_m) * LT + local % LT;
  if (gm >= pr.M || gn >= pr.Nc) return;
  const int S = pr.S;
  const f32x4 *p = (const f32x4 *)(pr.part + tile * S * (LT * LT) + local);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // eight loads in flight at a time; the additions stay in split order
  for (int k0 = 0; k0 < S; k0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = (k0 + k < S) ? p[(int64_t)(k0 + k) * (LT * LT / 4)] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      acc[0] += v[k][0];
      acc[1] += v[k][1];
      acc[2] += v[k][2];
      acc[3] += v[k][3];
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (gn + e < pr.Nc) emit_out<kBf16Out>(pr.out, gm * pr.ldo + gn + e, acc[e] * pr.scale);
}

template <bool kBf16Out>
__global__ __launch_bounds__(256) void lora_reduce(LoraProblem a, LoraProblem b, int64_t first, int64_t quads) {
  for (int64_t qd = (int64_t)blockIdx.x * 256 + threadIdx.x; qd < quads; qd += (int64_t)gridDim.x * 256) {
    if (qd < first)
      reduce_quad<kBf16Out>(a, qd);
    else
      reduce_quad<kBf16Out>(b, qd - first);
  }
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// Contraction splits: about 256 workgroups in all, chunks of whole groups.
static int64_t lora_chunk(int64_t tiles, int64_t kc) {
  const int64_t grp = LT * 4;
  int64_t s = cdiv(256, tiles);
  const int64_t max_s = cdiv(kc, grp);
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return cdiv(cdiv(kc, s), grp) * grp;
}

int lora_splits(int64_t tiles, int64_t kc) { return (int)cdiv(kc, lora_chunk(tiles, kc)); }

int64_t lora_tiles(int64_t m, int64_t n) { return cdiv(m, LT) * cdiv(n, LT); }

size_t lora_part_floats(int64_t m, int64_t n, int64_t kc) {
  const int64_t tiles = lora_tiles(m, n);
  const int S = lora_splits(tiles, kc);
  return S > 1 ? (size_t)tiles * S * LT * LT : 0;
}

namespace {

LoraProblem make_problem(const uint16_t *P, int64_t ldp, const uint16_t *Q, int64_t ldq, int64_t M, int64_t Nc,
                         int64_t Kc, float scale, void *out, float *part) {
  LoraProblem pr;
  pr.P = P;
  pr.ldp = ldp;
  pr.Q = Q;
  pr.ldq = ldq;
  pr.M = M;
  pr.Nc = Nc;
  pr.Kc = Kc;
  pr.tiles_m = cdiv(M, LT);
  const int64_t tiles = lora_tiles(M, Nc);
  pr.chunk = lora_chunk(tiles, Kc);
  pr.S = (int)cdiv(Kc, pr.chunk);
  pr.scale = scale;
  pr.out = out;
  pr.ldo = Nc;
  pr.part = part;
  return pr;
}

int64_t problem_blocks(const LoraProblem &pr) { return lora_tiles(pr.M, pr.Nc) * pr.S; }
int64_t problem_quads(const LoraProblem &pr) { return pr.S > 1 ? lora_tiles(pr.M, pr.Nc) * (LT * LT / 4) : 0; }

// Launches one product (nb == nullptr) or two of the same operand forms; the
// two must agree on the split length.  A split of exactly 512 is fetched in
// one round trip (8 steps, 147 KB of LDS: one workgroup per CU) when the
// launch fits one round of 256 workgroups; a larger launch (the two gradient
// products) fetches groups of 4 steps, two workgroups per CU, so that all of
// it is resident at once.
template <bool kAT, bool kBT, bool kBf16Out>
hipError_t launch_pair(const LoraProblem &a, const LoraProblem *nb, hipStream_t st) {
  const LoraProblem b = nb ? *nb : a;
  const int64_t wa = problem_blocks(a), wb = nb ? problem_blocks(b) : 0;
  const bool whole = a.chunk == LT * 8 && wa + wb <= 256;
  if (whole)
    lora_gemm<kAT, kBT, kBf16Out, 8><<<(unsigned)(wa + wb), 256, 0, st>>>(a, b, wa);
  else
    lora_gemm<kAT, kBT, kBf16Out, 4><<<(unsigned)(wa + wb), 256, 0, st>>>(a, b, wa);
  const int64_t qa = problem_quads(a), qb = nb ? problem_quads(b) : 0;
  if (qa + qb > 0) {
    int64_t blocks = cdiv(qa + qb, 256);
    if (blocks > 2048) blocks = 2048;
    lora_reduce<kBf16Out><<<(unsigned)blocks, 256, 0, st>>>(a, b, qa, qa + qb);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lora(LoraKind kind, const uint16_t *P, int64_t ldp, const uint16_t *Q, int64_t ldq, int64_t M,
                       int64_t Nc, int64_t Kc, float scale, void *out, float *part, hipStream_t st) {
  const LoraProblem pr = make_problem(P, ldp, Q, ldq, M, Nc, Kc, scale, out, part);
  switch (kind) {
    case LoraKind::kU:  // x A^T
      return launch_pair<false, false, true>(pr, nullptr, st);
    case LoraKind::kV:  // dy B
      return launch_pair<false, true, true>(pr, nullptr, st);
    case LoraKind::kGrad:  // v^T x, dy^T u
      return launch_pair<true, true, false>(pr, nullptr, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_lora_grads(const uint16_t *v, const uint16_t *x, const uint16_t *dy, const uint16_t *u, int64_t T,
                             int64_t N, int64_t K, int r, float scale_a, float scale_b, float *grad_A, float *grad_B,
                             float *part, size_t part_a_floats, hipStream_t st) {
  // grad_A = s_a v^T x [r x K] and grad_B = s_b dy^T u [N x r], contraction over the tokens
  const LoraProblem a = make_problem(v, r, x, K, r, K, T, scale_a, grad_A, part);
  const LoraProblem b = make_problem(dy, N, u, r, N, r, T, scale_b, grad_B, part + part_a_floats);
  if ((a.chunk == LT * 8) == (b.chunk == LT * 8)) return launch_pair<true, true, false>(a, &b, st);
  const hipError_t e = launch_pair<true, true, false>(a, nullptr, st);
  return e != hipSuccess ? e : launch_pair<true, true, false>(b, nullptr, st);
}

// Adapter products of a projection set (members i < count, ranks r each).
size_t lora_set_part_floats(int64_t T, int count, const int64_t *N, int64_t K, int r) {
  size_t v = 0, g = lora_part_floats((int64_t)count * r, K, T);
  for (int i = 0; i < count; ++i) {
    v += lora_part_floats(T, r, N[i]);
    g += lora_part_floats(N[i], r, T);
  }
  return std::max(lora_part_floats(T, (int64_t)count * r, K), std::max(v, g));
}

// Runs a list of products of one operand form, two per launch where their
// group lengths agree.
template <bool kAT, bool kBT, bool kBf16Out>
static hipError_t launch_list(const LoraProblem *pr, int n, hipStream_t st) {
  for (int i = 0; i < n;) {
    hipError_t e;
    if (i + 1 < n && (pr[i].chunk == LT * 8) == (pr[i + 1].chunk == LT * 8)) {
      e = launch_pair<kAT, kBT, kBf16Out>(pr[i], &pr[i + 1], st);
      i += 2;
    } else {
      e = launch_pair<kAT, kBT, kBf16Out>(pr[i], nullptr, st);
      i += 1;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// v_set [T x count r]: columns [i r, i r + r) = dy_i B_i.
hipError_t launch_lora_set_v(const uint16_t *const *dy, const uint16_t *const *B, const int64_t *N, int count,
                             int64_t T, int r, uint16_t *v_set, float *part, hipStream_t st) {
  LoraProblem pr[kMaxSetMembers];
  size_t off = 0;
  for (int i = 0; i < count; ++i) {
    pr[i] = make_problem(dy[i], N[i], B[i], r, T, r, N[i], 1.0f, v_set + (int64_t)i * r, part + off);
    pr[i].ldo = (int64_t)count * r;
    off += lora_part_floats(T, r, N[i]);
  }
  return launch_list<false, true, true>(pr, count, st);
}

// grad_A_set = scale v_set^T x [count r x K] and grad_B_i = scale dy_i^T u_i [N_i x r]
// (u_i = columns [i r, i r + r) of u_set).
hipError_t launch_lora_set_grads(const uint16_t *v_set, const uint16_t *x, const uint16_t *const *dy,
                                 const uint16_t *u_set, const int64_t *N, int count, int64_t T, int64_t K, int r,
                                 float scale, float *grad_A_set, float *const *grad_B, float *part, hipStream_t st) {
  LoraProblem pr[kMaxSetMembers + 1];
  const int64_t rt = (int64_t)count * r;
  pr[0] = make_problem(v_set, rt, x, K, rt, K, T, scale, grad_A_set, part);
  size_t off = lora_part_floats(rt, K, T);
  for (int i = 0; i < count; ++i) {
    pr[i + 1] = make_problem(dy[i], N[i], u_set + (int64_t)i * r, rt, N[i], r, T, scale, grad_B[i], part + off);
    off += lora_part_floats(N[i], r, T);
  }
  return launch_list<true, true, false>(pr, count + 1, st);
}

}  // namespace qlora
