// Dequant-fused bf16 MFMA GEMM of the QLoRA linear layer (gfx950).
//
// The frozen NF4 weight is decoded to BFloat16 inside the product every time
// it is used ("qlora" encyclopedia entry, tonho.wtf, section "a ideia"); the
// LoRA term s.(left factor).(right factor)^T of W' = W + s.B.A (nexusinovation
// tutorial, section "LoRA: O Padrão Ouro de Eficiência") is accumulated into
// the same fp32 tile.
//
//   out[M x Ncols] = scale * la lb^T + act . W_op           (bf16 out, fp32 acc)
//   forward : act = x  [T x n_in],  W_op = W_hat^T, Kc = n_in,  la = u, lb = B
//   grad_x  : act = dy [T x n_out], W_op = W_hat,   Kc = n_out, la = v, lb = A^T
//
// Workgroup = 8 waves on a 256 x 128 output tile, contraction step 64:
//   waves 0-3 (consumers) each own a 128 x 64 sub-tile and only read LDS and
//     issue v_mfma_f32_32x32x16_bf16;
//   waves 4-7 (producers) fetch the activation tile and the packed weight tile
//     two steps ahead into registers, decode the nibbles through the 16-entry
//     level table into bf16 (weight tile decoded once per workgroup, shared by
//     all 256 activation rows) and write the next LDS stage.
// One consumer and one producer wave share each SIMD, so the decode's vector
// ALU work issues alongside the matrix-core work.  Two LDS stages, one
// workgroup barrier per contraction step; both roles execute the same number
// of barriers.
//
// MFMA lane layouts (l = lane): A operand lane l holds A[l%32][8(l/32)..+7],
// B operand lane l holds B[8(l/32)..+7][l%32], result register q of lane l is
// D[8(q/4) + 4(l/32) + q%4][l%32].

#include "common.hpp"
#include "launch.hpp"

namespace qlora {

namespace {

constexpr int QBM = 256, QBN = 128, QBK = 64, QLD = 72;  // QLD: padded LDS row length (bf16)

__device__ __forceinline__ u32x4 ld8(const uint16_t *row, int64_t c, int64_t ncols, bool vec) {
  if (vec && c + 8 <= ncols) return *(const u32x4 *)(row + c);
  u32x4 v = {0u, 0u, 0u, 0u};
  for (int i = 0; i < 8; ++i)
    if (c + i < ncols) v[i >> 1] |= (uint32_t)row[c + i] << (16 * (i & 1));
  return v;
}

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

struct Stage {
  u32x4 a[8];   // activation: 8 rows x 8 contraction elements
  u32x4 code;   // weight codes (see Producer)
  uint32_t q[4];
  float s2[4];
};

template <bool kTransW>
struct Producer {
  const uint16_t *act;
  int64_t M, Kc, m0, c0, K, N, kblk_row;
  QWeight w;
  float mu;
  int ptid;
  bool act_vec;

  // kFull: the whole tile and every contraction step are in range and rows are
  // 16-byte aligned, so every load is unconditional (no branches, so the
  // compiler can keep two steps of loads in flight).
  template <bool kFull>
  __device__ __forceinline__ void load(int64_t kt, Stage &s) const {
    const int64_t k0 = kt * QBK;
    const int a_row = ptid >> 3, a_col = 8 * (ptid & 7);
    if (kFull) {
      const uint16_t *base = act + (m0 + a_row) * Kc + k0 + a_col;
#pragma unroll
      for (int i = 0; i < 8; ++i) s.a[i] = *(const u32x4 *)(base + (int64_t)(32 * i) * Kc);
      if (!kTransW) {
        const int64_t n = c0 + (ptid >> 1);
        s.code = *(const u32x4 *)(w.codes + n * (K / 2) + k0 / 2 + 16 * (ptid & 1));
        const int64_t blk = n * kblk_row + kt;
        s.q[0] = w.fp8[blk];
        s.s2[0] = w.s2[blk >> 8];
      } else {
        const int64_t kcol = c0 + 8 * (ptid >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t n = k0 + 4 * (ptid & 15) + i;
          s.code[i] = *(const uint32_t *)(w.codes + n * (K / 2) + kcol / 2);
          const int64_t blk = n * kblk_row + kcol / kBlock;
          s.q[i] = w.fp8[blk];
          s.s2[i] = w.s2[blk >> 8];
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t row = m0 + a_row + 32 * i;
      s.a[i] = (row < M) ? ld8(act + row * Kc, k0 + a_col, Kc, act_vec) : u32x4{0u, 0u, 0u, 0u};
    }
    if (!kTransW) {
      // one weight row (an output column), 32 consecutive contraction elements
      const int64_t n = c0 + (ptid >> 1);
      if (n < N) {
        s.code = *(const u32x4 *)(w.codes + n * (K / 2) + k0 / 2 + 16 * (ptid & 1));
        const int64_t blk = n * kblk_row + kt;
        s.q[0] = w.fp8[blk];
        s.s2[0] = w.s2[blk >> 8];
      } else {
        s.code = u32x4{0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
        s.q[0] = 0u;
        s.s2[0] = 0.f;
      }
    } else {
      // 4 consecutive weight rows (contraction) x 8 consecutive output columns;
      // the row group runs fastest across lanes so that the transposed LDS
      // writes of a wave land in consecutive banks
      const int64_t kcol = c0 + 8 * (ptid >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t n = k0 + 4 * (ptid & 15) + i;
        if (n < N && kcol < K) {
          s.code[i] = *(const uint32_t *)(w.codes + n * (K / 2) + kcol / 2);
          const int64_t blk = n * kblk_row + kcol / kBlock;
          s.q[i] = w.fp8[blk];
          s.s2[i] = w.s2[blk >> 8];
        } else {
          s.code[i] = 0x77777777u;
          s.q[i] = 0u;
          s.s2[i] = 0.f;
        }
      }
    }
  }

  // Decode one stage into LDS.  All 32 level-table reads are issued before any
  // of the arithmetic that consumes them, so their LDS latency is paid once.
  __device__ __forceinline__ void store(const Stage &s, uint16_t *sa, uint16_t *sb, const float *lut) const {
    const int a_row = ptid >> 3, a_col = 8 * (ptid & 7);
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4 *)&sa[(a_row + 32 * i) * QLD + a_col] = s.a[i];
    float lv[32];
    if (!kTransW) {
      // element e = 8 v + j of this lane's 32: nibble j of code word v
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int j = 0; j < 8; ++j) lv[8 * v + j] = lut[(s.code[v] >> (4 * j)) & 15u];
      __builtin_amdgcn_sched_barrier(0);
      // q = 0 with s2 = 0 decodes to c1hat = mu; masked rows carry the zero code, so they decode to 0
      const float ch = decode_constant(s.q[0], s.s2[0], mu);
      const int row = ptid >> 1, half = ptid & 1;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        u32x4 o;
#pragma unroll
        for (int d = 0; d < 4; ++d)
          o[d] = pack_bf16x2(decode_product(lv[8 * v + 2 * d], ch), decode_product(lv[8 * v + 2 * d + 1], ch));
        *(u32x4 *)&sb[row * QLD + 32 * half + 8 * v] = o;
      }
    } else {
      // element (row i, column c): nibble c of code word i
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) lv[8 * i + c] = lut[(s.code[i] >> (4 * c)) & 15u];
      __builtin_amdgcn_sched_barrier(0);
      float ch[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ch[i] = decode_constant(s.q[i], s.s2[i], mu);
      const int cg = ptid >> 4, rg = ptid & 15;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint2 o;
        o.x = pack_bf16x2(decode_product(lv[c], ch[0]), decode_product(lv[8 + c], ch[1]));
        o.y = pack_bf16x2(decode_product(lv[16 + c], ch[2]), decode_product(lv[24 + c], ch[3]));
        *(uint2 *)&sb[(8 * cg + c) * QLD + 4 * rg] = o;
      }
    }
  }
};

// Producer side of the pipeline: stage k+2 is fetched into registers while
// stage k+1 is decoded into LDS and the consumers multiply stage k.  Three
// register sets rotate; the loop is unrolled by three so that each set is a
// fixed group of registers.
template <bool kFull, bool kTransW>
__device__ __forceinline__ void producer_loop(const Producer<kTransW> &p, int64_t nk, uint16_t (*sa)[QBM * QLD],
                                              uint16_t (*sb)[QBN * QLD], const float *lut) {
  Stage s0, s1, s2;
  p.template load<kFull>(0, s0);
  p.template load<kFull>(min((int64_t)1, nk - 1), s1);
  __syncthreads();  // level table in LDS
  p.store(s0, sa[0], sb[0], lut);
  __syncthreads();  // stage 0 ready
  // The step body is unconditional: past the end it re-fetches the last stage
  // and writes the LDS buffer nobody reads any more, which keeps the loop free
  // of branches so that the fetch of stage k+2 stays in flight while stage k+1
  // is decoded.
#define QGEMM_PRODUCER_STEP(K_, CUR_NEXT, NEXT2)                                    \
  if ((K_) < nk) {                                                                  \
    p.template load<kFull>(min((K_) + 2, nk - 1), NEXT2);                           \
    __builtin_amdgcn_sched_barrier(0);                                              \
    p.store(CUR_NEXT, sa[((K_) + 1) & 1], sb[((K_) + 1) & 1], lut);                 \
    __syncthreads();                                                                \
  }
  for (int64_t kt = 0; kt < nk; kt += 3) {
    QGEMM_PRODUCER_STEP(kt, s1, s2)
    QGEMM_PRODUCER_STEP(kt + 1, s2, s0)
    QGEMM_PRODUCER_STEP(kt + 2, s0, s1)
  }
#undef QGEMM_PRODUCER_STEP
}

template <bool kTransW>
__global__ __launch_bounds__(512) void qgemm_ws(const uint16_t *__restrict__ act, int64_t M, int64_t Ncols,
                                                int64_t Kc, QWeight w, const uint16_t *__restrict__ la,
                                                const uint16_t *__restrict__ lb, int r, float scale,
                                                uint16_t *__restrict__ out, Codebook cb) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][QBM * QLD];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][QBN * QLD];
  __shared__ float lut[16];

  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.x * QBM, c0 = (int64_t)blockIdx.y * QBN;
  const int64_t nk = (Kc + QBK - 1) / QBK;
  const bool full = (m0 + QBM <= M) && (c0 + QBN <= Ncols) && (Kc % QBK == 0);

  if (tid >= 256) {
    // ------------------------------------------------------------ producers
    Producer<kTransW> p;
    p.act = act;
    p.M = M;
    p.Kc = Kc;
    p.m0 = m0;
    p.c0 = c0;
    p.K = w.n_in;
    p.N = w.n_out;
    p.kblk_row = w.n_in / kBlock;
    p.w = w;
    p.mu = *w.mu;
    p.ptid = tid - 256;
    p.act_vec = (Kc % 8) == 0;
    if (full)
      producer_loop<true>(p, nk, sa, sb, lut);
    else
      producer_loop<false>(p, nk, sa, sb, lut);
    return;
  }

  // -------------------------------------------------------------- consumers
  if (tid < 16) lut[tid] = cb.v[tid];
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lhi = lane >> 5;
  const bool lora_vec = (r % 8) == 0;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // LoRA term first: acc = scale * la lb^T (r zero-padded to a multiple of 16)
  for (int j0 = 0; j0 < r; j0 += 16) {
    u32x4 af[4], bf[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = m0 + wm * 128 + i * 32 + l32;
      af[i] = (row < M) ? ld8(la + row * r, j0 + 8 * lhi, r, lora_vec) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = c0 + wn * 64 + j * 32 + l32;
      if (!kTransW) {
        bf[j] = (col < Ncols) ? ld8(lb + col * r, j0 + 8 * lhi, r, lora_vec) : u32x4{0u, 0u, 0u, 0u};
      } else {
        // lb is A [r x Ncols]: gather 8 adapter rows of one column
        u32x4 v = {0u, 0u, 0u, 0u};
        for (int e = 0; e < 8; ++e) {
          const int jr = j0 + 8 * lhi + e;
          if (jr < r && col < Ncols) v[e >> 1] |= (uint32_t)lb[(int64_t)jr * Ncols + col] << (16 * (e & 1));
        }
        bf[j] = v;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma(af[i], bf[j], acc[i][j]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] *= scale;

  __syncthreads();  // level table in LDS
  __syncthreads();  // stage 0 ready

  for (int64_t kt = 0; kt < nk; ++kt) {
    const uint16_t *A = sa[kt & 1];
    const uint16_t *B = sb[kt & 1];
#pragma unroll
    for (int kk = 0; kk < QBK / 16; ++kk) {
      u32x4 af[4], bf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *(const u32x4 *)&A[(wm * 128 + i * 32 + l32) * QLD + kk * 16 + 8 * lhi];
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = *(const u32x4 *)&B[(wn * 64 + j * 32 + l32) * QLD + kk * 16 + 8 * lhi];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma(af[i], bf[j], acc[i][j]);
    }
    __syncthreads();
  }

  // epilogue: round to bf16 and store
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = c0 + wn * 64 + j * 32 + l32;
      if (col >= Ncols) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + wm * 128 + i * 32 + 8 * (q >> 2) + 4 * lhi + (q & 3);
        if (row < M) {
          __bf16 h = (__bf16)acc[i][j][q];
          out[row * Ncols + col] = __builtin_bit_cast(uint16_t, h);
        }
      }
    }
}

}  // namespace

hipError_t launch_qgemm(bool trans_w, const uint16_t *act, int64_t M, int64_t Ncols, int64_t Kc, const QWeight &w,
                        const uint16_t *la, const uint16_t *lb, int r, float scale, uint16_t *out,
                        const Codebook &cb, hipStream_t st) {
  dim3 g((unsigned)((M + QBM - 1) / QBM), (unsigned)((Ncols + QBN - 1) / QBN));
  if (trans_w)
    qgemm_ws<true><<<g, 512, 0, st>>>(act, M, Ncols, Kc, w, la, lb, r, scale, out, cb);
  else
    qgemm_ws<false><<<g, 512, 0, st>>>(act, M, Ncols, Kc, w, la, lb, r, scale, out, cb);
  return hipGetLastError();
}

}  // namespace qlora
