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
//             (with LoRA dropout the adapter term is masked element by element)
//
// Workgroup = 8 waves on a 256 x 128 output tile, contraction step 64:
//   waves 0-3 (consumers) each own a 128 x 64 sub-tile: they read LDS, issue
//     v_mfma_f32_32x32x16_bf16, and (full tiles) move the activation tile of
//     stage k+3 from global memory straight into a 3-stage LDS ring with
//     global_load_lds_dwordx4, so no register ever holds it;
//   waves 4-7 (producers) fetch the packed weight codes several steps ahead
//     into registers and decode them (the weight tile is decoded once per
//     workgroup and shared by all 256 activation rows): full tiles build each
//     block's 16 values bf16(fl32(level * constant)) as register byte tables
//     and select with v_perm_b32; partial tiles look the levels up in a
//     16-entry table in LDS and multiply.  They write the next weight stage to
//     LDS; for partial tiles they also carry the activation tile, masked,
//     through registers.
// One consumer and one producer wave share each SIMD, so the decode's vector
// ALU work issues alongside the matrix-core work.  One workgroup barrier per
// contraction step; both roles execute the same number of barriers.  The DMA
// is kept in the consumer waves because a wave that has issued LDS-DMA gets
// conservative full waits on every later use of a loaded register.
//
// MFMA lane layouts (l = lane): A operand lane l holds A[l%32][8(l/32)..+7],
// B operand lane l holds B[8(l/32)..+7][l%32], result register q of lane l is
// D[8(q/4) + 4(l/32) + q%4][l%32].

#include "common.hpp"
#include "launch.hpp"

namespace qlora {

namespace {

constexpr int QBM = 256, QBN = 128, QBK = 64;
// Weight tile in LDS, always with the weight's own contiguous axis (n_in)
// along LDS rows: forward 128 weight rows x 64 (row length QLD), grad_x 64
// weight rows x 128 (row length TLD).  Both are padded for conflict-free
// fragment reads.
constexpr int QLD = 72, TLD = 144;
static_assert(128 * QLD == 64 * TLD, "both weight-tile layouts fill the same LDS stage");
constexpr int kActStages = 3;                            // activation tile LDS ring
constexpr int kWStages = 3;                              // weight tile LDS ring

typedef __attribute__((address_space(1))) const void gptr_t;
typedef __attribute__((address_space(3))) void lptr_t;

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

// Activation tile in LDS: 256 rows of 64 bf16 (128 B, eight 16-byte chunks),
// unpadded; chunk c of row r sits at position c ^ ((r >> 1) & 7).  The LDS
// serves the 16-byte reads of 16 lanes at a time from 64 four-byte banks
// (256 B), i.e. two consecutive rows; under this swizzle the 16 rows of one
// fragment read fill the 64 banks exactly once.
__device__ __forceinline__ int act_off(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3); }

// Workgroup barrier without the memory fences of __syncthreads(): those would
// wait for every outstanding load, including the LDS-DMA of stages that are
// deliberately still in flight.  Each caller first waits for exactly what the
// other waves need (s_waitcnt), and the empty asm statements keep the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4 (left at its maximum), lgkmcnt in 11:8.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | ((vm >> 4) << 14); }

// One 16-byte-per-lane LDS-DMA: lane l reads 16 bytes at sbase + voff and
// writes them at LDS byte address lds + 16 l.  Written as inline asm so that
// the compiler does not treat the whole LDS as possibly being written by it:
// the builtin makes every later LDS read of the wave wait for all outstanding
// loads, including stages that are meant to stay in flight.  The instruction
// has no register result; its waits are issued explicitly by the caller, and
// voff must stay unmodified until they have been.
// m0 is named as clobbered: nothing else in these kernels uses it (checked in
// the generated code), and every DMA sets it right before use.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const char *sbase, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// The value held by the other lane of an adjacent pair (DPP quad_perm [1, 0, 3, 2]).
__device__ __forceinline__ uint32_t pair_swap(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)(lptr_t *)p; }

// Full tiles: consumer wave cw (0..3) moves rows [64 cw, 64 cw + 64) of the
// activation tile of stage kt into LDS buffer dst with 8 DMA instructions of 8
// rows each (lane l writes the 16 bytes at dst + 16 l: row 8 j + l/8 of the
// range, the chunk whose swizzled position is l % 8).  The swizzle of those
// rows depends on the parity of j only, so the per-lane byte offset takes two
// loop-invariant values (lane_off[j & 1]) and everything else is scalar.
__device__ __forceinline__ uint32_t dma_lane_offset(int lane, int64_t Kc, int parity) {
  const int row = lane >> 3, pos = lane & 7;
  const int chunk = pos ^ (4 * parity + (row >> 1));  // ((8 j + row) >> 1) & 7 for j of this parity
  return (uint32_t)((row * Kc + 8 * chunk) * 2);
}

// The activation DMA of one consumer wave cw: rows [64 cw, 64 cw + 64) of the
// tile, DMA j moving rows 8 j .. 8 j + 7 of them.  kClamp (a launch whose token
// count is not a multiple of QBM): lane rows at or past the tile's last valid
// row read that row instead, so every address stays inside the activation and
// the full-tile pipeline runs for any number of rows; the epilogue never
// stores those rows.  Without kClamp the per-lane offset takes the two
// loop-invariant values above; with it the offset is formed per DMA from the
// lane's row (three vector instructions).
template <bool kClamp>
struct ActDma {
  const char *base;   // kClamp: element (m0, first step) of the activation; else that of row m0 + 64 cw
  int64_t row_bytes;  // 2 Kc
  uint32_t off[2];    // !kClamp: lane offsets by the parity of j
  int lane_row, pos, last_row;  // kClamp: tile row of the lane at j = 0, its chunk slot, last valid row

  // Every input but the lane is wave-uniform.  The base goes through readfirstlane once here, so it
  // stays in scalar registers also where the object is set up under a branch on the wave index
  // (each half through uint32_t: readfirstlane returns a signed int, which must not be
  // sign-extended into the other half).
  __device__ __forceinline__ void init(const uint16_t *act, int64_t Kc, int64_t M, int64_t m0, int64_t kstep0,
                                       int cw, int lane) {
    row_bytes = 2 * Kc;
    const char *b = (const char *)(act + m0 * Kc + kstep0 * QBK);
    if (!kClamp) {
      b += 64 * cw * row_bytes;
      off[0] = dma_lane_offset(lane, Kc, 0);
      off[1] = dma_lane_offset(lane, Kc, 1);
    } else {
      lane_row = 64 * cw + (lane >> 3);
      pos = lane & 7;
      last_row = (int)min((int64_t)QBM, M - m0) - 1;
    }
    const uint64_t u = (uint64_t)(uintptr_t)b;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    base = (const char *)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
  }

  // DMAs j0 .. j0 + nj - 1 of stage kt into dst (this wave's 64 rows of an LDS stage)
  __device__ __forceinline__ void issue(int64_t kt, uint16_t *dst, int j0 = 0, int nj = 8) const {
    const uint32_t l0 = lds_addr(dst);
    const char *sb = base + kt * (QBK * 2);
#pragma unroll
    for (int j = j0; j < j0 + nj; ++j) {
      if (!kClamp) {
        dma16(sb + (int64_t)(8 * j) * row_bytes, off[j & 1], l0 + 8 * j * 64 * 2);
      } else {
        const int row = lane_row + 8 * j;
        const int chunk = pos ^ ((row >> 1) & 7);
        dma16(sb, (uint32_t)min(row, last_row) * (uint32_t)row_bytes + 16u * (uint32_t)chunk, l0 + 8 * j * 64 * 2);
      }
    }
  }

  // every DMA of this wave has landed; the offsets a DMA reads stay untouched until then
  __device__ __forceinline__ void wait_all() const {
    if (!kClamp)
      asm volatile("s_waitcnt vmcnt(0)" ::"v"(off[0]), "v"(off[1]) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::"v"(lane_row), "v"(pos) : "memory");
  }
};

// One stage of a producer lane: its 32 weight codes (one weight row, 32
// consecutive n_in positions) with the block's FP8 constant and group scale,
// and for partial tiles its share of the activation tile.
struct Stage {
  u32x4 a[8];  // activation (register path only): 8 rows x 8 contraction elements
  u32x4 code;
  uint32_t q;
  float s2;
};

// The 32 levels of a stage's codes and its block constant (partial tiles).
struct Levels {
  float lv[32];
  float ch;
};

// kDQ: the block constants are FP8 codes with group scales and a tensor mean
// (double quantization); otherwise w.s2 holds one fp32 constant per block.
template <bool kTransW, bool kDQ>
struct Producer {
  const uint16_t *act;
  int64_t M, Kc, m0, c0, K, N, kblk_row;
  QWeight w;
  float mu;
  int ptid;
  bool act_vec;
  int64_t kstep0;  // first contraction step of this workgroup's split

  // Partial tiles: the activation tile goes through registers with masking.
  __device__ __forceinline__ void load_act(int64_t kt, Stage &s) const {
    const int64_t k0 = (kstep0 + kt) * QBK;
    const int a_row = ptid >> 3, a_col = 8 * (ptid & 7);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t row = m0 + a_row + 32 * i;
      s.a[i] = (row < M) ? ld8(act + row * Kc, k0 + a_col, Kc, act_vec) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  __device__ __forceinline__ void store_act(const Stage &s, uint16_t *dst) const {
    const int a_row = ptid >> 3, chunk = ptid & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4 *)&dst[act_off(a_row + 32 * i, chunk)] = s.a[i];
  }

  // Packed weight codes, FP8 constant and group scale of stage kt.  Each lane
  // owns one weight row and 32 consecutive n_in positions (half an NF4 block):
  //   forward: weight rows c0 .. c0+127 (2 lanes a row), n_in = k0 .. k0+63
  //   grad_x : weight rows k0 .. k0+63 (4 lanes a row), n_in = c0 .. c0+127
  // Full tiles address them from the lane's stage-0 position plus a per-stage
  // stride (code_step bytes, blk_step blocks).
  const uint8_t *code0;
  int64_t code_step, blk0, blk_step;

  __device__ __forceinline__ void init_addressing() {
    const int64_t n = kTransW ? (ptid >> 2) : c0 + (ptid >> 1);
    const int64_t col = kTransW ? c0 + 32 * (ptid & 3) : 32 * (ptid & 1);
    code_step = kTransW ? QBK * (K / 2) : QBK / 2;
    blk_step = kTransW ? QBK * kblk_row : 1;
    code0 = w.codes + n * (K / 2) + col / 2 + kstep0 * code_step;
    blk0 = n * kblk_row + col / kBlock + kstep0 * blk_step;
  }

  template <bool kFull>
  __device__ __forceinline__ void load_w(int64_t kt, Stage &s) const {
    if (kFull) {
      s.code = *(const u32x4 *)(code0 + kt * code_step);
      const int64_t blk = blk0 + kt * blk_step;
      if (kDQ) {
        s.q = w.fp8[blk];
        s.s2 = w.s2[blk >> 8];
      } else {
        s.q = 0u;
        s.s2 = w.s2[blk];
      }
      return;
    }
    const int64_t k0 = (kstep0 + kt) * QBK;
    const int64_t n = kTransW ? k0 + (ptid >> 2) : c0 + (ptid >> 1);
    const int64_t col = kTransW ? c0 + 32 * (ptid & 3) : k0 + 32 * (ptid & 1);
    if (n < N && col < K) {
      s.code = *(const u32x4 *)(w.codes + n * (K / 2) + col / 2);
      const int64_t blk = n * kblk_row + col / kBlock;
      if (kDQ) {
        s.q = w.fp8[blk];
        s.s2 = w.s2[blk >> 8];
      } else {
        s.q = 0u;
        s.s2 = w.s2[blk];
      }
    } else {
      s.code = u32x4{0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
      s.q = 0u;
      s.s2 = 0.f;
    }
  }

  // Partial tiles: the levels of a stage's 32 codes from the 16-entry table
  // in LDS, and its block constant.  Each byte of the masked words (c << 2) & 0x3C3C3C3C and
  // (c >> 2) & 0x3C3C3C3C is four times a code (even and odd elements), i.e.
  // the byte offset of its level, so one extract per code forms its address.
  __device__ __forceinline__ void read_levels(const Stage &s, const float *lut, Levels &L) const {
    const char *base = (const char *)lut;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      uint32_t ev = (s.code[v] << 2) & 0x3C3C3C3Cu, od = (s.code[v] >> 2) & 0x3C3C3C3Cu;
      // opaque to the optimizer, which would otherwise rebuild a shift and a mask per code
      asm("" : "+v"(ev), "+v"(od));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        L.lv[8 * v + 2 * k] = *(const float *)(base + __builtin_amdgcn_ubfe(ev, 8 * k, 8));
        L.lv[8 * v + 2 * k + 1] = *(const float *)(base + __builtin_amdgcn_ubfe(od, 8 * k, 8));
      }
    }
    // q = 0 with s2 = 0 decodes to c1hat = mu; masked rows carry the zero code, so they decode to 0
    L.ch = kDQ ? decode_constant(s.q, s.s2, mu) : s.s2;
  }

  // Full tiles: the decoded stage straight from its codes into LDS, with no
  // table in memory: the block's 16 decoded values are held in registers as
  // byte tables and each code selects its bf16 value with v_perm_b32
  // (decode_word; bit-identical to the product form).  The two lanes of an
  // adjacent pair decode the two halves of one block, so they share its
  // tables: each builds those of 8 levels (the odd lane levels 8..15) and
  // takes the other 8 from its partner with a DPP swap.  A lane's tables
  // thus list its own levels first, and the odd lane's codes select with
  // bit 3 flipped.  Four 16-byte stores.
  __device__ __forceinline__ void write_rt(const Stage &s, const Codebook &cb, uint16_t *sb) const {
    const float ch = kDQ ? decode_constant(s.q, s.s2, mu) : s.s2;
    const bool odd = ptid & 1;
    uint32_t p[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float l0 = odd ? cb.v[8 + 2 * m] : cb.v[2 * m], l1 = odd ? cb.v[9 + 2 * m] : cb.v[2 * m + 1];
      p[m] = pack_bf16x2(decode_product(l0, ch), decode_product(l1, ch));
    }
    DecodeTable t;
    uint32_t lo[2], hi[2];
    table_half(p, lo, hi);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      t.lo[j] = lo[j];
      t.hi[j] = hi[j];
      t.lo[2 + j] = pair_swap(lo[j]);
      t.hi[2 + j] = pair_swap(hi[j]);
    }
    const uint32_t flip = odd ? 0x88888888u : 0u;
    uint16_t *dst = kTransW ? &sb[(ptid >> 2) * TLD + 32 * (ptid & 3)] : &sb[(ptid >> 1) * QLD + 32 * (ptid & 1)];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      uint32_t o[4];
      decode_word(s.code[v] ^ flip, t, o);
      *(u32x4 *)&dst[8 * v] = u32x4{o[0], o[1], o[2], o[3]};
    }
  }

  // Partial tiles: the decoded stage into LDS, fl32 products rounded to bf16,
  // 16-byte stores.
  __device__ __forceinline__ void store_w(const Levels &L, uint16_t *sb) const {
    uint16_t *dst = kTransW ? &sb[(ptid >> 2) * TLD + 32 * (ptid & 3)] : &sb[(ptid >> 1) * QLD + 32 * (ptid & 1)];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        o[d] = pack_bf16x2(decode_product(L.lv[8 * v + 2 * d], L.ch), decode_product(L.lv[8 * v + 2 * d + 1], L.ch));
      *(u32x4 *)&dst[8 * v] = o;
    }
  }
};

// Producer side of the pipeline: at step k the consumers multiply stage k
// (from registers) and read stage k+1 from LDS, while the producers write
// stage k+2 into the buffers of stage k (read during step k-1).  Stages 0 and
// 1 are written before the loop, each followed by a barrier.  Past the end the
// last stage is repeated, into buffers nobody reads.  The loops are unrolled
// over their register sets with no conditions inside, so each set keeps fixed
// registers.
//
// Full tiles: at step k the producers decode stage k+2 from its codes (fetched
// three steps earlier) into LDS, then fetch the codes of stage k+5 into the
// same registers.  Code sets rotate by three (unrolled by three).  The caller
// fetches the codes of stages 0, 1 and 2 (fetch_first_codes), so that their
// latency can overlap other work.  The decode reads no memory: with the level
// table in LDS the producers' level reads (32 KB per step) competed with the
// consumers' fragment reads.
template <bool kTransW, bool kDQ>
__device__ __forceinline__ void fetch_first_codes(const Producer<kTransW, kDQ> &p, int64_t nk, Stage &c0, Stage &c1,
                                                  Stage &c2) {
  p.template load_w<true>(0, c0);
  p.template load_w<true>(min((int64_t)1, nk - 1), c1);
  p.template load_w<true>(min((int64_t)2, nk - 1), c2);
}

template <bool kTransW, bool kDQ>
__device__ __forceinline__ void producer_loop_full(const Producer<kTransW, kDQ> &p, int64_t nk, uint16_t (*sb)[QBN * QLD],
                                                   Stage &c0, Stage &c1, Stage &c2, const Codebook &cb) {
  auto st = [nk](int64_t k) { return min(k, nk - 1); };
  p.write_rt(c0, cb, sb[0]);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  wg_barrier();  // stage 0 ready
  p.write_rt(c1, cb, sb[1]);
  p.template load_w<true>(st(3), c0);
  p.template load_w<true>(st(4), c1);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  wg_barrier();  // stage 1 ready
#define QGEMM_PRODUCER_STEP(K_, CUR, BUF)                                              \
  if ((K_) < nk) {                                                                    \
    p.write_rt(CUR, cb, sb[BUF]);                                                     \
    __builtin_amdgcn_sched_barrier(0);                                                \
    p.template load_w<true>(st((K_) + 5), CUR);                                       \
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));                                   \
    wg_barrier();                                                                     \
  }
  int64_t kt = 0;
  for (; kt + 3 <= nk; kt += 3) {
    QGEMM_PRODUCER_STEP(kt, c2, 2)
    QGEMM_PRODUCER_STEP(kt + 1, c0, 0)
    QGEMM_PRODUCER_STEP(kt + 2, c1, 1)
  }
  QGEMM_PRODUCER_STEP(kt, c2, 2)
  QGEMM_PRODUCER_STEP(kt + 1, c0, 0)
#undef QGEMM_PRODUCER_STEP
}

// Partial tiles: the activation tile rides along with the codes, masked; at
// step k the producers read the levels of stage k+2 and write it (codes and
// activation fetched two steps earlier), then fetch stage k+4.  Sets rotate
// by three (unrolled by three).
template <bool kTransW, bool kDQ>
__device__ __forceinline__ void producer_loop_partial(const Producer<kTransW, kDQ> &p, int64_t nk,
                                                      uint16_t (*sa)[QBM * 64], uint16_t (*sb)[QBN * QLD],
                                                      const float *lut) {
  auto st = [nk](int64_t k) { return min(k, nk - 1); };
  Stage c0, c1, c2;
  Levels l;
  auto load = [&](int64_t k, Stage &c) {
    p.load_act(k, c);
    p.template load_w<false>(k, c);
  };
  auto store = [&](const Stage &c, int64_t k) {
    p.read_levels(c, lut, l);
    p.store_act(c, sa[k % kActStages]);
    p.store_w(l, sb[k % kWStages]);
  };
  load(0, c0);
  load(st(1), c1);
  load(st(2), c2);
  store(c0, 0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  wg_barrier();  // stage 0 ready
  store(c1, 1);
  load(st(3), c0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  wg_barrier();  // stage 1 ready
#define QGEMM_PRODUCER_STEP(K_, CSTORE, CLOAD)                                        \
  if ((K_) < nk) {                                                                    \
    store(CSTORE, (K_) + 2);                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                \
    load(st((K_) + 4), CLOAD);                                                        \
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));                                   \
    wg_barrier();                                                                     \
  }
  int64_t kt = 0;
  for (; kt + 3 <= nk; kt += 3) {
    QGEMM_PRODUCER_STEP(kt, c2, c1)
    QGEMM_PRODUCER_STEP(kt + 1, c0, c2)
    QGEMM_PRODUCER_STEP(kt + 2, c1, c0)
  }
  QGEMM_PRODUCER_STEP(kt, c2, c1)
  QGEMM_PRODUCER_STEP(kt + 1, c0, c2)
#undef QGEMM_PRODUCER_STEP
}

// The four 16-wide contraction slices of one stage for a consumer wave's
// 128 x 64 sub-tile: fragments of slice kk+1 are read while slice kk
// multiplies.
struct NoHook {
  __device__ __forceinline__ void operator()(int) const {}
};

template <bool kTransW, typename Hook = NoHook>
__device__ __forceinline__ void consumer_slices(const uint16_t *A, const uint16_t *B, int wm, int wn, int lane,
                                                f32x16 (&acc)[4][2], const Hook &hook = Hook()) {
  const int l32 = lane & 31, lhi = lane >> 5;
  u32x4 af[2][4], bf[2][2];
  auto load_frags = [&](int kk, u32x4 (&a)[4], u32x4 (&b)[2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *(const u32x4 *)&A[act_off(wm * 128 + i * 32 + l32, 2 * kk + lhi)];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (!kTransW) {
        b[j] = *(const u32x4 *)&B[(wn * 64 + j * 32 + l32) * QLD + kk * 16 + 8 * lhi];
      } else {
        // LDS transpose read (16-lane groups): source lane s of group g
        // points at weight row 16 kk + 8 (g/2) + s/4 (+4), n_in column
        // 16 (g%2) + 4 (s%4) of this 32-column sub-tile; lane l then holds
        // 4 consecutive weight rows of column l%32.
        const int sl = lane & 15, g = lane >> 4;
        const int nrow = 16 * kk + 8 * (g >> 1) + (sl >> 2);
        const int ncol = wn * 64 + j * 32 + 16 * (g & 1) + 4 * (sl & 3);
        typedef short v4s __attribute__((ext_vector_type(4)));
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (v4s __attribute__((address_space(3))) *)(lptr_t *)&B[nrow * TLD + ncol]);
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (v4s __attribute__((address_space(3))) *)(lptr_t *)&B[(nrow + 4) * TLD + ncol]);
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        b[j] = u32x4{l2.x, l2.y, h2.x, h2.y};
      }
    }
  };
  load_frags(0, af[0], bf[0]);
#pragma unroll
  for (int kk = 0; kk < QBK / 16; ++kk) {
    if (kk + 1 < QBK / 16) load_frags(kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
    hook(kk);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma(af[kk & 1][i], bf[kk & 1][j], acc[i][j]);
  }
}

// Fragments of slice kk of one stage for a consumer wave's 128 x 64
// sub-tile (the same addressing as consumer_slices).
struct StageFrags {
  u32x4 a[QBK / 16][4], b[QBK / 16][2];
};

__device__ __forceinline__ u32x4 load_a_frag(const uint16_t *A, int wm, int lane, int kk, int i) {
  return *(const u32x4 *)&A[act_off(wm * 128 + i * 32 + (lane & 31), 2 * kk + (lane >> 5))];
}

template <bool kTransW>
__device__ __forceinline__ u32x4 load_b_frag(const uint16_t *B, int wn, int lane, int kk, int j) {
  if (!kTransW) return *(const u32x4 *)&B[(wn * 64 + j * 32 + (lane & 31)) * QLD + kk * 16 + 8 * (lane >> 5)];
  const int sl = lane & 15, g = lane >> 4;
  const int nrow = 16 * kk + 8 * (g >> 1) + (sl >> 2);
  const int ncol = wn * 64 + j * 32 + 16 * (g & 1) + 4 * (sl & 3);
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (v4s __attribute__((address_space(3))) *)(lptr_t *)&B[nrow * TLD + ncol]);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (v4s __attribute__((address_space(3))) *)(lptr_t *)&B[(nrow + 4) * TLD + ncol]);
  const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
  return u32x4{l2.x, l2.y, h2.x, h2.y};
}

// LoRA term of the output tile, staged through LDS in the same layouts as the
// main contraction (one 64-wide chunk of the rank r at a time, zero past r):
// the left factor la [M x r] (row stride ld_la) as an activation tile, the right factor as a
// weight tile (forward: lb = B [Ncols x r], rows = output columns; grad_x:
// lb = A [r x Ncols], rows = the rank).  All 512 threads stage with 16-byte
// loads where the rank allows it, every load of a chunk issued before the
// first LDS store (one memory round trip per chunk).
template <bool kTransW>
__device__ __forceinline__ void stage_lora(const uint16_t *la, int64_t ld_la, const uint16_t *lb, int r, int j0, int64_t M,
                                           int64_t Ncols, int64_t m0, int64_t c0, int tid, uint16_t *sa_dst,
                                           uint16_t *sb_dst) {
  const bool vec = (r % 8) == 0 && (ld_la % 8) == 0;
  constexpr int kA = QBM * 8 / 512, kB = 2;  // per thread: 256 rows x 8 chunks; 1024 chunks of the right factor
  u32x4 va[kA], vb[kB];
#pragma unroll
  for (int it = 0; it < kA; ++it) {
    const int idx = tid + 512 * it, row = idx >> 3, ch = idx & 7;
    const int64_t grow = m0 + row;
    va[it] = grow < M ? ld8(la + grow * ld_la, j0 + 8 * ch, r, vec) : u32x4{0u, 0u, 0u, 0u};
  }
  if (!kTransW) {
#pragma unroll
    for (int it = 0; it < kB; ++it) {  // 128 output columns x 8 chunks of the rank
      const int idx = tid + 512 * it, row = idx >> 3, ch = idx & 7;
      const int64_t col = c0 + row;
      vb[it] = col < Ncols ? ld8(lb + col * r, j0 + 8 * ch, r, vec) : u32x4{0u, 0u, 0u, 0u};
    }
  } else {
    const bool cvec = (Ncols % 8) == 0;
#pragma unroll
    for (int it = 0; it < kB; ++it) {  // 64 rank rows x 16 chunks of 8 columns
      const int idx = tid + 512 * it, jr = idx >> 4, ch = idx & 15;
      const int j = j0 + jr;
      vb[it] = j < r ? ld8(lb + (int64_t)j * Ncols, c0 + 8 * ch, Ncols, cvec) : u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int it = 0; it < kA; ++it) {
    const int idx = tid + 512 * it;
    *(u32x4 *)&sa_dst[act_off(idx >> 3, idx & 7)] = va[it];
  }
#pragma unroll
  for (int it = 0; it < kB; ++it) {
    const int idx = tid + 512 * it;
    if (!kTransW)
      *(u32x4 *)&sb_dst[(idx >> 3) * QLD + 8 * (idx & 7)] = vb[it];
    else
      *(u32x4 *)&sb_dst[(idx >> 4) * TLD + 8 * (idx & 15)] = vb[it];
  }
}

// The producer state of member mi of a set (mu: the member's tensor mean,
// loaded by the caller; ptid: the lane's index among the 256 decoding lanes).
template <bool kTransW, bool kDQ>
__device__ __forceinline__ Producer<kTransW, kDQ> member_producer(const QgemmMember &mm, const uint16_t *x, int64_t M,
                                                                  int64_t m0, int64_t c0, int ptid, float mu,
                                                                  int64_t kstep0) {
  Producer<kTransW, kDQ> p;
  const int64_t Kc = kTransW ? mm.w.n_out : mm.w.n_in;
  p.act = kTransW ? mm.act : x;
  p.M = M;
  p.Kc = Kc;
  p.m0 = m0;
  p.c0 = c0;
  p.K = mm.w.n_in;
  p.N = mm.w.n_out;
  p.kblk_row = mm.w.n_in / kBlock;
  p.w = mm.w;
  p.mu = mu;
  p.ptid = ptid;
  p.act_vec = (Kc % 8) == 0;
  p.kstep0 = kstep0;
  p.init_addressing();
  return p;
}

__device__ __forceinline__ QgemmMember set_member(const QgemmSet &s, int i) {
  return i == 0 ? s.m[0] : i == 1 ? s.m[1] : i == 2 ? s.m[2] : s.m[3];
}

// One launch covers a projection set (members sharing n_in; one member for a
// single linear):
//   forward: the grid's column tiles run over the members in order; tile y
//     belongs to the last member whose tile0 <= y: out = its y, act = x, the
//     weight is its W, la = columns [i r, i r + r) of u_set (row stride
//     set.ld_la), lb = its B, r = the member rank.
//   grad_x : every tile contracts over all members in order (the sum over the
//     set), one pipeline run per member: act = its dy, the weight is its W;
//     the adapter term uses la = v_set, lb = A_set and r = the set's total
//     rank; out = grad_x.
// kDrop (grad_x only): the adapter term is masked by the LoRA dropout words.
// kFull: every tile of the grid is full in columns and contraction steps, and
// in rows unless kClamp; the partial-tile path is not compiled in.
// kClamp (with kFull only): M is not a multiple of QBM; the last row tile's
// missing rows read a valid row (ActDma) and are never stored, so it runs the
// full-tile pipeline.
// Split contraction (part != nullptr): workgroup z of the grid's third
// dimension contracts steps [z split_steps, (z + 1) split_steps) of every
// member and writes its fp32 tile to part[z][M][set.part_cols] (forward: a
// member's column c at column 128 tile0 + c); split 0 also carries the adapter
// term; qgemm_split_reduce adds the splits in order.
template <bool kTransW, bool kDQ, bool kDrop, bool kClamp, bool kFull>
__global__ __launch_bounds__(512) void qgemm_ws(QgemmSet set, int64_t M, const uint16_t *__restrict__ x,
                                                const uint16_t *__restrict__ la, const uint16_t *__restrict__ lb,
                                                int r, float scale, uint16_t *__restrict__ gx, Codebook cb,
                                                const uint32_t *__restrict__ keep, float *__restrict__ part,
                                                int64_t split_steps) {
  static_assert(kFull || !kClamp, "clamped rows only on grids of full tiles");
  __shared__ __attribute__((aligned(16))) uint16_t sa[kActStages][QBM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sb[kWStages][QBN * QLD];  // = 64 * TLD
  __shared__ float lut[16];

  const int tid = threadIdx.x;
  // Tile of this workgroup.  Workgroups go to the 8 XCDs round robin by linear
  // id, and each XCD has its own L2.  When the grid allows it, XCD k takes a
  // block of R/4 row tiles x C/2 column tiles (rows fastest, so the row tiles
  // that share a weight tile run together): each activation row tile is then
  // read by 2 XCDs and each weight tile by 4, against 1 and 8 for the plain
  // order (whose weight re-reads dominate the traffic).
  int64_t bx = blockIdx.x, by = blockIdx.y;
  {
    const int64_t R = gridDim.x, C = gridDim.y;
    if (R % 4 == 0 && C % 2 == 0) {
      const int64_t id = bx + by * R, xcd = id % 8, slot = id / 8, rb = R / 4;
      bx = (xcd / 2) * rb + slot % rb;
      by = (xcd % 2) * (C / 2) + slot / rb;
    }
  }
  const int64_t m0 = bx * QBM;
  int mf = 0;  // forward: the member of this column tile
  if (!kTransW)
    for (int i = 1; i < set.count; ++i)
      if (by >= set_member(set, i).tile0) mf = i;
  const QgemmMember fm = set_member(set, mf);
  const int64_t Ncols = kTransW ? set.m[0].w.n_in : fm.w.n_out;
  const int64_t c0 = (by - (kTransW ? 0 : fm.tile0)) * QBN;
  const uint16_t *la_t = kTransW ? la : la + (int64_t)mf * r;
  const uint16_t *lb_t = kTransW ? lb : fm.lb;
  uint16_t *out = kTransW ? gx : fm.out;
  const int m_begin = kTransW ? 0 : mf, m_end = kTransW ? set.count : mf + 1;
  // full (per member): every column and contraction step of the tile is in
  // range (and, without kClamp, every row)
  const bool rows_ok = kFull || m0 + QBM <= M;
  // this workgroup's contraction steps (a split, or all of them) and its rank
  // of the adapter term (only split 0 adds it)
  const int64_t kstep0 = part ? (int64_t)blockIdx.z * split_steps : 0;
  const int r_eff = blockIdx.z == 0 ? r : 0;
  auto member_steps = [&](int64_t Kc) {
    const int64_t nk = (Kc + QBK - 1) / QBK;
    return part ? min(split_steps, nk - kstep0) : nk;
  };

  // Level table for the producers' decode of partial tiles.
  if (!kFull) {
    if (tid < 16) lut[tid] = cb.v[tid];
    __syncthreads();
  }

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lhi = lane >> 5;
  const int cw = __builtin_amdgcn_readfirstlane(wave);  // consumer wave: DMA rows [64 cw, 64 cw + 64)

  // The pipeline's first memory accesses go out before the LoRA term, so that
  // their latency overlaps its staging: for full tiles of the first member the
  // producers fetch the codes of stages 0-2 and the consumers start the
  // activation DMA of stages 0 and 1 (stage 2's buffer still holds the LoRA
  // staging).
  const QgemmMember m_first = set_member(set, m_begin);
  const int64_t Kc_first = kTransW ? m_first.w.n_out : m_first.w.n_in;
  const int64_t nk_first = member_steps(Kc_first);
  const bool full_first = kFull || (rows_ok && (c0 + QBN <= Ncols) && (Kc_first % QBK == 0));
  Stage pre0, pre1, pre2;
  ActDma<kClamp> dma_first;
  // every member's tensor mean, fetched with the first codes
  float mu0 = 0.f, mu1 = 0.f, mu2 = 0.f, mu3 = 0.f;
  if (tid >= 256) {
    if (kDQ) {
      mu0 = *set_member(set, m_begin).w.mu;
      if (m_begin + 1 < m_end) mu1 = *set_member(set, m_begin + 1).w.mu;
      if (m_begin + 2 < m_end) mu2 = *set_member(set, m_begin + 2).w.mu;
      if (m_begin + 3 < m_end) mu3 = *set_member(set, m_begin + 3).w.mu;
    }
    if (full_first)
      fetch_first_codes(member_producer<kTransW, kDQ>(m_first, x, M, m0, c0, tid - 256, 0.f, kstep0), nk_first, pre0, pre1,
                        pre2);
  } else if (full_first) {
    const uint16_t *act = kTransW ? m_first.act : x;
    dma_first.init(act, Kc_first, M, m0, kstep0, cw, lane);
    dma_first.issue(0, sa[0] + 64 * cw * 64);
    dma_first.issue(min((int64_t)1, nk_first - 1), sa[1] + 64 * cw * 64);
  }

  // LoRA term first, scaled: acc = scale * la lb^T, staged chunk by chunk in
  // activation stage 2 and weight stage 1; the consumer waves multiply,
  // everyone stages.  The producers skip the last chunk's closing barrier:
  // while the consumers multiply it they decode stage 0 into weight stage 0,
  // and their "stage 0 ready" barrier pairs with the consumers' closing one
  // (which the consumers' first member then does not repeat), so the stage 1
  // writes into weight stage 1 start only after the LoRA term is read.
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  for (int j0 = 0; j0 < r_eff; j0 += QBK) {
    stage_lora<kTransW>(la_t, set.ld_la, lb_t, r, j0, M, Ncols, m0, c0, tid, sa[2], sb[1]);
    // every wave's early DMA of stages 0 and 1 has landed before the barrier
    // (the staging's loads, issued after them, have returned already); naming
    // the lane offsets keeps their registers untouched until then
    if (tid < 256) dma_first.wait_all();
    __syncthreads();
    if (tid < 256) {
      consumer_slices<kTransW>(sa[2], sb[1], wm, wn, lane, acc);
      __syncthreads();
    } else if (j0 + QBK < r_eff) {
      __syncthreads();
    }
  }
  // no adapter term (a split past the first): the early DMA has landed before
  // the consumers' "stage 0 ready" barrier below
  if (r_eff == 0 && tid < 256) dma_first.wait_all();
  if (tid < 256) {
    if (kTransW && kDrop) {
      // LoRA dropout (grad_x): the adapter term of (row, column) is kept where
      // bit row % 32 of word [row / 32][column] is set.  The 16 accumulators
      // of a lane in a 32 x 32 sub-tile share one column and one 32-row block.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t rb = m0 + wm * 128 + i * 32;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t col = c0 + wn * 64 + j * 32 + l32;
          const uint32_t kw = (rb < M && col < Ncols) ? keep[(rb >> 5) * Ncols + col] : 0u;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int bit = 8 * (q >> 2) + 4 * lhi + (q & 3);
            acc[i][j][q] = ((kw >> bit) & 1u) ? acc[i][j][q] * scale : 0.f;
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[i][j][q] *= scale;
    }
  }

  if (tid >= 256) {
    // ------------------------------------------------------------ producers
    for (int mi = m_begin; mi < m_end; ++mi) {
      const QgemmMember mm = set_member(set, mi);
      const int64_t Kc = kTransW ? mm.w.n_out : mm.w.n_in;
      const int64_t nk = member_steps(Kc);
      const bool full = kFull || (rows_ok && (c0 + QBN <= Ncols) && (Kc % QBK == 0));
      if (mi > m_begin) wg_barrier();  // the previous member's pipeline has drained
      const int mo = mi - m_begin;
      const float mu = mo == 0 ? mu0 : mo == 1 ? mu1 : mo == 2 ? mu2 : mu3;
      const Producer<kTransW, kDQ> p = member_producer<kTransW, kDQ>(mm, x, M, m0, c0, tid - 256, mu, kstep0);
      if (full) {
        if (mi > m_begin) fetch_first_codes(p, nk, pre0, pre1, pre2);  // the first member's went out early
        producer_loop_full(p, nk, sb, pre0, pre1, pre2, cb);
      } else if (!kFull) {
        producer_loop_partial(p, nk, sa, sb, lut);
      }
    }
    return;
  }

  // -------------------------------------------------------------- consumers
  // full tiles: stages 0, 1 and 2 of the activation ring (the first member's
  // stages 0 and 1 went out before the LoRA term)
  for (int mi = m_begin; mi < m_end; ++mi) {
  const QgemmMember mm = set_member(set, mi);
  const uint16_t *act = kTransW ? mm.act : x;
  const int64_t Kc = kTransW ? mm.w.n_out : mm.w.n_in;
  const int64_t nk = member_steps(Kc);
  const bool full = kFull || (rows_ok && (c0 + QBN <= Ncols) && (Kc % QBK == 0));
  if (mi > m_begin) wg_barrier();  // every wave is done with the previous member's LDS stages
  ActDma<kClamp> dma;
  dma.init(act, Kc, M, m0, kstep0, cw, lane);
  if (full) {
    if (mi > m_begin) {
      dma.issue(0, sa[0] + 64 * cw * 64);
      dma.issue(min((int64_t)1, nk - 1), sa[1] + 64 * cw * 64);
    }
    dma.issue(min((int64_t)2, nk - 1), sa[2] + 64 * cw * 64);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(16, 0));  // stage 0 has landed
  }
  // stage 0 ready (the first member's: at the LoRA term's last barrier, when
  // there is an adapter term)
  if (mi > m_begin || r_eff == 0) wg_barrier();
  StageFrags f;
#pragma unroll
  for (int kk = 0; kk < QBK / 16; ++kk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[kk][i] = load_a_frag(sa[0], wm, lane, kk, i);
#pragma unroll
    for (int j = 0; j < 2; ++j) f.b[kk][j] = load_b_frag<kTransW>(sb[0], wn, lane, kk, j);
  }
  // stage 0 is in registers, and this wave's DMA of stage 1 has landed
  if (full)
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(8, 0));
  else
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  wg_barrier();  // stage 1 ready

  // Step k: the 32 MFMAs of stage k run from registers; each fragment register
  // is reloaded with the same fragment of stage k+1 (in LDS since the previous
  // barrier) right after the last MFMA that reads it, so the MFMAs never wait
  // for LDS within a step.  One load, DMA or nothing follows each MFMA, so the
  // wave keeps the matrix core fed while it issues them: A fragment i of
  // slice kk after MFMA (kk, i, 1); the two B fragments of slice kk early in
  // slice kk+1 (after the last slice: after the loop); the two DMAs of a slice
  // after its MFMAs (kk, 2, 0) and (kk, 3, 0).  Stage k+3 of the activation
  // ring goes by DMA into the buffer of stage k (read during step k-1).  At the
  // last step the loads read a stage nobody uses.  Exactly 8 DMAs per step, so
  // waiting for at most 8 outstanding before the barrier means stage k+2 has
  // landed; every read of stage k+1 has returned by then too, except the last
  // B fragments: the weight ring is three stages deep, so the producers
  // overwrite their stage only at step k+2.
  static_assert(kWStages == kActStages, "one ring index serves both rings");
  // LDS instructions of the B fragments read after the last MFMA: one 16-byte
  // read per fragment, or two 8-byte transpose reads
  constexpr int kBReadOps = kTransW ? 4 : 2;
  int ring = 0;  // kt % kActStages, kept by rotation (a 64-bit remainder costs the scalar unit dozens of instructions)
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int ring1 = ring + 1 == kActStages ? 0 : ring + 1;
    uint16_t *dma_dst = sa[ring] + 64 * cw * 64;
    const int64_t dma_kt = min(kt + 3, nk - 1);
    const uint16_t *na = sa[ring1], *nb = sb[ring1];
    ring = ring1;
#pragma unroll
    for (int kk = 0; kk < QBK / 16; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i][0] = mfma(f.a[kk][i], f.b[kk][0], acc[i][0]);
        __builtin_amdgcn_sched_barrier(0);
        if (kk > 0 && i < 2) f.b[kk - 1][i] = load_b_frag<kTransW>(nb, wn, lane, kk - 1, i);
        if (i >= 2 && full) dma.issue(dma_kt, dma_dst, 2 * kk + i - 2, 1);
        __builtin_amdgcn_sched_barrier(0);
        acc[i][1] = mfma(f.a[kk][i], f.b[kk][1], acc[i][1]);
        __builtin_amdgcn_sched_barrier(0);
        f.a[kk][i] = load_a_frag(na, wm, lane, kk, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) f.b[QBK / 16 - 1][j] = load_b_frag<kTransW>(nb, wn, lane, QBK / 16 - 1, j);
    // These last B reads (kBReadOps LDS instructions) may still be in flight
    // at the barrier: their weight stage is overwritten only at step k+2.
    if (full)
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(8, kBReadOps));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, kBReadOps));
    wg_barrier();
  }
  // No LDS-DMA may still be writing when the next member's stages start or the
  // workgroup's LDS is released; the wait names the lane offsets so that their
  // registers stay untouched until then.
  dma.wait_all();
  }  // members

  if (part) {
    // a split: the fp32 tile goes straight from the accumulators to part[z]
    // (each store instruction covers 32 consecutive columns of two rows)
    const int64_t pcols = set.part_cols;
    float *pz = part + (int64_t)blockIdx.z * M * pcols + (kTransW ? 0 : fm.tile0 * QBN);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = c0 + wn * 64 + j * 32 + l32;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int64_t row = m0 + wm * 128 + i * 32 + 8 * (q >> 2) + 4 * lhi + (q & 3);
          if (row < M && col < Ncols) pz[row * pcols + col] = acc[i][j][q];
        }
      }
    return;
  }

  // Epilogue through LDS: the tile is rounded to bf16 into [256][136] (the
  // activation ring's storage), then written out as 16-byte row chunks.  The
  // barrier (consumers only; the producers have ended and no longer count)
  // also waits for every consumer's last DMA.
  __syncthreads();
  constexpr int OLD = QBN + 8;
  uint16_t *ot = &sa[0][0];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = wm * 128 + i * 32 + 8 * (q >> 2) + 4 * lhi + (q & 3);
        __bf16 h = (__bf16)acc[i][j][q];
        ot[row * OLD + wn * 64 + j * 32 + l32] = __builtin_bit_cast(uint16_t, h);
      }
  __syncthreads();
  const bool out_vec = (Ncols % 8) == 0;
  for (int idx = tid; idx < QBM * (QBN / 8); idx += 256) {
    const int row = idx >> 4, ch = idx & 15;
    const int64_t grow = m0 + row, gcol = c0 + 8 * ch;
    if (grow >= M || gcol >= Ncols) continue;
    const u32x4 v = *(const u32x4 *)&ot[row * OLD + 8 * ch];
    if (out_vec && gcol + 8 <= Ncols) {
      *(u32x4 *)&out[grow * Ncols + gcol] = v;
    } else {
      for (int e = 0; e < 8 && gcol + e < Ncols; ++e) out[grow * Ncols + gcol + e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// The outputs of a split launch: one, or a forward set's members, whose
// columns [col0[i], col0[i] + ncols[i]) of the partial tiles go to out[i]
// [M x ncols[i]].
struct SplitOut {
  int count;
  int64_t col0[kMaxSetMembers], ncols[kMaxSetMembers];
  uint16_t *out[kMaxSetMembers];
};

// The splits of a grid: sum over the splits, in split order, rounded to bf16
// once (8 columns per thread; Ncols, the partial tiles' width, is a multiple
// of QBN here).
__global__ __launch_bounds__(256) void qgemm_split_reduce(const float *__restrict__ part, int S, int64_t M,
                                                          int64_t Ncols, SplitOut so) {
  const int64_t n8 = M * Ncols / 8, zs = M * Ncols / 4;  // zs: one split in float4 units
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    // destination of these 8 columns (members' column ranges are multiples of 8)
    uint16_t *dst;
    if (so.count == 1) {
      dst = so.out[0] + 8 * i;
    } else {
      const int64_t row = (8 * i) / Ncols, col = 8 * i - row * Ncols;
      int m = 0;
      for (int k = 1; k < so.count; ++k)
        if (col >= so.col0[k]) m = k;
      dst = so.out[m] + row * so.ncols[m] + (col - so.col0[m]);
    }
    const f32x4 *p = (const f32x4 *)part + 2 * i;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    for (int z0 = 0; z0 < S; z0 += 4) {
      f32x4 v[4][2];
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        const bool in = z0 + z < S;
        v[z][0] = in ? p[(int64_t)(z0 + z) * zs] : f32x4{0.f, 0.f, 0.f, 0.f};
        v[z][1] = in ? p[(int64_t)(z0 + z) * zs + 1] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int z = 0; z < 4; ++z)
        if (z0 + z < S) {
          a += v[z][0];
          b += v[z][1];
        }
    }
    *(u32x4 *)dst = u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                          pack_bf16x2(b[2], b[3])};
  }
}

SplitOut split_out(uint16_t *out, int64_t ncols) {
  SplitOut so{};
  so.count = 1;
  so.col0[0] = 0;
  so.ncols[0] = ncols;
  so.out[0] = out;
  return so;
}

// ---------------------------------------------------------------------------
// Few-token tiles.  With a few dozen tokens a 256-row tile is mostly padding:
// its matrix work is wasted and the step time is the decode, which only the
// four producer waves of qgemm_ws do.  qgemm_sm takes kRows x 128 output tiles
// (kRows = 64 or 128) in workgroups of four waves, two workgroups per CU, and
// every wave both decodes (the producer lane mapping of qgemm_ws: one unit of
// 32 codes per lane and step, the same register byte tables) and multiplies
// (tile rows 0..kRows-1, columns 32 w .. 32 w + 31), so that two waves per
// SIMD issue decode instructions.  The activation tile (kRows x 64 per step)
// goes through registers into LDS, rows at or past M reading row M - 1 (never
// stored).  Every load is an ordinary compiler-tracked load, so the waits the
// compiler places are exact.  Codes and activation are loaded three steps
// ahead of their LDS store into one of three register sets.  With 64 rows the
// LDS ring has three stages (stage k multiplied while stage k+2 is written,
// 78 KB); with 128 rows two (stage k+1 written, 68 KB), so that two
// workgroups still fit a CU.  Single linears whose tiles are full in columns
// and contraction, without a dropout mask; a split contraction (blockIdx.z)
// as in qgemm_ws.
struct SmStage {
  Stage w;
  u32x4 a0, a1;  // row tid / 4, chunks 2 (tid % 4) and 2 (tid % 4) + 1
  u32x4 a2, a3;  // 128-row tiles: the same chunks of row tid / 4 + 64
};

// The 8 MFMAs of one stage of a 64-row tile for wave w: A fragments of rows
// 0..63 (two 32-row halves), the B fragment of columns 32 w .. 32 w + 31.
template <bool kTransW>
__device__ __forceinline__ void sm_stage_mfma(const uint16_t *A, const uint16_t *B, int w, int lane,
                                              f32x16 (&acc)[2]) {
  u32x4 a[QBK / 16][2], b[QBK / 16];
#pragma unroll
  for (int kk = 0; kk < QBK / 16; ++kk) {
    a[kk][0] = load_a_frag(A, 0, lane, kk, 0);
    a[kk][1] = load_a_frag(A, 0, lane, kk, 1);
    b[kk] = load_b_frag<kTransW>(B, w >> 1, lane, kk, w & 1);
  }
#pragma unroll
  for (int kk = 0; kk < QBK / 16; ++kk) {
    acc[0] = mfma(a[kk][0], b[kk], acc[0]);
    acc[1] = mfma(a[kk][1], b[kk], acc[1]);
  }
}

// The 16 MFMAs of one stage of a 128-row tile: the fragments of slice kk+1
// read while slice kk multiplies (registers for two slices).
template <bool kTransW>
__device__ __forceinline__ void sm_stage_mfma(const uint16_t *A, const uint16_t *B, int w, int lane,
                                              f32x16 (&acc)[4]) {
  u32x4 a[2][4], b[2];
  auto frags = [&](int kk, u32x4 (&fa)[4], u32x4 &fb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = load_a_frag(A, 0, lane, kk, i);
    fb = load_b_frag<kTransW>(B, w >> 1, lane, kk, w & 1);
  };
  frags(0, a[0], b[0]);
#pragma unroll
  for (int kk = 0; kk < QBK / 16; ++kk) {
    if (kk + 1 < QBK / 16) frags(kk + 1, a[(kk + 1) & 1], b[(kk + 1) & 1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = mfma(a[kk & 1][i], b[kk & 1], acc[i]);
  }
}

template <bool kTransW, bool kDQ, int kRows>
__global__ __launch_bounds__(256, 2) void qgemm_sm(QgemmSet set, int64_t M, const uint16_t *__restrict__ x,
                                                   const uint16_t *__restrict__ la, const uint16_t *__restrict__ lb,
                                                   int r, float scale, uint16_t *__restrict__ gx, Codebook cb,
                                                   float *__restrict__ part, int64_t split_steps) {
  constexpr int kSt = kRows == 64 ? 3 : 2;  // LDS stages
  constexpr int kTiles = kRows / 32;        // 32-row MFMA tiles; also 16-byte activation chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t sa[kSt][kRows * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sb[kSt][QBN * QLD];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, lhi = lane >> 5;
  const QgemmMember mm = set.m[0];
  const int64_t Ncols = kTransW ? mm.w.n_in : mm.w.n_out, Kc = kTransW ? mm.w.n_out : mm.w.n_in;
  const int64_t m0 = (int64_t)blockIdx.x * kRows, c0 = (int64_t)blockIdx.y * QBN;
  const uint16_t *act = kTransW ? mm.act : x;
  const uint16_t *lb_t = kTransW ? lb : mm.lb;
  uint16_t *out = kTransW ? gx : mm.out;
  const int64_t kstep0 = part ? (int64_t)blockIdx.z * split_steps : 0;
  const int64_t nk = part ? min(split_steps, Kc / QBK - kstep0) : Kc / QBK;
  const int r_eff = blockIdx.z == 0 ? r : 0;
  const float mu = kDQ ? *mm.w.mu : 0.f;
  const Producer<kTransW, kDQ> p = member_producer<kTransW, kDQ>(mm, x, M, m0, c0, tid, mu, kstep0);

  // this lane's activation rows (clamped) and chunk pair
  const int arow = tid >> 2, ach = 2 * (tid & 3);
  const uint16_t *asrc = act + min(m0 + arow, M - 1) * Kc + kstep0 * QBK + 8 * ach;
  const uint16_t *asrc2 = act + min(m0 + arow + 64, M - 1) * Kc + kstep0 * QBK + 8 * ach;
  auto st = [nk](int64_t k) { return min(k, nk - 1); };
  auto load = [&](int64_t k, SmStage &c) {
    p.template load_w<true>(k, c.w);
    c.a0 = *(const u32x4 *)(asrc + k * QBK);
    c.a1 = *(const u32x4 *)(asrc + k * QBK + 8);
    if (kRows == 128) {
      c.a2 = *(const u32x4 *)(asrc2 + k * QBK);
      c.a3 = *(const u32x4 *)(asrc2 + k * QBK + 8);
    }
  };
  auto store = [&](const SmStage &c, int buf) {
    p.write_rt(c.w, cb, sb[buf]);
    *(u32x4 *)&sa[buf][act_off(arow, ach)] = c.a0;
    *(u32x4 *)&sa[buf][act_off(arow, ach + 1)] = c.a1;
    if (kRows == 128) {
      *(u32x4 *)&sa[buf][act_off(arow + 64, ach)] = c.a2;
      *(u32x4 *)&sa[buf][act_off(arow + 64, ach + 1)] = c.a3;
    }
  };

  SmStage s0, s1, s2;
  load(0, s0);
  load(st(1), s1);
  load(st(2), s2);

  f32x16 acc[kTiles];
#pragma unroll
  for (int i = 0; i < kTiles; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[i][q] = 0.f;
  // LoRA term (first split only): scale * la lb^T, one 64-wide chunk of the
  // rank at a time through the last LDS stage (zero past r and past M)
  constexpr int kL = kSt - 1;
  const bool lvec = (r % 8) == 0 && (set.ld_la % 8) == 0;
  for (int j0 = 0; j0 < r_eff; j0 += QBK) {
    u32x4 va[kTiles], vb[4];
#pragma unroll
    for (int it = 0; it < kTiles; ++it) {  // kRows rows x 8 chunks of the rank
      const int idx = tid + 256 * it, row = idx >> 3, ch = idx & 7;
      const int64_t grow = m0 + row;
      va[it] = grow < M ? ld8(la + grow * set.ld_la, j0 + 8 * ch, r, lvec) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = tid + 256 * it;
      if (!kTransW) {  // 128 output columns x 8 chunks of the rank
        const int row = idx >> 3, ch = idx & 7;
        vb[it] = ld8(lb_t + (c0 + row) * r, j0 + 8 * ch, r, lvec);
      } else {  // 64 rank rows x 16 chunks of 8 columns
        const int jr = idx >> 4, ch = idx & 15;
        vb[it] = j0 + jr < r ? *(const u32x4 *)(lb_t + (int64_t)(j0 + jr) * Ncols + c0 + 8 * ch)
                             : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int it = 0; it < kTiles; ++it) {
      const int idx = tid + 256 * it;
      *(u32x4 *)&sa[kL][act_off(idx >> 3, idx & 7)] = va[it];
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = tid + 256 * it;
      if (!kTransW)
        *(u32x4 *)&sb[kL][(idx >> 3) * QLD + 8 * (idx & 7)] = vb[it];
      else
        *(u32x4 *)&sb[kL][(idx >> 4) * TLD + 8 * (idx & 15)] = vb[it];
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    wg_barrier();
    sm_stage_mfma<kTransW>(sa[kL], sb[kL], w, lane, acc);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    wg_barrier();  // the last stage is free again
  }
#pragma unroll
  for (int i = 0; i < kTiles; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[i][q] *= scale;

  int64_t kt = 0;
  if constexpr (kSt == 3) {
    // at step k: multiply stage k, write stage k+2 (its set then fetches k+5)
    store(s0, 0);
    load(st(3), s0);
    store(s1, 1);
    load(st(4), s1);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    wg_barrier();  // stages 0 and 1 ready
#define QGEMM_SM_STEP(K_, CUR, BUF, NEXT)                                              \
  if ((K_) < nk) {                                                                    \
    sm_stage_mfma<kTransW>(sa[BUF], sb[BUF], w, lane, acc);                   \
    store(CUR, NEXT);                                                                 \
    load(st((K_) + 5), CUR);                                                          \
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));                                   \
    wg_barrier();                                                                     \
  }
    for (; kt + 3 <= nk; kt += 3) {
      QGEMM_SM_STEP(kt, s2, 0, 2)
      QGEMM_SM_STEP(kt + 1, s0, 1, 0)
      QGEMM_SM_STEP(kt + 2, s1, 2, 1)
    }
    QGEMM_SM_STEP(kt, s2, 0, 2)
    QGEMM_SM_STEP(kt + 1, s0, 1, 0)
#undef QGEMM_SM_STEP
  } else {
    // at step k: multiply stage k, write stage k+1 into the other stage (its set
    // then fetches k+4)
    store(s0, 0);
    load(st(3), s0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    wg_barrier();  // stage 0 ready
#define QGEMM_SM_STEP(K_, CUR)                                                         \
  if ((K_) < nk) {                                                                    \
    const int buf = (int)((K_) & 1);                                                  \
    sm_stage_mfma<kTransW>(sa[buf], sb[buf], w, lane, acc);                   \
    store(CUR, buf ^ 1);                                                              \
    load(st((K_) + 4), CUR);                                                          \
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));                                   \
    wg_barrier();                                                                     \
  }
    for (; kt + 3 <= nk; kt += 3) {
      QGEMM_SM_STEP(kt, s1)
      QGEMM_SM_STEP(kt + 1, s2)
      QGEMM_SM_STEP(kt + 2, s0)
    }
    QGEMM_SM_STEP(kt, s1)
    QGEMM_SM_STEP(kt + 1, s2)
#undef QGEMM_SM_STEP
  }

  // element q of acc[i]: tile row 32 i + 8 (q / 4) + 4 (lane / 32) + q % 4, column 32 w + lane % 32
  const int64_t col = c0 + 32 * w + l32;
  if (part) {
    float *pz = part + (int64_t)blockIdx.z * M * Ncols;
#pragma unroll
    for (int i = 0; i < kTiles; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + 32 * i + 8 * (q >> 2) + 4 * lhi + (q & 3);
        if (row < M) pz[row * Ncols + col] = acc[i][q];
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < kTiles; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t row = m0 + 32 * i + 8 * (q >> 2) + 4 * lhi + (q & 3);
      __bf16 h = (__bf16)acc[i][q];
      if (row < M) out[row * Ncols + col] = __builtin_bit_cast(uint16_t, h);
    }
}

template <int kRows>
void launch_sm(bool trans_w, bool dq, dim3 g, hipStream_t st, const QgemmSet &s, int64_t M, const uint16_t *x,
               const uint16_t *la, const uint16_t *lb, int r, float scale, uint16_t *gx, const Codebook &cb,
               float *part, int64_t split_steps) {
  if (trans_w) {
    if (dq)
      qgemm_sm<true, true, kRows><<<g, 256, 0, st>>>(s, M, x, la, lb, r, scale, gx, cb, part, split_steps);
    else
      qgemm_sm<true, false, kRows><<<g, 256, 0, st>>>(s, M, x, la, lb, r, scale, gx, cb, part, split_steps);
  } else {
    if (dq)
      qgemm_sm<false, true, kRows><<<g, 256, 0, st>>>(s, M, x, la, lb, r, scale, gx, cb, part, split_steps);
    else
      qgemm_sm<false, false, kRows><<<g, 256, 0, st>>>(s, M, x, la, lb, r, scale, gx, cb, part, split_steps);
  }
}

// Tiles of a grid: any (some may be partial), all full, or all full with the
// last row tile's missing rows clamped.
enum class Tiles { kAny, kFull, kFullClamped };

template <bool kTransW, bool kDQ, bool kDrop>
void launch_ws(Tiles tiles, dim3 g, hipStream_t st, const QgemmSet &s, int64_t M, const uint16_t *x,
               const uint16_t *la, const uint16_t *lb, int r, float scale, uint16_t *gx, const Codebook &cb,
               const uint32_t *keep, float *part, int64_t split_steps) {
  if (tiles == Tiles::kFullClamped)
    qgemm_ws<kTransW, kDQ, kDrop, true, true><<<g, 512, 0, st>>>(s, M, x, la, lb, r, scale, gx, cb, keep, part,
                                                                  split_steps);
  else if (tiles == Tiles::kFull)
    qgemm_ws<kTransW, kDQ, kDrop, false, true><<<g, 512, 0, st>>>(s, M, x, la, lb, r, scale, gx, cb, keep, part,
                                                                   split_steps);
  else
    qgemm_ws<kTransW, kDQ, kDrop, false, false><<<g, 512, 0, st>>>(s, M, x, la, lb, r, scale, gx, cb, keep,
                                                                    part, split_steps);
}

}  // namespace

// A single linear whose tile grid fills the 256 CUs poorly (few tokens, or a
// tile count just past a multiple of 256) splits its contraction.  One
// workgroup runs per CU, so a launch of W workgroups takes ceil(W / 256)
// rounds, each as long as one workgroup: about 4 steps of set-up and epilogue
// plus its contraction steps (64 wide, about 1 us each at full occupancy).
// The split count minimises that estimate plus the reduction's reading of the
// fp32 partials (at about 4 GB per ms), with at least 4 steps per split.  Only
// shapes whose tiles are full in columns and contraction split, so every
// workgroup runs the full-tile pipeline.
QgemmSplit qgemm_split(int64_t M, int64_t Ncols, int64_t Kc, double *cost) {
  QgemmSplit sp{1, 0};
  if (cost) *cost = 1e30;
  if (M < 1 || Ncols % QBN != 0 || Kc % QBK != 0) return sp;
  const int64_t tiles = (M + QBM - 1) / QBM * (Ncols / QBN), nk = Kc / QBK;
  double best = 0.0;
  for (int64_t S = 1; S <= std::min<int64_t>(64, nk / 4) || S == 1; ++S) {
    const int64_t steps = (nk + S - 1) / S, splits = (nk + steps - 1) / steps;
    if (splits != S) continue;
    const double rounds = (double)((tiles * S + 255) / 256);
    const double reduce_us = S > 1 ? (double)S * M * Ncols * 4.0 / 4e6 + 3.0 : 0.0;
    const double cost = rounds * (4.0 + (double)steps) + reduce_us;
    if (S == 1 || cost < best) {
      best = cost;
      sp = S > 1 ? QgemmSplit{(int)S, steps} : QgemmSplit{1, 0};
    }
  }
  if (cost) *cost = best;
  return sp;
}

// Few-token tiles (qgemm_sm) for launches of at most this many tokens: 64-row
// tiles up to 64 tokens, 128-row tiles above.
constexpr int64_t kSmMaxRows = 128;
constexpr int sm_rows(int64_t M) { return M <= 64 ? 64 : 128; }

// The split of a few-token launch: two workgroups run per CU (512 at once);
// the estimate is rounds x (about 4 steps of set-up + steps per split) at
// about 0.9 us a step, plus the fp32 partials written and read back at about
// 2 bytes per ps and a few us for the reduction's launch (fitted to split
// sweeps at 4096 x 4096, 11008 x 4096 and 22016 x 8192 with 16 and 64 tokens).
QgemmSplit qgemm_sm_split(int64_t M, int64_t Ncols, int64_t Kc, double *cost = nullptr) {
  QgemmSplit sp{1, 0};
  if (cost) *cost = 1e30;
  if (M < 1 || Ncols % QBN != 0 || Kc % QBK != 0) return sp;
  const int rows = sm_rows(M);
  const int64_t tiles = (M + rows - 1) / rows * (Ncols / QBN), nk = Kc / QBK;
  double best = 0.0;
  for (int64_t S = 1; S <= std::min<int64_t>(64, nk / 4) || S == 1; ++S) {
    const int64_t steps = (nk + S - 1) / S, splits = (nk + steps - 1) / steps;
    if (splits != S) continue;
    const double rounds = (double)((tiles * S + 511) / 512);
    const double reduce_us = S > 1 ? (double)S * M * Ncols * 4.0 / 2e6 + 3.0 : 0.0;
    const double cost = rounds * (4.0 + (double)steps) * 0.9 + reduce_us;
    if (S == 1 || cost < best) {
      best = cost;
      sp = S > 1 ? QgemmSplit{(int)S, steps} : QgemmSplit{1, 0};
    }
  }
  if (cost) *cost = best;
  return sp;
}

size_t qgemm_split_floats(int64_t M, int64_t Ncols, int64_t Kc) {
  const QgemmSplit sp = qgemm_split(M, Ncols, Kc);
  size_t f = sp.splits > 1 ? (size_t)sp.splits * M * Ncols : 0;
  if (M <= kSmMaxRows) {
    const QgemmSplit ss = qgemm_sm_split(M, Ncols, Kc);
    if (ss.splits > 1) f = std::max(f, (size_t)ss.splits * M * Ncols);
  }
  return f;
}

// grad_x of a set at a few tokens, member by member: the fp32 partial tiles of
// every member's splits (at least one each), side by side along z.
size_t qgemm_set_dx_member_floats(int64_t M, int count, const int64_t *n_out, int64_t n_in) {
  if (M > kSmMaxRows || n_in % QBN != 0) return 0;
  size_t f = 0;
  for (int i = 0; i < count; ++i) {
    if (n_out[i] % QBK != 0) return 0;
    f += (size_t)std::max(1, qgemm_sm_split(M, n_in, n_out[i]).splits) * M * n_in;
  }
  return f;
}

hipError_t launch_qgemm_set(bool trans_w, const QgemmSet &set, int64_t M, const uint16_t *x, const uint16_t *la,
                            const uint16_t *lb, int r, float scale, uint16_t *gx, const Codebook &cb, hipStream_t st,
                            const uint32_t *keep, float *part) {
  if (set.count < 1 || set.count > kMaxSetMembers) return hipErrorInvalidValue;
  QgemmSet s = set;
  int64_t ytiles = 0, kc_max = 0;
  if (!trans_w) {
    for (int i = 0; i < s.count; ++i) {
      s.m[i].tile0 = ytiles;
      ytiles += (s.m[i].w.n_out + QBN - 1) / QBN;
    }
    kc_max = s.m[0].w.n_in;
  } else {
    ytiles = (s.m[0].w.n_in + QBN - 1) / QBN;
    for (int i = 0; i < s.count; ++i) kc_max = std::max(kc_max, s.m[i].w.n_out);
  }
  for (int i = s.count; i < kMaxSetMembers; ++i) s.m[i] = s.m[0];
  const int64_t Ncols = trans_w ? s.m[0].w.n_in : s.m[0].w.n_out;
  // Every tile full in columns and contraction steps: the grid runs the
  // full-tile pipeline only, with the last row tile's missing rows reading a
  // valid row when M is not a multiple of QBM (byte offsets within a tile
  // stay below 2^32).
  bool cols_k_full = true;
  for (int i = 0; i < s.count; ++i) {
    const int64_t nc = trans_w ? s.m[0].w.n_in : s.m[i].w.n_out, kc = trans_w ? s.m[i].w.n_out : s.m[i].w.n_in;
    cols_k_full = cols_k_full && nc % QBN == 0 && kc % QBK == 0;
  }
  const bool dq = s.m[0].w.dq;
  if (s.count == 1 && cols_k_full && M <= kSmMaxRows && !keep) {
    // few tokens: qgemm_sm
    const QgemmSplit sp = part ? qgemm_sm_split(M, Ncols, kc_max) : QgemmSplit{1, 0};
    float *pz = sp.splits > 1 ? part : nullptr;
    const int rows = sm_rows(M);
    const dim3 g((unsigned)((M + rows - 1) / rows), (unsigned)(Ncols / QBN), (unsigned)sp.splits);
    if (rows == 64)
      launch_sm<64>(trans_w, dq, g, st, s, M, x, la, lb, r, scale, gx, cb, pz, sp.steps);
    else
      launch_sm<128>(trans_w, dq, g, st, s, M, x, la, lb, r, scale, gx, cb, pz, sp.steps);
    if (pz) {
      uint16_t *out = trans_w ? gx : s.m[0].out;
      int64_t blocks = (M * Ncols / 8 + 255) / 256;
      if (blocks > 2048) blocks = 2048;
      qgemm_split_reduce<<<(unsigned)blocks, 256, 0, st>>>(pz, sp.splits, M, Ncols, split_out(out, Ncols));
    }
    return hipGetLastError();
  }
  // grad_x of a set at a few tokens: each member on the few-token tiles, every
  // split of every member writing its fp32 partial tile (a member's first
  // split adds its share s v_i A_i of the adapter term), and one reduction over
  // all of them; against one launch of 256-row tiles contracting over every
  // member, by the split cost models (about 5 us per extra launch).
  if (trans_w && s.count > 1 && cols_k_full && M <= kSmMaxRows && part && !keep) {
    int64_t kc_all = 0;
    for (int i = 0; i < s.count; ++i) kc_all += s.m[i].w.n_out;
    double c_set = 0.0, c_members = 5.0 * (s.count - 1);
    qgemm_split(M, Ncols, kc_all, &c_set);
    QgemmSplit spm[kMaxSetMembers];
    for (int i = 0; i < s.count; ++i) {
      double c = 0.0;
      spm[i] = qgemm_sm_split(M, Ncols, s.m[i].w.n_out, &c);
      c_members += c;
    }
    if (c_members < c_set) {
      const int rows = sm_rows(M), rm = r / s.count;  // every member's rank
      int64_t z = 0;
      for (int i = 0; i < s.count; ++i) {
        QgemmSet one{};
        one.count = 1;
        one.ld_la = s.ld_la;
        one.m[0] = s.m[i];
        one.part_cols = Ncols;
        const int S = spm[i].splits;
        const int64_t steps = S > 1 ? spm[i].steps : s.m[i].w.n_out / QBK;
        const dim3 g((unsigned)((M + rows - 1) / rows), (unsigned)(Ncols / QBN), (unsigned)S);
        const uint16_t *la_i = la + (int64_t)i * rm, *lb_i = lb + (int64_t)i * rm * Ncols;
        float *pz = part + z * M * Ncols;
        if (rows == 64)
          launch_sm<64>(true, dq, g, st, one, M, x, la_i, lb_i, rm, scale, gx, cb, pz, steps);
        else
          launch_sm<128>(true, dq, g, st, one, M, x, la_i, lb_i, rm, scale, gx, cb, pz, steps);
        z += S;
      }
      int64_t blocks = (M * Ncols / 8 + 255) / 256;
      if (blocks > 2048) blocks = 2048;
      qgemm_split_reduce<<<(unsigned)blocks, 256, 0, st>>>(part, (int)z, M, Ncols, split_out(gx, Ncols));
      return hipGetLastError();
    }
  }
  // A forward set at a few tokens: each member on the few-token tiles (one
  // launch and reduction per member, about 5 us each) can beat one launch of
  // all the members on 256-row tiles; the split cost models decide.
  if (!trans_w && s.count > 1 && cols_k_full && M <= kSmMaxRows && part) {
    double c_set = 0.0, c_members = 5.0 * (s.count - 1);
    qgemm_split(M, ytiles * QBN, kc_max, &c_set);
    for (int i = 0; i < s.count; ++i) {
      double c = 0.0;
      qgemm_sm_split(M, s.m[i].w.n_out, kc_max, &c);
      c_members += c;
    }
    if (c_members < c_set) {
      for (int i = 0; i < s.count; ++i) {
        QgemmSet one{};
        one.count = 1;
        one.ld_la = s.ld_la;
        one.m[0] = s.m[i];
        one.m[0].tile0 = 0;
        const hipError_t e =
            launch_qgemm_set(false, one, M, x, la + (int64_t)i * r, lb, r, scale, gx, cb, st, nullptr, part);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
  }
  Tiles tiles = Tiles::kAny;
  if (cols_k_full && M % QBM == 0)
    tiles = Tiles::kFull;
  else if (cols_k_full && kc_max < ((int64_t)1 << 22))
    tiles = Tiles::kFullClamped;
  // A split contracts the same range of steps of every member: grad_x of a set
  // splits only when its members share n_out; a forward set (members share
  // n_in) when every member's columns are whole tiles, its partial tiles side
  // by side.
  bool same_kc = true;
  for (int i = 1; i < s.count; ++i) same_kc = same_kc && s.m[i].w.n_out == s.m[0].w.n_out;
  const int64_t pcols = trans_w || s.count == 1 ? Ncols : ytiles * QBN;
  s.part_cols = pcols;
  QgemmSplit sp{1, 0};
  if (part && (s.count == 1 || (trans_w && same_kc) || (!trans_w && cols_k_full))) sp = qgemm_split(M, pcols, kc_max);
  float *pz = sp.splits > 1 ? part : nullptr;
  const dim3 g((unsigned)((M + QBM - 1) / QBM), (unsigned)ytiles, (unsigned)sp.splits);
  if (!trans_w) {  // the forward never takes a dropout mask
    if (dq)
      launch_ws<false, true, false>(tiles, g, st, s, M, x, la, lb, r, scale, gx, cb, nullptr, pz, sp.steps);
    else
      launch_ws<false, false, false>(tiles, g, st, s, M, x, la, lb, r, scale, gx, cb, nullptr, pz, sp.steps);
  } else if (keep) {
    if (dq)
      launch_ws<true, true, true>(tiles, g, st, s, M, x, la, lb, r, scale, gx, cb, keep, pz, sp.steps);
    else
      launch_ws<true, false, true>(tiles, g, st, s, M, x, la, lb, r, scale, gx, cb, keep, pz, sp.steps);
  } else {
    if (dq)
      launch_ws<true, true, false>(tiles, g, st, s, M, x, la, lb, r, scale, gx, cb, nullptr, pz, sp.steps);
    else
      launch_ws<true, false, false>(tiles, g, st, s, M, x, la, lb, r, scale, gx, cb, nullptr, pz, sp.steps);
  }
  if (pz) {
    SplitOut so = split_out(trans_w ? gx : s.m[0].out, Ncols);
    if (!trans_w && s.count > 1) {
      so.count = s.count;
      for (int i = 0; i < s.count; ++i) {
        so.col0[i] = s.m[i].tile0 * QBN;
        so.ncols[i] = s.m[i].w.n_out;
        so.out[i] = s.m[i].out;
      }
    }
    int64_t blocks = (M * pcols / 8 + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    qgemm_split_reduce<<<(unsigned)blocks, 256, 0, st>>>(pz, sp.splits, M, pcols, so);
  }
  return hipGetLastError();
}

hipError_t launch_qgemm(bool trans_w, const uint16_t *act, int64_t M, int64_t Ncols, int64_t Kc, const QWeight &w,
                        const uint16_t *la, const uint16_t *lb, int r, float scale, uint16_t *out,
                        const Codebook &cb, hipStream_t st, const uint32_t *keep, float *part) {
  (void)Ncols;
  (void)Kc;
  QgemmSet s{};
  s.count = 1;
  s.ld_la = r;
  s.m[0].w = w;
  if (trans_w) {
    s.m[0].act = act;
    return launch_qgemm_set(true, s, M, nullptr, la, lb, r, scale, out, cb, st, keep, part);
  }
  s.m[0].lb = lb;
  s.m[0].out = out;
  return launch_qgemm_set(false, s, M, act, la, nullptr, r, scale, nullptr, cb, st, nullptr, part);
}

}  // namespace qlora
