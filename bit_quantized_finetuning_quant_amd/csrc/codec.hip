// NF4 + FP8 double-quantization codec kernels for gfx950.
//
// Method: the "qlora" encyclopedia entry (tonho.wtf), section "como funciona":
// 4-bit levels from standard-normal quantiles with an exact zero, one absmax
// constant per 64-element block, constants quantized to FP8 in blocks of 256.
//
// Kernels
//   zero_words        clears the status word and the exponent bins
//   quantize_blocks   absmax, nearest code by exact thresholds, nibble packing,
//                     exact exponent-binned partial sums of the absmax values
//   mean_from_bins    one thread: exact sum -> fp32 mean (round to nearest even)
//   double_quantize   one workgroup per 256-block group: fp32 scale, e4m3 codes
//   dequantize_bf16   streaming decode to bf16 (HBM bound)

#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace qlora {

__global__ void zero_words(uint32_t *p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Largest fp32 strictly below f (f finite).
__device__ __forceinline__ float next_down(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0u) return __uint_as_float(0x80000001u);
  return __uint_as_float((u & 0x80000000u) ? u + 1u : u - 1u);
}

// Threshold j of a block with constant c1: x is above midpoint j of the
// levels exactly when x > tau_j (fp32 compare).  tau_j is the fp32 rounding
// down of the exact product M_j c1 (exact in fp64: M_j has at most 26
// significant bits, c1 24); an exact tie on the negative side (j < 7) counts
// as above (toward zero), so tau_j moves one step further down there.
__device__ __forceinline__ float threshold(double m, double c1, int j) {
  const double t = m * c1;  // exact in fp64
  float f = (float)t;
  const double fd = (double)f;
  if (fd > t || (fd == t && j < 7)) f = next_down(f);
  return f;
}

// The 15 thresholds of a block.
struct Thresholds {
  float t[15];
};

// The number of thresholds below x, #{j : x > tau_j}, for non-decreasing
// tau_0..tau_14 (M_j increases with j, c1 >= 0, and rounding down keeps the
// order): four steps of a binary search, each comparing x with the one
// threshold the previous steps select.  The candidates are selected as values
// (a conditional between two array elements would be a conditional address,
// which puts the array in scratch memory).
__device__ __forceinline__ float pick(bool c, float a, float b) { return c ? a : b; }

__device__ __forceinline__ uint32_t code_of(float x, const Thresholds &tau) {
  const float *t = tau.t;
  const bool b3 = x > t[7];
  const bool b2 = x > pick(b3, t[11], t[3]);
  const bool b1 = x > pick(b3, pick(b2, t[13], t[9]), pick(b2, t[5], t[1]));
  const float u = pick(b3, pick(b2, pick(b1, t[14], t[12]), pick(b1, t[10], t[8])),
                       pick(b2, pick(b1, t[6], t[4]), pick(b1, t[2], t[0])));
  const bool b0 = x > u;
  return 8u * b3 + 4u * b2 + 2u * b1 + (uint32_t)b0;
}

// 8 lanes own one 64-element block (8 elements each); a 256-thread workgroup
// covers 32 blocks per pass and strides over the tensor.  Lane s of a block
// forms thresholds s and s + 8 and the 8 lanes exchange them.
template <bool kBf16Src>
__global__ __launch_bounds__(256) void quantize_blocks(const void *__restrict__ src, int64_t numel,
                                                       int64_t nblocks, uint8_t *__restrict__ codes,
                                                       int64_t codes_bytes, float *__restrict__ c1_out,
                                                       unsigned long long *__restrict__ bins,
                                                       uint32_t *__restrict__ status, Midpoints mid) {
  __shared__ unsigned long long sbins[256];
  __shared__ double smid[16];
  sbins[threadIdx.x] = 0ull;
  if (threadIdx.x < 15) smid[threadIdx.x] = mid.m[threadIdx.x];
  __syncthreads();
  const int sub = threadIdx.x & 7;
  const double m_lo = smid[sub], m_hi = sub < 7 ? smid[sub + 8] : 0.0;
  bool bad = false;
  for (int64_t b = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3); b < nblocks; b += (int64_t)gridDim.x * 32) {
    const int64_t e0 = b * kBlock + sub * 8;
    float x[8];
    if (e0 + 8 <= numel) {
      if (kBf16Src) {
        u32x4 v = *(const u32x4 *)((const uint16_t *)src + e0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = bf16_lo(v[i]);
          x[2 * i + 1] = bf16_hi(v[i]);
        }
      } else {
        f32x4 v0 = *(const f32x4 *)((const float *)src + e0);
        f32x4 v1 = *(const f32x4 *)((const float *)src + e0 + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = v0[i];
          x[4 + i] = v1[i];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float v = 0.f;
        if (e0 + i < numel) {
          v = kBf16Src ? __uint_as_float((uint32_t)((const uint16_t *)src)[e0 + i] << 16)
                       : ((const float *)src)[e0 + i];
        }
        x[i] = v;
      }
    }
    // block absmax: max of |x| bit patterns (monotone for non-negative floats)
    uint32_t am = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = max(am, __float_as_uint(x[i]) & 0x7FFFFFFFu);
    am = max(am, (uint32_t)__shfl_xor((int)am, 1, 8));
    am = max(am, (uint32_t)__shfl_xor((int)am, 2, 8));
    am = max(am, (uint32_t)__shfl_xor((int)am, 4, 8));
    if (am >= 0x7F800000u) bad = true;
    const float c1 = __uint_as_float(am);
    const double cd = (double)c1;
    const float t_lo = threshold(m_lo, cd, sub), t_hi = threshold(m_hi, cd, sub + 8);
    Thresholds tau;
#pragma unroll
    for (int j = 0; j < 8; ++j) tau.t[j] = __shfl(t_lo, j, 8);
#pragma unroll
    for (int j = 8; j < 15; ++j) tau.t[j] = __shfl(t_hi, j - 8, 8);
    uint32_t packed = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= code_of(x[i], tau) << (4 * i);
    const int64_t byte0 = e0 >> 1;
    if (byte0 + 4 <= codes_bytes) {
      *(uint32_t *)(codes + byte0) = packed;
    } else {
      for (int i = 0; i < 4; ++i)
        if (byte0 + i < codes_bytes) codes[byte0 + i] = (uint8_t)(packed >> (8 * i));
    }
    if (sub == 0) {
      c1_out[b] = c1;
      const uint32_t ex = am >> 23;
      if (ex < 255u) {
        const uint32_t frac = am & 0x7FFFFFu;
        const unsigned long long mant = ex ? (frac | 0x800000u) : frac;
        if (mant) atomicAdd(&sbins[ex ? ex : 1u], mant);
      }
    }
  }
  if (bad) atomicOr(status, 1u);
  __syncthreads();
  const unsigned long long s = sbins[threadIdx.x];
  if (s) atomicAdd(&bins[(blockIdx.x % kBinCopies) * 256 + threadIdx.x], s);
}

// Exact mean of the block constants.  bins[e] holds the sum of the 24-bit
// significands of all constants with biased exponent e (subnormals in bin 1),
// so the exact sum is Z * 2^-149 with Z = sum_e bins[e] << (e - 1).  The mean
// Z * 2^-149 / n is rounded to the nearest fp32 (ties to even) by long
// division of Z * 2^64 by n and inspection of the quotient's bits.
__global__ __launch_bounds__(256) void mean_from_bins(const unsigned long long *__restrict__ bins, int64_t nblocks,
                                                      float *__restrict__ mu) {
  // the copies of each bin are added by 256 threads at once (each bin sum stays
  // below nblocks * 2^24 <= 2^55), then one thread forms the exact quotient
  __shared__ unsigned long long sb[256];
  {
    unsigned long long t = 0;
#pragma unroll
    for (int c = 0; c < kBinCopies; ++c) t += bins[c * 256 + threadIdx.x];
    sb[threadIdx.x] = t;
  }
  __syncthreads();
  // Z = sum_e sb[e] << (e - 1), in 32-bit limbs: bin e adds three limbs at
  // limb offset (e - 1 + 64) / 32 (the 64 extra bits keep the quotient's
  // fraction); the 64-bit limb sums stay below 2^40, and integer addition in
  // any order is exact
  __shared__ unsigned long long limb[12];
  if (threadIdx.x < 12) limb[threadIdx.x] = 0ull;
  __syncthreads();
  {
    const int e = threadIdx.x;
    const unsigned long long v = (e >= 1 && e < 255) ? sb[e] : 0ull;
    if (v) {
      const int sh = e - 1 + 64;
      const int wo = sh >> 5, bo = sh & 31;
      atomicAdd(&limb[wo], (unsigned long long)(uint32_t)(v << bo));
      atomicAdd(&limb[wo + 1], (unsigned long long)(uint32_t)((v << bo) >> 32));
      if (bo) atomicAdd(&limb[wo + 2], (unsigned long long)(uint32_t)(v >> (64 - bo)));
    }
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  // limbs and quotient digits live in LDS: they are indexed with run-time
  // values, which would put a private array in scratch memory
  __shared__ uint32_t w[12], q[12];
  {
    unsigned long long carry = 0;
    for (int k = 0; k < 12; ++k) {
      const unsigned long long t = limb[k] + carry;
      w[k] = (uint32_t)t;
      carry = t >> 32;
    }
  }
  const uint64_t n = (uint64_t)nblocks;
  uint64_t rem = 0;
  // base-2^32 long division by n (n < 2^31, rem < n, so cur < n 2^32 < 2^63
  // and the quotient digit is below 2^32): the fp64 quotient is within one of
  // the digit (cur exact below 2^53; above, n >= 2^21 bounds the error), and
  // an exact integer correction makes it the digit
  for (int k = 11; k >= 0; --k) {
    const uint64_t cur = (rem << 32) | w[k];
    int64_t d = (int64_t)((double)cur / (double)n);
    int64_t r = (int64_t)cur - d * (int64_t)n;
    while (r < 0) {
      --d;
      r += (int64_t)n;
    }
    while (r >= (int64_t)n) {
      ++d;
      r -= (int64_t)n;
    }
    q[k] = (uint32_t)d;
    rem = (uint64_t)r;
  }
  int top = -1;
  for (int k = 11; k >= 0; --k)
    if (q[k]) {
      top = k;
      break;
    }
  if (top < 0) {  // zero sum
    *mu = 0.f;
    return;
  }
  const int L = 32 * top + (32 - __clz(q[top]));
  const int s = max(L - 24, 64);
  // the quotient's bits from bit i up (i >= 0), zero past the top limb
  auto bits_from = [&](int i) -> uint64_t {
    const int wi = i >> 5, bi = i & 31;
    const uint64_t lo = wi < 12 ? q[wi] : 0u, mid = wi + 1 < 12 ? q[wi + 1] : 0u, hi = wi + 2 < 12 ? q[wi + 2] : 0u;
    return ((lo | (mid << 32)) >> bi) | (bi ? hi << (64 - bi) : 0ull);
  };
  uint32_t m = (uint32_t)(bits_from(s) & 0x1FFFFFFull);  // bits s .. s + 24
  const uint32_t guard = (uint32_t)(bits_from(s - 1) & 1ull);
  // sticky: any bit below s - 1, or a nonzero remainder
  const int sb_w = (s - 1) >> 5, sb_b = (s - 1) & 31;
  bool sticky = rem != 0 || (sb_b && (q[sb_w] & ((1u << sb_b) - 1u)) != 0u);
  for (int k = 0; k < sb_w && !sticky; ++k) sticky = q[k] != 0u;
  if (guard && (sticky || (m & 1u))) ++m;
  *mu = __uint_as_float(((uint32_t)(s - 64) << 23) + m);
}

// e4m3 code of the real value v (given as an fp64 quotient of two fp32
// numbers): nearest value, ties to the even mantissa, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne(double v) {
  const uint32_t sign = (__double_as_longlong(v) < 0) ? 0x80u : 0u;
  const double a = fabs(v);
  uint32_t mag;
  if (a >= 448.0) {
    mag = 0x7Eu;
  } else if (a < 0x1p-6) {
    mag = (uint32_t)__builtin_rint(a * 512.0);  // subnormal grid 2^-9; 8 -> smallest normal
  } else {
    const int e = (int)((__double_as_longlong(a) >> 52) & 0x7FF) - 1023;
    const double scaled = a * __longlong_as_double((long long)(1023 + 3 - e) << 52);  // a * 2^(3-e), exact
    mag = (uint32_t)((e + 7) << 3) + ((uint32_t)__builtin_rint(scaled) - 8u);  // carry moves into the exponent
  }
  return sign | mag;
}

__global__ __launch_bounds__(256) void double_quantize(const float *__restrict__ c1, int64_t nblocks,
                                                       const float *__restrict__ mu_p,
                                                       uint8_t *__restrict__ q_out,
                                                       float *__restrict__ s2_out) {
  __shared__ uint32_t wmax[4];
  const int64_t b = (int64_t)blockIdx.x * kGroup + threadIdx.x;
  const float mu = *mu_p;
  const float d = (b < nblocks) ? __fsub_rn(c1[b], mu) : 0.f;
  uint32_t a = __float_as_uint(d) & 0x7FFFFFFFu;
  for (int off = 32; off >= 1; off >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, off, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = a;
  __syncthreads();
  a = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float s2 = __fdiv_rn(__uint_as_float(a), 448.0f);
  if (threadIdx.x == 0) s2_out[blockIdx.x] = s2;
  if (b < nblocks) q_out[b] = (s2 > 0.f) ? (uint8_t)e4m3_rne((double)d / (double)s2) : (uint8_t)0;
}

// Streaming decode of one or several weights in one launch.  Each weight's
// 8-element chunks are grouped in passes of 1024; a workgroup takes one pass at
// a time (grid-stride over the passes of all the weights, a pass never spans
// two weights).  Load j of every lane reads the 4 code bytes of chunk
// base + 256 j + lane, so each load and each 16-byte store instruction of a
// wave covers one contiguous run (256 B of codes, 1 KiB of output); all four
// chunks' codes and constants are loaded before any is decoded.  The output is
// written with non-temporal stores (it is not read back here).  Measured: 6.9
// TB/s for a 22016 x 8192 weight against 5.0 TB/s for one chunk per thread with
// 4-byte loads and ordinary stores.  kDQ is the storage form of every weight
// of the launch (a runtime switch costs a quarter of the throughput); without
// double quantization s2 holds the fp32 block constants (no mean, no FP8).
constexpr int kDeqPass = 1024;  // chunks per pass

template <bool kDQ>
__global__ __launch_bounds__(256) void dequantize_bf16(DequantSet set, int64_t passes, Codebook cb) {
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = cb.v[threadIdx.x];
  __syncthreads();
  // grid-stride over the passes (the workgroups in flight cover one contiguous
  // window of memory); passes only increase, so the weight's pointers and mean
  // are reloaded only when a workgroup crosses into the next weight
  QWeight w = set.w[0];
  uint16_t *out = set.out[0];
  int64_t pass0 = 0, next = -1, numel = 0, nchunks = 0, codes_bytes = 0;
  float mu = 0.f;
  for (int64_t ps = blockIdx.x; ps < passes; ps += gridDim.x) {
    if (ps >= next) {
      int mi = 0;
      for (int i = 1; i < set.count; ++i)
        if (ps >= set.pass0[i]) mi = i;
      w = set.w[mi];
      out = set.out[mi];
      pass0 = set.pass0[mi];
      next = mi + 1 < set.count ? set.pass0[mi + 1] : passes;
      numel = w.n_out * w.n_in;
      nchunks = (numel + 7) >> 3;
      codes_bytes = (numel + 1) >> 1;
      mu = kDQ ? *w.mu : 0.f;
    }
    const int64_t base = (ps - pass0) * kDeqPass;
    uint32_t pk[4];
    float ch[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t c = base + j * 256 + threadIdx.x;
      uint32_t packed = 0x77777777u;
      int64_t blk = 0;
      if (c < nchunks) {
        if ((c << 3) + 8 <= numel) {
          packed = *(const uint32_t *)(w.codes + (c << 2));
        } else {
          for (int i = 0; i < 4; ++i)
            if ((c << 2) + i < codes_bytes)
              packed = (packed & ~(0xFFu << (8 * i))) | ((uint32_t)w.codes[(c << 2) + i] << (8 * i));
        }
        blk = (c << 3) >> 6;
      }
      pk[j] = packed;
      ch[j] = kDQ ? decode_constant(w.fp8[blk], w.s2[blk >> 8], mu) : w.s2[blk];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t c = base + j * 256 + threadIdx.x;
      if (c >= nchunks) continue;
      const int64_t e0 = c << 3;
      u32x4v o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = decode_product(lut[(pk[j] >> (8 * i)) & 15u], ch[j]);
        const float hi = decode_product(lut[(pk[j] >> (8 * i + 4)) & 15u], ch[j]);
        o[i] = pack_bf16x2(lo, hi);
      }
      if (e0 + 8 <= numel) {
        __builtin_nontemporal_store(o, (u32x4v *)(out + e0));
      } else {
        for (int i = 0; i < 8; ++i)
          if (e0 + i < numel) out[e0 + i] = (uint16_t)(o[i >> 1] >> (16 * (i & 1)));
      }
    }
  }
}

static inline int grid_for(int64_t items, int64_t per_wg, int64_t cap) {
  int64_t g = (items + per_wg - 1) / per_wg;
  if (g > cap) g = cap;
  return (int)(g < 1 ? 1 : g);
}

hipError_t launch_quantize(const void *w, bool bf16_src, bool dq, int64_t numel, uint8_t *codes, uint8_t *fp8,
                           float *s2, float *mu, uint32_t *status, unsigned long long *bins, float *c1,
                           const Midpoints &mid, hipStream_t st) {
  const int64_t nblocks = (numel + kBlock - 1) / kBlock;
  const int64_t ngroups = (nblocks + kGroup - 1) / kGroup;
  const int64_t codes_bytes = (numel + 1) / 2;
  // status word + padding (64 words) followed by the bin copies
  const int words = 64 + (int)(kQuantizeBinBytes / 4);
  zero_words<<<(words + 255) / 256, 256, 0, st>>>(status, words);
  const int g = grid_for(nblocks, 32, 8192);
  if (bf16_src)
    quantize_blocks<true><<<g, 256, 0, st>>>(w, numel, nblocks, codes, codes_bytes, c1, bins, status, mid);
  else
    quantize_blocks<false><<<g, 256, 0, st>>>(w, numel, nblocks, codes, codes_bytes, c1, bins, status, mid);
  if (dq) {
    mean_from_bins<<<1, 256, 0, st>>>(bins, nblocks, mu);
    double_quantize<<<(unsigned)ngroups, 256, 0, st>>>(c1, nblocks, mu, fp8, s2);
  }
  return hipGetLastError();
}

// One launch per storage form present in the set.
static hipError_t launch_dequantize_form(const DequantSet &set_in, bool dq, const Codebook &cb, hipStream_t st) {
  DequantSet set{};
  for (int i = 0; i < set_in.count; ++i)
    if (set_in.w[i].dq == dq) {
      set.w[set.count] = set_in.w[i];
      set.out[set.count] = set_in.out[i];
      ++set.count;
    }
  if (set.count == 0) return hipSuccess;
  int64_t passes = 0;
  for (int i = 0; i < set.count; ++i) {
    set.pass0[i] = passes;
    const int64_t nchunks = (set.w[i].n_out * set.w[i].n_in + 7) / 8;
    passes += (nchunks + kDeqPass - 1) / kDeqPass;
  }
  for (int i = set.count; i < kMaxDequantSet; ++i) {
    set.w[i] = set.w[0];
    set.out[i] = set.out[0];
    set.pass0[i] = passes;
  }
  const int g = (int)std::min<int64_t>(passes, 8192);
  if (dq)
    dequantize_bf16<true><<<g, 256, 0, st>>>(set, passes, cb);
  else
    dequantize_bf16<false><<<g, 256, 0, st>>>(set, passes, cb);
  return hipGetLastError();
}

hipError_t launch_dequantize_set(const DequantSet &set, const Codebook &cb, hipStream_t st) {
  if (set.count < 1 || set.count > kMaxDequantSet) return hipErrorInvalidValue;
  const hipError_t e = launch_dequantize_form(set, true, cb, st);
  return e != hipSuccess ? e : launch_dequantize_form(set, false, cb, st);
}

hipError_t launch_dequantize(const QWeight &w, uint16_t *out, const Codebook &cb, hipStream_t st) {
  DequantSet s{};
  s.count = 1;
  s.w[0] = w;
  s.out[0] = out;
  return launch_dequantize_set(s, cb, st);
}

}  // namespace qlora
