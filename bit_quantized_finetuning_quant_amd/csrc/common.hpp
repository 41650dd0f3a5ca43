// Shared device helpers of the gfx950 QLoRA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

constexpr int kBlock = 64;   // elements per NF4 block (one absmax constant each)
constexpr int kGroup = 256;  // block constants per FP8 double-quantization group
constexpr uint32_t kZeroCode = 7;

// Kernel-argument copy of the 16 NF4 levels (held in SGPRs by the kernels that
// take it, copied to LDS where a per-lane lookup is needed).
struct Codebook {
  float v[16];
};

// Exact midpoints between adjacent NF4 levels (each needs at most 26
// significant bits, so it is exact in fp64).  Used by the quantizer to build
// its per-block thresholds.
struct Midpoints {
  double m[15];
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// e4m3 ("fn") byte -> its exact value: bias 7, 3 mantissa bits, exponent
// field 0 = subnormal m * 2^-9.  NaN patterns never occur in stored data.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  // Branch-free: both the normal and the subnormal encodings are formed and
  // one is selected, and the sign is OR-ed in (a divergent branch here would
  // make the compiler drain outstanding loads at the join).
  const uint32_t e = (b >> 3) & 0xFu;
  const uint32_t m = b & 7u;
  const uint32_t normal = ((e + 120u) << 23) | (m << 20);
  const uint32_t subnormal = __float_as_uint((float)m * 0x1p-9f);  // exact
  const uint32_t mag = e ? normal : subnormal;
  return __uint_as_float(mag | ((b & 0x80u) << 24));
}

// Block constant decode: fl32(fl32(e4m3(q) * s2) + mu), two roundings.  The
// multiply and the add must not be contracted into one fused multiply-add
// (HIP's __fmul_rn / __fadd_rn are plain operators, so the pragma is what
// keeps them apart; the library is also built with -ffp-contract=off).
__device__ __forceinline__ float decode_constant(uint32_t q, float s2, float mu) {
#pragma clang fp contract(off)
  const float p = e4m3_to_f32(q) * s2;
  return p + mu;
}

// One decoded weight before the bf16 rounding: fl32(CB[code] * c1hat).
__device__ __forceinline__ float decode_product(float level, float c1hat) {
#pragma clang fp contract(off)
  return level * c1hat;
}

// Two fp32 -> packed bf16 pair (round to nearest even; gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace qlora
