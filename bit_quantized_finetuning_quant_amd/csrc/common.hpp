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

// e4m3 ("fn") byte -> its exact value (bias 7, 3 mantissa bits, exponent
// field 0 = subnormal m * 2^-9; 0x7F and 0xFF are NaN, which stored data
// never holds).  gfx950's v_cvt_f32_fp8 reads the OCP e4m3 format; every
// e4m3 value is an fp32 value, so the conversion is exact.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }

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

// Decode without a memory lookup.  The 16 decoded values of one block,
// t[k] = bf16_rne(fl32(CB[k] * c1hat)), are held in registers as byte
// tables: lo[j] holds the low bytes of t[4j .. 4j+3], hi[j] the high bytes.
// A code then selects its two bytes with v_perm_b32 (which picks bytes 0..7
// of the 64-bit pair {S0, S1}, S1 the low word): one permute over each half
// of a table and a per-byte select on the code's bit 3.  Every decoded value
// is computed exactly as in the lookup form, so the two are bit-identical.
struct DecodeTable {
  uint32_t lo[4], hi[4];
};

// lo[j] and hi[j] of 8 consecutive levels from their 4 packed bf16 pairs
// p[m] = t[2m] | t[2m+1] << 16.
__device__ __forceinline__ void table_half(const uint32_t (&p)[4], uint32_t (&lo)[2], uint32_t (&hi)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    lo[j] = __builtin_amdgcn_perm(p[2 * j + 1], p[2 * j], 0x06040200u);
    hi[j] = __builtin_amdgcn_perm(p[2 * j + 1], p[2 * j], 0x07050301u);
  }
}

// Byte b of the result is byte (code_b) of a 16-byte table, for four codes
// given as the bytes of sel (low 3 bits) and mask (0xFF where the code's bit 3
// is set).
__device__ __forceinline__ uint32_t table_bytes(const uint32_t (&tb)[4], uint32_t sel, uint32_t mask) {
  const uint32_t a = __builtin_amdgcn_perm(tb[1], tb[0], sel), b = __builtin_amdgcn_perm(tb[3], tb[2], sel);
  return (b & mask) | (a & ~mask);
}

// One word of 8 codes (low nibble first) -> 4 words of bf16 pairs; word d
// holds element 2d in its low half and element 2d + 1 in its high half.
__device__ __forceinline__ void decode_word(uint32_t c, const DecodeTable &t, uint32_t (&o)[4]) {
  const uint32_t c4 = c >> 4;
  // bytes of c: even codes n0, n2, n4, n6 in bits 0..3; bytes of c4: odd codes
  const uint32_t se = c & 0x07070707u, so = c4 & 0x07070707u;
  // 0xFF in byte b where bit 3 of code b is set: v_perm selectors 8..11 give 0xFF or 0x00 from the
  // top bit of bytes 1, 3, 5, 7 of {S0, S1}; the shifts bring bit 3 (even codes) or bit 7 (odd
  // codes) of byte b there
  const uint32_t me = __builtin_amdgcn_perm(c << 4, c << 12, 0x0B090A08u);
  const uint32_t mo = __builtin_amdgcn_perm(c, c << 8, 0x0B090A08u);
  const uint32_t le = table_bytes(t.lo, se, me), he = table_bytes(t.hi, se, me);
  const uint32_t lq = table_bytes(t.lo, so, mo), hq = table_bytes(t.hi, so, mo);
  const uint32_t x0 = __builtin_amdgcn_perm(he, le, 0x05010400u);  // t[n0] | t[n2] << 16
  const uint32_t y0 = __builtin_amdgcn_perm(hq, lq, 0x05010400u);  // t[n1] | t[n3] << 16
  const uint32_t x1 = __builtin_amdgcn_perm(he, le, 0x07030602u);  // t[n4] | t[n6] << 16
  const uint32_t y1 = __builtin_amdgcn_perm(hq, lq, 0x07030602u);  // t[n5] | t[n7] << 16
  o[0] = __builtin_amdgcn_perm(y0, x0, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(y0, x0, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(y1, x1, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(y1, x1, 0x07060302u);
}

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace qlora
