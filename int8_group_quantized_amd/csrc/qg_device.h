// Device-side helpers shared by the gfx950 kernels: vector types, 16-bit
// float conversions, and the register-level expansion of packed codes into
// exact bf16 integers (dequantization with the scale left for later, so every
// product of an activation and a code is exact).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qg_internal.h"

namespace qg {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;


__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

__device__ __forceinline__ float scale_to_f32(uint32_t b, bool s_bf16) {
  return s_bf16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

// fp32 -> bf16 / fp16 with round-to-nearest-even (the hardware default mode).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Fixed-grid quantizer for one weight: clamp(rne(w / s), lo, hi) with IEEE
// division; s == 0 and NaN quotients give 0, infinite quotients saturate.
__device__ __forceinline__ int quantize_to_grid(float w, float s, float lo, float hi) {
  if (s == 0.0f) return 0;
  const float t = w / s;
  if (t != t) return 0;
  return (int)fminf(fmaxf(__builtin_rintf(t), lo), hi);
}

// One 32-bit word of INT4 codes (eight offset-binary nibbles, nibble p at bits
// 4p, holding elements i = p/2 + 4*(p%2) ... i.e. nibbles 0..3 are the even
// elements and 4..7 the odd ones) -> eight bf16 values 128 + u, element order.
// OR-ing a nibble into the mantissa of 128.0 (0x4300) gives 128 + u exactly;
// the constant offset 136 = 128 + 8 is removed after the product (see the
// GEMM kernels), which keeps this expansion at one or two ALU ops per pair.
__device__ __forceinline__ bf16x8 int4_word_to_biased_bf16(uint32_t w) {
  u32x4 r;
  r[0] = (w & 0x000F000Fu) | 0x43004300u;
  r[1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
  r[2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
  r[3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
  return __builtin_bit_cast(bf16x8, r);
}

// The bias 136 = 128 + 8 in all eight lanes of a B operand (bf16 0x4308).
__device__ __forceinline__ bf16x8 bias136_bf16x8() {
  u32x4 r = {0x43084308u, 0x43084308u, 0x43084308u, 0x43084308u};
  return __builtin_bit_cast(bf16x8, r);
}

// Sign-extended byte e of w as fp32 (one byte-select convert instruction).
__device__ __forceinline__ float sbyte_to_f32(uint32_t w, int e) {
  return (float)((int)(w << (24 - 8 * e)) >> 24);
}

// Two fp32 values -> one word of two bf16 (RNE; exact for small integers).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Two 32-bit words of INT8 codes (bytes = elements 0..7, two's complement)
// -> eight exact bf16 integers: eight byte-select converts and four pair
// packs (exact, |q| <= 128).
__device__ __forceinline__ bf16x8 int8_words_to_bf16(uint32_t lo, uint32_t hi) {
  const u32x4 r = {pack_bf16x2(sbyte_to_f32(lo, 0), sbyte_to_f32(lo, 1)),
                   pack_bf16x2(sbyte_to_f32(lo, 2), sbyte_to_f32(lo, 3)),
                   pack_bf16x2(sbyte_to_f32(hi, 0), sbyte_to_f32(hi, 1)),
                   pack_bf16x2(sbyte_to_f32(hi, 2), sbyte_to_f32(hi, 3))};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;

// Activation precision of the GEMM kernels: operands travel as raw 32-bit
// words (two 16-bit values each) and these traits give the matching matrix
// instruction, the INT4 expansion constant (the smallest value of the format
// whose unit in the last place is 1: bf16 128, fp16 1024, so OR-ing a nibble
// u into its mantissa gives magic + u exactly), the offset magic + 8 that the
// expanded codes carry, the exact pair conversion of INT8 codes, and the RNE
// output conversion.
template <bool XH>
struct Act;

template <>
struct Act<false> {   // bf16 activations and output
  static constexpr uint32_t kMagic = 0x43004300u;    // two bf16 128.0
  static constexpr uint32_t kOffset = 0x43084308u;   // two bf16 136.0
  static __device__ __forceinline__ f32x4 mma(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // 32x32x16: lane L holds row / column L % 32, K slice 8 (L / 32) .. +7.
  static __device__ __forceinline__ f32x16 mma32(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }
  static __device__ __forceinline__ uint16_t out(float f) { return f32_to_bf16_bits(f); }
};

template <>
struct Act<true> {    // fp16 activations and output
  static constexpr uint32_t kMagic = 0x64006400u;    // two fp16 1024.0
  static constexpr uint32_t kOffset = 0x64086408u;   // two fp16 1032.0
  static __device__ __forceinline__ f32x4 mma(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mma32(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // Round-toward-zero pair conversion: exact for the integer codes.
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
  }
  static __device__ __forceinline__ uint16_t out(float f) { return f32_to_f16_bits(f); }
};

// Two words of INT8 codes -> eight exact 16-bit integers in the format of A.
template <class A>
__device__ __forceinline__ u32x4 int8_words_to_act(uint32_t lo, uint32_t hi) {
  return u32x4{A::pack2(sbyte_to_f32(lo, 0), sbyte_to_f32(lo, 1)),
               A::pack2(sbyte_to_f32(lo, 2), sbyte_to_f32(lo, 3)),
               A::pack2(sbyte_to_f32(hi, 0), sbyte_to_f32(hi, 1)),
               A::pack2(sbyte_to_f32(hi, 2), sbyte_to_f32(hi, 3))};
}

// One word of INT4 codes -> eight values magic + u (element order), with the
// magic held in a vector register by the caller (see the GEMM kernels).
__device__ __forceinline__ u32x4 int4_word_to_act(uint32_t w, uint32_t magic) {
  return u32x4{(w & 0x000F000Fu) | magic, ((w >> 4) & 0x000F000Fu) | magic,
               ((w >> 8) & 0x000F000Fu) | magic, ((w >> 12) & 0x000F000Fu) | magic};
}

}  // namespace qg
