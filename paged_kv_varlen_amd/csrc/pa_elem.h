// The element type of the operator's data tensors (query, key, value, the two
// caches and the output) as the kernels use it: fp16 or bf16, both 16 bits,
// chosen at compile time.  The caches are copied bit for bit whatever the
// type; only the matrix products, the rounding of the softmax weights P and of
// the output, and the row sum of the rounded weights depend on it.
//
// The model card ("com.microsoft.PagedAttention", Type constraints) names
// fp16; the Qwen3.8 export issue ("Add Qwen3.8 packed hybrid PagedAttention
// export for ORT GenAI Engine", Phase 1 scope) targets fp16 and bf16, and the
// "WS2 CP-Aware Attention Contract" example (Qwen3-8B TP=2 CP=2) runs in bf16.
// Both types accumulate in fp32 and round once at the final write (WS2,
// Reduction Semantics).  With INT8 and INT4 caches the matrix products take
// the codes converted to the data type (exact: |code| <= 127).
#pragma once

#include <stdint.h>

namespace pa {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <bool BF16>
struct Elem;

template <>
struct Elem<false> {  // IEEE binary16
  typedef _Float16 T;
  typedef _Float16 x8 __attribute__((ext_vector_type(8)));
  typedef _Float16 x4 __attribute__((ext_vector_type(4)));
  typedef _Float16 x2 __attribute__((ext_vector_type(2)));
  static __device__ inline f32x16_t mfma_32x32x16(x8 a, x8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ inline f32x4_t mfma_16x16x32(x8 a, x8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ inline f32x4_t mfma_16x16x16(x4 a, x4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  // c + a.x + a.y, the two values exactly as rounded (v_dot2 with (1, 1))
  static __device__ inline float sum2(x2 a, float c) {
    const x2 one = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
    return __builtin_amdgcn_fdot2(a, one, c, false);
  }
  static __device__ inline T round(float x) { return static_cast<_Float16>(x); }
  static __device__ inline uint16_t bits(float x) { return __builtin_bit_cast(uint16_t, round(x)); }
  static __device__ inline float value(uint16_t b) { return static_cast<float>(__builtin_bit_cast(_Float16, b)); }
  // eight int8 codes (byte k of {w0, w1} is code k) as values, exactly: the
  // byte u = code + 128 becomes the low mantissa byte of the half 1024 + u
  // (v_perm_b32 puts it beside the high byte 0x64), and 1152 is subtracted
  static __device__ inline x8 from_codes(uint32_t w0, uint32_t w1) {
    const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
    const uint32_t h[4] = {__builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u),
                           __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u),
                           __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u),
                           __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)};
    const x2 bias = {static_cast<_Float16>(1152.f), static_cast<_Float16>(1152.f)};
    x8 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const x2 v = __builtin_bit_cast(x2, h[k]) - bias;
      r[2 * k] = v[0];
      r[2 * k + 1] = v[1];
    }
    return r;
  }
  // int4 codes as values: a 4-bit two's complement code c, its top bit
  // flipped, is c + 8 in [0, 15]; placed under the exponent of 1024 it gives
  // the half 1024 + c + 8, and 1032 is subtracted (exact)
  static __device__ inline x2 minus_1032(uint32_t h) {
    const x2 bias = {static_cast<_Float16>(1032.f), static_cast<_Float16>(1032.f)};
    return __builtin_bit_cast(x2, h | 0x64006400u) - bias;
  }
  // eight int4 codes (nibble e of w is code e) as values: the even codes (low
  // nibbles) and odd ones (high nibbles) of each byte are paired by v_perm_b32
  static __device__ inline x8 from_nibbles8(uint32_t w) {
    const uint32_t u = w ^ 0x88888888u;
    const uint32_t lo = u & 0x0F0F0F0Fu, hi = (u >> 4) & 0x0F0F0F0Fu;
    const uint32_t h[4] = {__builtin_amdgcn_perm(hi, lo, 0x0c040c00u), __builtin_amdgcn_perm(hi, lo, 0x0c050c01u),
                           __builtin_amdgcn_perm(hi, lo, 0x0c060c02u), __builtin_amdgcn_perm(hi, lo, 0x0c070c03u)};
    x8 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const x2 v = minus_1032(h[k]);
      r[2 * k] = v[0];
      r[2 * k + 1] = v[1];
    }
    return r;
  }
  // the same eight codes in the order 0, 2, 1, 3, 4, 6, 5, 7: v_perm_b32 places
  // each low or high nibble (code + 8) straight under the exponent byte of
  // 1024, so no OR is needed
  static __device__ inline x8 from_nibbles8_swapped(uint32_t w) {
    const uint32_t u = w ^ 0x88888888u;
    const uint32_t lo = u & 0x0F0F0F0Fu, hi = (u >> 4) & 0x0F0F0F0Fu;
    const uint32_t h[4] = {__builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u),   // codes 0, 2
                           __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u),   // codes 1, 3
                           __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u),   // codes 4, 6
                           __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u)};  // codes 5, 7
    const x2 bias = {static_cast<_Float16>(1032.f), static_cast<_Float16>(1032.f)};
    x8 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const x2 v = __builtin_bit_cast(x2, h[k]) - bias;
      r[2 * k] = v[0];
      r[2 * k + 1] = v[1];
    }
    return r;
  }
};

template <>
struct Elem<true> {  // bfloat16: the upper half of a binary32
  typedef __bf16 T;
  typedef __bf16 x8 __attribute__((ext_vector_type(8)));
  typedef __bf16 x4 __attribute__((ext_vector_type(4)));
  typedef __bf16 x2 __attribute__((ext_vector_type(2)));
  typedef short s4 __attribute__((ext_vector_type(4)));
  static __device__ inline f32x16_t mfma_32x32x16(x8 a, x8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ inline f32x4_t mfma_16x16x32(x8 a, x8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ inline f32x4_t mfma_16x16x16(x4 a, x4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b), c, 0, 0,
                                                     0);
  }
  static __device__ inline float sum2(x2 a, float c) {
    const x2 one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
    return __builtin_amdgcn_fdot2_f32_bf16(a, one, c, false);
  }
  // round to nearest, ties to even (v_cvt_pk_bf16_f32)
  static __device__ inline T round(float x) { return static_cast<__bf16>(x); }
  static __device__ inline uint16_t bits(float x) { return __builtin_bit_cast(uint16_t, round(x)); }
  static __device__ inline float value(uint16_t b) { return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16); }
  // eight int8 codes (byte k of {w0, w1} is code k) as values, exactly
  // (integers up to 127 in magnitude fit the 8-bit significand)
  static __device__ inline x8 from_codes(uint32_t w0, uint32_t w1) {
    x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      r[e] = static_cast<__bf16>(static_cast<float>(static_cast<int8_t>((e < 4 ? w0 : w1) >> (8 * (e & 3)))));
    return r;
  }
  // eight int4 codes (nibble e of w is code e) as values
  static __device__ inline x8 from_nibbles8(uint32_t w) {
    x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      r[e] = static_cast<__bf16>(static_cast<float>(static_cast<int>(w << (28 - 4 * e)) >> 28));
    return r;
  }
  // the same eight codes in the order 0, 2, 1, 3, 4, 6, 5, 7
  static __device__ inline x8 from_nibbles8_swapped(uint32_t w) {
    constexpr int kCode[8] = {0, 2, 1, 3, 4, 6, 5, 7};
    x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      r[e] = static_cast<__bf16>(static_cast<float>(static_cast<int>(w << (28 - 4 * kCode[e])) >> 28));
    return r;
  }
};

}  // namespace pa
