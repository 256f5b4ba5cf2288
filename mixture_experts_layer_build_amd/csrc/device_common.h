// Device-side helpers: bf16 conversion, MXFP8 (E4M3 + E8M0) encoding,
// MFMA vector types. Included by the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mok {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;

__host__ __device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__host__ __device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

__host__ __device__ __forceinline__ float bf16_to_f32(uint16_t b) { return u2f((uint32_t)b << 16); }

typedef __attribute__((ext_vector_type(2))) float f32x2v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;

// fp32 -> bf16 bits, round to nearest even. On the device this is gfx950's
// packed conversion instruction (v_cvt_pk_bf16_f32): compared on the GPU
// with the integer rounding of the host path over 1.4e8 bit patterns of
// every exponent, it gave the same bits for every finite input, subnormals
// included; only NaN payloads may differ (both stay NaN). The integer form
// costs a divergent branch per value.
__host__ __device__ __forceinline__ uint16_t f32_to_bf16(float f) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(uint16_t, (__bf16)f);
#else
  uint32_t u = f2u(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
#endif
}

__host__ __device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){lo, hi}, bf16x2v));
#else
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
#endif
}

// floor(log2 |v|) of a non-zero fp32 magnitude given by its bits (sign clear),
// exact, subnormals included.
__host__ __device__ __forceinline__ int floor_log2_bits(uint32_t mag) {
  int ef = (int)(mag >> 23);
  if (ef > 0) return ef - 127;
  return (31 - __builtin_clz(mag)) - 149;  // mantissa only: value = m * 2^-149
}

// MXFP8 block exponent X from the block's largest magnitude (fp32 bits, sign
// clear): clamp(floor(log2 amax) - 8, -127, 127); -127 for amax == 0.
__host__ __device__ __forceinline__ int mx_block_exponent(uint32_t amax_bits) {
  if (amax_bits == 0) return -127;
  int x = floor_log2_bits(amax_bits) - 8;
  return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// E4M3 ("FN": bias 7, no infinity, 0x7F NaN, max 448) code of v / 2^X,
// rounded to nearest even on the E4M3 grid, magnitudes above 448
// saturating to 0x7E, sign kept. Integer arithmetic on the fp32 bits, so
// the result is exact for every finite input (no flush of subnormals).
__host__ __device__ __forceinline__ uint32_t e4m3_encode_scaled(float v, int X) {
  uint32_t u = f2u(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t mag = u & 0x7FFFFFFFu;
  if (mag == 0) return sign;
  int ef = (int)(mag >> 23);
  uint32_t S;   // integer significand
  int e2;       // |v| = S * 2^e2
  if (ef > 0) {
    S = (mag & 0x7FFFFFu) | 0x800000u;
    e2 = ef - 150;
  } else {
    S = mag;
    e2 = -149;
  }
  int L = floor_log2_bits(mag) - X;              // floor(log2 |v / 2^X|)
  int qe = (L < -6 ? -6 : L) - 3;                // exponent of one grid step at that binade
  int sh = qe - (e2 - X);                        // right shift that maps S onto grid steps
  uint32_t n;
  if (sh <= 0) {
    n = S << (-sh);                              // exact (only tiny shifts occur: |v/2^X| < 2^9)
  } else if (sh > 25) {
    n = 0;
  } else {
    n = S >> sh;
    uint32_t rem = S & ((1u << sh) - 1u);
    uint32_t half = 1u << (sh - 1);
    if (rem > half || (rem == half && (n & 1u))) n += 1u;
  }
  uint32_t code;
  if (L < -6) {
    code = n;                                    // subnormal steps of 2^-9; n == 8 is 0x08 = 2^-6
  } else {
    code = (uint32_t)((L + 7) << 3) + n - 8u;    // n == 16 carries into the next binade
  }
  if (code > 0x7Eu) code = 0x7Eu;
  return code | sign;
}

#if defined(__HIP_DEVICE_COMPILE__)
// E4M3 codes of v0..v3 / 2^X, byte i = code of v_i, with exactly the
// rounding and saturation of e4m3_encode_scaled, on the scaled conversion
// instruction of gfx950 (two codes per instruction). The instruction divides
// by its scale operand and rounds to nearest even, but turns magnitudes
// above the E4M3 range into NaN, so each input is first clamped to
// +-448 * 2^X (everything up to the 464 tie rounds to 448 anyway). Checked
// bit for bit against e4m3_encode_scaled over every block exponent,
// rounding ties, subnormals, signed zeros and the saturation band.
__device__ __forceinline__ uint32_t e4m3x4_encode_scaled(float v0, float v1, float v2, float v3, int X) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  const float s = __builtin_ldexpf(1.0f, X);
  const float lim = __builtin_ldexpf(448.0f, X);
  v0 = __builtin_fminf(__builtin_fmaxf(v0, -lim), lim);
  v1 = __builtin_fminf(__builtin_fmaxf(v1, -lim), lim);
  v2 = __builtin_fminf(__builtin_fmaxf(v2, -lim), lim);
  v3 = __builtin_fminf(__builtin_fmaxf(v3, -lim), lim);
  s16x2 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, v0, v1, s, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, v2, v3, s, true);
  return (uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16);
}
#else
__device__ uint32_t e4m3x4_encode_scaled(float v0, float v1, float v2, float v3, int X);  // device only
#endif

#if defined(__HIP_DEVICE_COMPILE__)
// Value of byte b (0-3, a constant after unrolling) of `word` as an E4M3
// code, times `scale` = 2^X, on gfx950's scaled conversion instruction (one
// value per instruction). Compared on the GPU with e4m3_decode_scaled below
// for every code but the two NaN codes (which the encoder never writes),
// every X in [-127, 127] and every byte position: identical bits.
__device__ __forceinline__ float e4m3_decode_byte_scaled(uint32_t word, int b, float scale) {
  switch (b) {
    case 0: return __builtin_amdgcn_cvt_scalef32_f32_fp8((int)word, scale, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_f32_fp8((int)word, scale, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_f32_fp8((int)word, scale, 2);
    default: return __builtin_amdgcn_cvt_scalef32_f32_fp8((int)word, scale, 3);
  }
}
#else
__device__ float e4m3_decode_byte_scaled(uint32_t word, int b, float scale);  // device only
#endif

// Value of E4M3 code `code` (low 8 bits) times 2^X: a 4-bit significand
// scaled by a power of two, so the fp32 result is exact (subnormals too).
__host__ __device__ __forceinline__ float e4m3_decode_scaled(uint32_t code, int X) {
  // subnormal codes (e == 0) are m * 2^(1 - 10 + X), normal ones (8 + m) *
  // 2^(e - 10 + X): integer selects and one ldexp, no branch
  const uint32_t e = (code >> 3) & 15u, m = code & 7u;
  const uint32_t sig = m | (e != 0 ? 8u : 0u);
  const int ex = (e != 0 ? (int)e : 1) - 10 + X;
  const float mag = __builtin_ldexpf((float)sig, ex);
  return (code & 0x80u) ? -mag : mag;
}

typedef unsigned int u32x4 __attribute__((vector_size(16)));

// Raw buffer resource over [base, base + bytes): loads at offsets at or past
// `bytes` return zeros. Word 3 selects 32-bit data format (gfx9 family).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Wave-wide helpers (wave64).
__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

}  // namespace mok
