// Device helpers for the low part of X with bf16 compute (the format is
// described beside lo_index() in muon_internal.h): 16 residuals of one
// lane's block as int8 codes times a shared power-of-two step.
#pragma once

#include "muon_internal.h"

namespace muon {

// The step 2^(E - 142) and its inverse 2^(142 - E) as floats, both exact;
// 0 when E < 16.
__device__ __forceinline__ float lo8_step(uint32_t e) {
  return e >= 16 ? __builtin_bit_cast(float, (e - 15u) << 23) : 0.0f;
}
__device__ __forceinline__ float lo8_inv_step(uint32_t e) {
  return e >= 16 ? __builtin_bit_cast(float, (269u - e) << 23) : 0.0f;
}

// bf16(x), rounded to nearest even, as a float
__device__ __forceinline__ float lo8_high(float x) { return static_cast<float>(static_cast<__bf16>(x)); }

typedef __bf16 lo8_bf16x2 __attribute__((ext_vector_type(2)));
typedef float lo8_f32x2 __attribute__((ext_vector_type(2)));
// bf16(lo) in the low half and bf16(hi) in the high half of a word, both
// rounded to nearest even by one packed conversion (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((lo8_f32x2){lo, hi}, lo8_bf16x2));
}

// Codes of x[r] - bf16(x[r]), r = 0..15, packed four to a word (code r in
// byte r % 4 of word r / 4), and the shared exponent.  The subtraction and
// the scaling are exact; the code is rounded to nearest, ties to even.
//   * The shared exponent is the largest exponent field of the bf16(x[r]).
//     Rounding to bf16 is monotonic in |x|, so it is the exponent field of
//     bf16(max |x[r]|): one conversion per block instead of sixteen.
//   * bf16 values are made two at a time (one packed conversion per pair).
//   * Rounding to an integer: adding 1.5 * 2^23 to a value in [-128, 128]
//     leaves it in [2^23, 2^24), where the spacing of floats is 1, so the
//     fused multiply-add rounds the scaled residual to the nearest integer
//     (ties to even, as rintf) and the sum's low byte is the code in two's
//     complement.  A clamp to 1.5 * 2^23 +- 127 keeps the code in [-127, 127].
struct Lo8 {
  uint32_t w[4];
  uint32_t e;
};
// With hi given, hi[k] receives bf16(x[2k]) | bf16(x[2k+1]) << 16 as well.
__device__ __forceinline__ Lo8 lo8_encode(const float* x, uint32_t* hi = nullptr) {
  Lo8 o;
  float m = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(x[r]));
  o.e = (__builtin_bit_cast(uint32_t, lo8_high(m)) >> 23) & 0xffu;
  const float inv = lo8_inv_step(o.e);
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
  uint32_t b[16];
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const uint32_t hb = bf16_pair(x[r], x[r + 1]);
    if (hi != nullptr) hi[r / 2] = hb;
    const float h0 = __builtin_bit_cast(float, hb << 16);
    const float h1 = __builtin_bit_cast(float, hb & 0xffff0000u);
    const float t0 = fminf(fmaxf(fmaf(x[r] - h0, inv, kMagic), kMagic - 127.0f), kMagic + 127.0f);
    const float t1 = fminf(fmaxf(fmaf(x[r + 1] - h1, inv, kMagic), kMagic - 127.0f), kMagic + 127.0f);
    b[r] = __builtin_bit_cast(uint32_t, t0);
    b[r + 1] = __builtin_bit_cast(uint32_t, t1);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o.w[k] = (b[4 * k] & 0xffu) | ((b[4 * k + 1] & 0xffu) << 8) | ((b[4 * k + 2] & 0xffu) << 16) | (b[4 * k + 3] << 24);
  return o;
}

// Code r of a lane's block (its residual is the code times the step).
__device__ __forceinline__ float lo8_code(const uint32_t* w, int r) {
  return static_cast<float>(static_cast<int8_t>((w[r >> 2] >> (8 * (r & 3))) & 0xffu));
}

}  // namespace muon
