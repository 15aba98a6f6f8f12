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

// Codes of x[r] - bf16(x[r]), r = 0..15, packed four to a word (code r in
// byte r % 4 of word r / 4), and the shared exponent.  The subtraction and
// the scaling are exact; the code is rounded to nearest.
struct Lo8 {
  uint32_t w[4];
  uint32_t e;
};
__device__ __forceinline__ Lo8 lo8_encode(const float* x) {
  Lo8 o;
  o.e = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t e = (__builtin_bit_cast(uint32_t, lo8_high(x[r])) >> 23) & 0xffu;
    o.e = e > o.e ? e : o.e;
  }
  const float inv = lo8_inv_step(o.e);
#pragma unroll
  for (int k = 0; k < 4; ++k) o.w[k] = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float q = __builtin_rintf((x[r] - lo8_high(x[r])) * inv);
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    o.w[r >> 2] |= (static_cast<uint32_t>(static_cast<int32_t>(q)) & 0xffu) << (8 * (r & 3));
  }
  return o;
}

// Residual r of a lane's block from its four code words and step.
__device__ __forceinline__ float lo8_decode(const uint32_t* w, int r, float step) {
  return static_cast<float>(static_cast<int8_t>((w[r >> 2] >> (8 * (r & 3))) & 0xffu)) * step;
}

}  // namespace muon
