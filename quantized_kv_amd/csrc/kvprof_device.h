// Device-side helpers shared by the HIP translation units of libkvprof (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvp {

constexpr double kInvSqrt128 = 0x1.6a09e667f3bccp-4;  // float64 nearest to 1/sqrt(128)

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// E8M0 exponent of a block: the smallest e with amax <= 448 * 2^e. Writing amax = mu * 2^E with
// mu in [1, 2), 448 = 1.75 * 2^8 gives e = E - 8 when mu <= 1.75 and E - 7 otherwise.
__device__ __forceinline__ int e8m0_exp(float amax) {
  if (!(amax > 0.f)) return -127;
  int E;
  double mu = frexp((double)amax, &E);  // amax = mu * 2^E, mu in [0.5, 1)
  mu *= 2.0;
  E -= 1;
  int e = (mu <= 1.75) ? E - 8 : E - 7;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// float32 -> E4M3FN byte with round-to-nearest-even on the bit pattern. |v| <= 448 by construction
// of the block exponent; the sign of zero is kept.
__device__ __forceinline__ uint8_t e4m3_rne(float v) {
  uint32_t bits = __float_as_uint(v);
  uint8_t sign = (bits >> 24) & 0x80;
  float a = fabsf(v);
  if (a < 0x1p-6f) {  // subnormal grid m * 2^-9
    int n = (int)__builtin_rintf(a * 512.f);
    return sign | (n >= 8 ? 0x08 : (uint8_t)n);
  }
  uint32_t ab = __float_as_uint(a);
  int E = int((ab >> 23) & 0xFF) - 127;
  uint32_t m = ab & 0x7FFFFF;
  uint32_t keep = m >> 20, rem = m & 0xFFFFF;
  if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) keep++;
  if (keep == 8) { keep = 0; E++; }
  return sign | (uint8_t)(((E + 7) << 3) | keep);
}

__device__ __forceinline__ float e4m3_value(uint8_t c) {
  int e = (c >> 3) & 0xF, m = c & 7;
  float a = (e == 0) ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
  return (c & 0x80) ? -a : a;
}

// The value e4m3_value(e4m3_rne(v)) for |v| <= 448, without branches: in the normal range the
// float32 mantissa is rounded to 3 bits on the bit pattern (round to nearest even; a carry moves into
// the exponent), below 2^-6 onto the subnormal grid m 2^-9. Equal to the encode-decode pair for every
// float32 in range (an exhaustive comparison on the host; tests/test_e4m3_rounding.py compares the same
// form with the oracle's E4M3 rounding at every tie and carry boundary).
__device__ __forceinline__ float e4m3_grid(float v) {
  const float a = fabsf(v);
  const uint32_t ab = __float_as_uint(a);
  const float nrm = __uint_as_float((ab + 0x7FFFFu + ((ab >> 20) & 1u)) & 0xFFF00000u);
  const float sub = __builtin_rintf(a * 512.f) * 0x1p-9f;
  return copysignf(a < 0x1p-6f ? sub : nrm, v);
}

// Byte offsets inside one packed 4-bit K/V blob (layout in include/kvprof.h).
struct Int4Layout {
  int64_t n;      // quantized tokens N - R
  int64_t G;      // K token groups
  size_t kc, km, vc, vm, kr, vr;  // byte offsets inside a blob
};

__host__ __device__ inline Int4Layout int4_layout(int64_t N, int d, int R) {
  Int4Layout L;
  L.n = N - R;
  L.G = (L.n + 31) / 32;
  L.kc = 16;
  L.km = L.kc + (size_t)L.G * 32 * d / 2;
  L.vc = L.km + (size_t)L.G * d * 4;
  L.vm = L.vc + (size_t)L.n * d / 2;
  L.kr = L.vm + (size_t)L.n * (d / 32) * 4;
  L.vr = L.kr + (size_t)R * d * 4;
  return L;
}

}  // namespace kvp
