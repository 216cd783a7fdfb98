// FP4 E2M1 encoding of one channel group with its E4M3FN scale, shared by the
// quantise / append kernels and by the scan that appends the new entries it
// scores.  Rounding readings and their exactness are described in
// quantize.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

// RNE of v >= 0 into E4M3FN, saturating at 448 (code 0x7E).
__device__ __forceinline__ uint32_t e4m3_rne(double v) {
  if (!(v > 0.0)) return 0u;
  if (v >= 448.0) return 0x7Eu;
  int e = ilogb(v);            // v in [2^e, 2^(e+1))
  if (e < -6) e = -6;          // subnormals share the quantum of exponent -6
  double n = rint(ldexp(v, 3 - e));   // units of 2^(e-3): [8, 16] normal, [0, 8] subnormal
  int code = (e + 7) * 8 + (int)n - 8;
  return (uint32_t)(code > 0x7E ? 0x7E : code);
}

// E4M3FN code (0..0x7E) -> its value.
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  uint32_t e = code >> 3, m = code & 7u;
  return e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8u + m), (int)e - 10);
}

// E2M1 magnitude code of a = |x| for scale s > 0, ties to the even code.
__device__ __forceinline__ uint32_t e2m1_mag(float a, float s) {
  return (uint32_t)(a > 0.25f * s) + (uint32_t)(a >= 0.75f * s) + (uint32_t)(a > 1.25f * s) +
         (uint32_t)(a >= 1.75f * s) + (uint32_t)(a > 2.5f * s) + (uint32_t)(a >= 3.5f * s) +
         (uint32_t)(a > 5.0f * s);
}

// Encodes one group of G fp32 values at src into G/2 code bytes at cdst
// (channel 2k in the low nibble of byte k) and one scale byte at *sdst.
template <int G>
__device__ __forceinline__ void encode_group(const float *__restrict__ src, uint8_t *__restrict__ cdst,
                                             uint8_t *__restrict__ sdst) {
  const float4 *s4 = reinterpret_cast<const float4 *>(src);
  float v[G];
#pragma unroll
  for (int i = 0; i < G / 4; ++i) {
    float4 f = s4[i];
    v[4 * i] = f.x;
    v[4 * i + 1] = f.y;
    v[4 * i + 2] = f.z;
    v[4 * i + 3] = f.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < G; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t scode = e4m3_rne((double)amax / 6.0);
  const float s = e4m3_value(scode);
  uint32_t packed[G / 8];
#pragma unroll
  for (int w = 0; w < G / 8; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float xv = v[8 * w + k];
      const uint32_t mag = (scode == 0) ? 0u : e2m1_mag(fabsf(xv), s);
      const uint32_t code = (xv < 0.0f ? 8u : 0u) | mag;
      word |= code << (4 * k);
    }
    packed[w] = word;
  }
  if constexpr (G == 16) {
    *reinterpret_cast<uint2 *>(cdst) = make_uint2(packed[0], packed[1]);
  } else {
    *reinterpret_cast<uint4 *>(cdst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  }
  *sdst = (uint8_t)scode;
}

}  // namespace csa2
