// S1: FP4 E2M1 encoding with one E4M3FN scale per channel group.
//
// Format [P3 "4비트로 적어도 되는 이유": NVFP4 without the second-level global
// scale, one 8-bit scale per 16 values; 448 x 6 = 2,688 range].  Rounding
// readings: scale = round-to-nearest-even (RNE) of amax/6 into E4M3FN,
// saturating at 448; value = RNE of |x|/scale into E2M1, saturating at 6;
// sign bit = (x < 0).
//
// Both roundings are decided exactly:
//  * amax/6 is formed in fp64.  amax has a 24-bit significand, so amax/6 is
//    either exactly an E4M3 rounding midpoint or at least ~2^-26 (relative)
//    away from one, far more than the 2^-53 error of the fp64 quotient.
//  * E2M1 rounding compares |x| with scale * {0.25, 0.75, 1.25, 1.75, 2.5,
//    3.5, 5}.  The scale has at most 4 significant bits and each constant at
//    most 3, so every threshold product is exact in fp32.
// One thread encodes one group; consecutive threads take consecutive groups
// of a row, so the fp32 reads and the code writes are coalesced.  The grid is
// bounded (grid_blocks) and strides over larger inputs.
#include "device.h"
#include "internal.h"

namespace csa2 {
namespace {

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

// Encodes one group of G fp32 values at src into G/2 code bytes at cdst and
// one scale byte at *sdst.
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

template <int G>
__global__ void __launch_bounds__(256)
quantize_kernel(const float *__restrict__ x, int64_t n, int dim, const int64_t *__restrict__ dst_rows,
                uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, int64_t plane_rows) {
  const int ngroups = dim / G;
  const int64_t total = n * ngroups;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = idx / ngroups;
    const int g = (int)(idx - r * ngroups);
    const int64_t dst = dst_rows ? dst_rows[r] : r;
    if (dst < 0 || dst >= plane_rows) continue;
    encode_group<G>(x + r * dim + (int64_t)g * G, codes + dst * (dim / 2) + (int64_t)g * (G / 2),
                    scales + dst * ngroups + g);
  }
}

// Appends n entries to both planes of a cache in one launch: threads
// [0, 32n) encode the 512-channel latents (32 groups of 16 per row), threads
// [32n, 36n) the 128-channel indexer keys (4 groups of 32 per row).
__global__ void __launch_bounds__(256)
append_kernel(const float *__restrict__ lat, const float *__restrict__ ik, int64_t n,
              const int64_t *__restrict__ dst_rows, uint8_t *__restrict__ kv_codes,
              uint8_t *__restrict__ kv_scales, uint8_t *__restrict__ ik_codes,
              uint8_t *__restrict__ ik_scales, int64_t plane_rows) {
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n * 36;
       idx += (int64_t)gridDim.x * blockDim.x) {
    if (idx < n * 32) {
      const int64_t r = idx >> 5;
      const int g = (int)(idx & 31);
      const int64_t dst = dst_rows[r];
      if (dst < 0 || dst >= plane_rows) continue;
      encode_group<16>(lat + r * 512 + g * 16, kv_codes + dst * 256 + g * 8, kv_scales + dst * 32 + g);
    } else {
      const int64_t j = idx - n * 32;
      const int64_t r = j >> 2;
      const int g = (int)(j & 3);
      const int64_t dst = dst_rows[r];
      if (dst < 0 || dst >= plane_rows) continue;
      encode_group<32>(ik + r * 128 + g * 32, ik_codes + dst * 64 + g * 16, ik_scales + dst * 4 + g);
    }
  }
}

}  // namespace

hipError_t launch_quantize(const float *x, int64_t n, int dim, int group, const int64_t *dst_rows,
                           uint8_t *codes, uint8_t *scales, int64_t plane_rows, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = grid_blocks(n * (dim / group), 256);
  if (group == 16)
    quantize_kernel<16><<<blocks, 256, 0, stream>>>(x, n, dim, dst_rows, codes, scales, plane_rows);
  else
    quantize_kernel<32><<<blocks, 256, 0, stream>>>(x, n, dim, dst_rows, codes, scales, plane_rows);
  return hipGetLastError();
}

hipError_t launch_append(const float *lat, const float *ik, int64_t n, const int64_t *dst_rows,
                         uint8_t *kv_codes, uint8_t *kv_scales, uint8_t *ik_codes, uint8_t *ik_scales,
                         int64_t plane_rows, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = grid_blocks(n * 36, 256);
  append_kernel<<<blocks, 256, 0, stream>>>(lat, ik, n, dst_rows, kv_codes, kv_scales, ik_codes, ik_scales,
                                            plane_rows);
  return hipGetLastError();
}

}  // namespace csa2
