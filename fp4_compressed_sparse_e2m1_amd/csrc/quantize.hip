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
#include "encode.h"
#include "internal.h"

namespace csa2 {
namespace {

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
