// Device helpers shared by the CSA2 kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Order-preserving map fp32 -> uint32 (larger score -> larger key).  Key 0 is
// reserved for "no candidate": every non-NaN float maps above it (-inf maps to
// 0x007FFFFF), so a selection never picks a 0 key.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Eight E2M1 codes (one dword, channel 2k in the low nibble of byte k) ->
// eight fp16 values in channel order.  The gfx950 scaled conversion applies
// only the exponent of its fp32 scale, so it is used with scale 1.0 (exact)
// and the E4M3 block scale is applied separately.
__device__ __forceinline__ f16x8 e2m1x8_to_f16(uint32_t w) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Four E4M3FN bytes of one dword -> four fp16 values (exact, unit scale).
__device__ __forceinline__ void e4m3x4_to_f16(uint32_t w, _Float16 *out) {
  f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

// Eight E4M3FN bytes (two dwords, element order) -> f16x8.
__device__ __forceinline__ f16x8 e4m3x8_to_f16(uint32_t w0, uint32_t w1) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// One E4M3FN byte (in the low 8 bits) -> fp16 (exact).
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t byte) {
  f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(byte, 1.0f, false);
  return v[0];
}

// Q enters the f16 contractions (logits, index scores) times a power of two
// 2^k per head, chosen from the head's largest bf16 magnitude so that it lands
// in [2^15, 2^16): no value overflows f16, every value at least 2^-29 times
// the head's largest is an f16 normal and converts exactly (8 significant
// bits), smaller ones round toward zero on the f16 subnormal grid, and the f32
// results are scaled back by 2^-k exactly.  k is at most 100 (a head whose
// largest |q| is below 2^-85 keeps a smaller factor), so 2^-k times a softmax
// scale or an index weight stays a normal f32.

// Running maximum of the magnitude bits (sign cleared, so they order as the
// magnitudes) of eight bf16 values, two lanes of 16 bits.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 bf16x8_absmax(uint4 v, u16x2 m) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
  return m;
}
__device__ __forceinline__ uint32_t absmax_bits(u16x2 m) { return m[0] > m[1] ? m[0] : m[1]; }

// the exponent k for a head whose largest magnitude bits are mx
__device__ __forceinline__ int q_prescale_exp(uint32_t mx) {
  const int k = 142 - (int)(mx >> 7);     // 142: the biased exponent of 2^15
  return k < 100 ? k : 100;
}

// 2^k as a float, -126 <= k <= 127
__device__ __forceinline__ float exp2i(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// eight bf16 values times up (a power of two) in f16; exact whenever the
// products are f16 normals
__device__ __forceinline__ f16x8 bf16x8_to_f16_scaled(uint4 v, float up) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  f16x8 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 pr = __builtin_bit_cast(
        f16x2, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w[i] << 16) * up, __uint_as_float(w[i] & 0xFFFF0000u) * up));
    h[2 * i] = pr[0];
    h[2 * i + 1] = pr[1];
  }
  return h;
}

// max(x, 0) in one instruction: median of x, 0 and the largest float (+inf
// inputs, outside the contract, would clamp to that value).
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.402823466e38f); }

// max(a, b) in one instruction: median of a, b and the largest float.
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, 3.402823466e38f); }

// Lane permutations inside a row of 16 lanes (DPP): XOR 1 and XOR 2 within a
// quad, mirror within each half row of 8.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7 - i within each 8 lanes
constexpr int kDppRowRor8 = 0x128;     // lane i <- lane (i + 8) mod 16 within each 16 lanes

// Maximum over each aligned group of 8 lanes, in every lane of the group.
__device__ __forceinline__ float max8(float m) {
  m = fmax2(m, dpp<kDppXor1>(m));
  m = fmax2(m, dpp<kDppXor2>(m));
  return fmax2(m, dpp<kDppHalfMirror>(m));
}

// Value of lane l ^ 16: the 16-lane rows of each half wave trade places
// (ds_swizzle in bit-mask mode: and 0x1F, or 0, xor 0x10; no LDS memory).
__device__ __forceinline__ float swap_rows16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}

// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48, in each of them.
__device__ __forceinline__ uint32_t umax_rows(uint32_t x) {
  const uint32_t o16 = (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x401F);
  x = x > o16 ? x : o16;
  const auto sw = __builtin_amdgcn_permlane32_swap((int)x, (int)x, false, false);
  const uint32_t o32 = (uint32_t)((__lane_id() & 32) ? sw[0] : sw[1]);
  return x > o32 ? x : o32;
}

// Maximum of unsigned keys over each aligned group of 8 lanes, in every lane
// of the group.
__device__ __forceinline__ uint32_t umax8(uint32_t k) {
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0xB1, 0xF, 0xF, false);
  k = k > o ? k : o;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x4E, 0xF, 0xF, false);
  k = k > o ? k : o;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x141, 0xF, 0xF, false);
  return k > o ? k : o;
}

// Value of lane l + 16 for lanes 0..15 (and 32..47): the odd 16-lane rows are
// swapped into the even ones.
__device__ __forceinline__ float from_next_row(float x) {
  const int xi = __float_as_int(x);
  const auto sw = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  return __int_as_float(sw[1]);
}

// Orders the LDS accesses of one wave before and after it (no work-group
// barrier: the other waves are not involved).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// D = A(16x16) * B(16x16) + C on the matrix cores.  Lane l holds
// A[l % 16][4*(l/16) .. +3], B[4*(l/16) .. +3][l % 16] and
// C[4*(l/16) .. +3][l % 16].
__device__ __forceinline__ f32x4 mfma16x16x16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Transposed LDS read of 16-bit data: within each group of 16 lanes, lane i
// receives element (i % 4) of the 4-element rows addressed by lanes
// i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 (in that order).
__device__ __forceinline__ f16x4 lds_read_tr16(const _Float16 *p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
  return __builtin_bit_cast(f16x4, v);
}

// D = A(16x32) * B(32x16) + C on the matrix cores.  Lane l holds
// A[l % 16][8*(l/16) .. +7], B[8*(l/16) .. +7][l % 16] and
// C[4*(l/16) .. +3][l % 16].
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace csa2
