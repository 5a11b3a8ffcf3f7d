// Device helpers shared by the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kBlock = 128;      // quantisation group width and weight block edge
constexpr float kFp8Max = 448.0f;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ----------------------------------------------------------------------------- e4m3
// Two fp32 values -> two OCP e4m3 bytes (round to nearest even) in the low half
// of the result. Callers clamp to +-448 first, so no value saturates here.
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
}

__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// ----------------------------------------------------------------------------- NaN-keeping quantisation
// IEEE 754-2019 maximum / minimum (v_maximum_f32 / v_minimum_f32 on gfx950):
// a NaN operand gives NaN, where fmaxf / fminf would drop it.  The quantisers
// take their group maxima and clamps with these, so a NaN value turns its
// group's scale and its own code into NaN and reaches the outputs.
__device__ __forceinline__ float nan_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float nan_min(float a, float b) { return __builtin_elementwise_minimum(a, b); }

// v clamped to the e4m3 range [-448, 448]; NaN stays NaN (and encodes as NaN).
__device__ __forceinline__ float clamp_fp8(float v) { return nan_min(nan_max(v, -kFp8Max), kFp8Max); }

// fp32 scale of a 1x128 group with largest magnitude amax: amax / 448 (IEEE
// division), 1 for an all-zero group, NaN when amax is NaN.
__device__ __forceinline__ float group_scale(float amax) { return amax == 0.f ? 1.0f : amax / kFp8Max; }

// ----------------------------------------------------------------------------- MX scales
// E8M0 code (e + 127, at least 0) of the MX scale 2^e of a block whose largest
// magnitude is amax >= 0: the smallest e with amax <= 448 * 2^e.  With
// amax = m 2^p (1 <= m < 2) and 448 = 1.75 * 2^8, e = p - 8 when m <= 1.75
// and p - 7 otherwise: integer work on the fp32 bits, exact for every input
// (zero and subnormals give code 0, the smallest scale 2^-127).  A NaN amax
// gives 0xFF, the E8M0 NaN.
__device__ __forceinline__ uint32_t mx_code(float amax) {
  const uint32_t b = __float_as_uint(amax);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0xffu;
  const int c = static_cast<int>(b >> 23) - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  return c > 0 ? static_cast<uint32_t>(c) : 0u;
}

// 1 / 2^e = 2^(127 - code) for an MX code from mx_code (code <= 248), and
// NaN for the NaN code 0xFF.
__device__ __forceinline__ float mx_inv_scale(uint32_t code) {
  return code == 0xffu ? __uint_as_float(0x7fc00000u) : __uint_as_float((254u - code) << 23);
}

// ----------------------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// max over the 16 lanes that share lane/16 (the 16 columns of one MFMA row group)
__device__ __forceinline__ float max16(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// ----------------------------------------------------------------------------- byte transpose
// Four dwords r0..r3 (byte b of r_i = element (i, b)) -> c0..c3 with byte i of
// c_b = element (i, b).  v_perm_b32 picks result bytes from {S0:S1}; selector
// values 0-3 address S1, 4-7 address S0.
__device__ __forceinline__ void transpose4x4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                             uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                             uint32_t& c3) {
  uint32_t t0 = __builtin_amdgcn_perm(r1, r0, 0x06020400u);  // r0.0 r1.0 r0.2 r1.2
  uint32_t t1 = __builtin_amdgcn_perm(r1, r0, 0x07030501u);  // r0.1 r1.1 r0.3 r1.3
  uint32_t t2 = __builtin_amdgcn_perm(r3, r2, 0x06020400u);  // r2.0 r3.0 r2.2 r3.2
  uint32_t t3 = __builtin_amdgcn_perm(r3, r2, 0x07030501u);  // r2.1 r3.1 r2.3 r3.3
  c0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  c1 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  c2 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  c3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// ----------------------------------------------------------------------------- MFMA
// D(16x16 fp32) = A(16x128 e4m3) * B(128x16 e4m3) + C.  Lane l holds 32 bytes
// of A row l%16 and of B column l%16 (the same K slots for both), and
// returns rows 4*(l/16)+i, i<4, of column l%16.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same with E8M0 block scales applied by the matrix core (32-deep K
// blocks).  Lane l passes in byte 0 of sa / sb the scale of A row (B column)
// l%16 for K block l/16, i.e. K 32(l/16)..+31.  Its data bytes 0-15 are
// K 16(l/16)..+15 and bytes 16-31 are K 64 + 16(l/16)..+15, so K block b
// sits in lane groups 2(b%2) and 2(b%2)+1 at bytes 16(b/2)..+15 (measured on
// gfx950 with single nonzero bytes and distinct per-lane scales).
__device__ __forceinline__ v4f mfma_fp8_16x16x128_mx(v8i a, v8i b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// A in E2M1 (FP4), B in e4m3, E8M0 scales as above.  Lane l's 16 A bytes
// (a[0..3]; a[4..7] are ignored) are K 32(l/16)..+31 in order, low nibble
// first, so its scale covers exactly its own data (measured on gfx950 like
// the layout above).
__device__ __forceinline__ v4f mfma_fp4_fp8_16x16x128_mx(v8i a, v8i b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, sa, 0, sb);
}

// ----------------------------------------------------------------------------- misc
__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace moe
