// falcon_device.h - device-side helpers shared by the gfx950 kernels of libfalcon:
// bf16 conversion, split-bf16 operands and the 16x16x32 bf16 MFMA fragment
// conventions.
//
// MFMA fragment convention used everywhere (v_mfma_f32_16x16x32_bf16, wave64):
//   A (16 x 32, row-major M x K):  lane l supplies A[l % 16][8 * (l / 16) + 0..7]
//   B (32 x 16, K x N):            lane l supplies B[8 * (l / 16) + 0..7][l % 16]
//   C (16 x 16, fp32):             lane l holds   C[4 * (l / 16) + r][l % 16], r = 0..3
// Only the pairing of A's and B's k-slots matters for the product, so every
// operand is stored K-contiguous in LDS ("row r, then k") and each lane reads
// 8 consecutive k values of one row with a single 16-byte (bf16) or two
// 16-byte (fp32) LDS reads.
//
// Split-bf16 ("bf16x3", Henry, Tang & Heinecke, ARITH 2019): an fp32 value a is
// carried as hi = bf16(a), lo = bf16(a - hi); a*b ~ hi_a*hi_b + hi_a*lo_b +
// lo_a*hi_b with fp32 accumulation, about 2^-16 relative error per product.
// Operands that are exact bf16 inputs (q, k) need no split.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace falcon {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware,
// v_cvt_pk_bf16_f32, two values per instruction).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

// Two fp32 -> one packed bf16 pair (a in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const floatx2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Split-bf16 of a pair: h = bf16(a) | bf16(b) << 16, l = the packed remainders.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& h, uint32_t& l) {
  h = pack_bf16x2(a, b);
  l = pack_bf16x2(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xFFFF0000u));
}

__device__ __forceinline__ float bf16_round(float x) {
  return __uint_as_float(f32_to_bf16_bits(x) << 16);
}

// Load one element of an input tensor as float.
__device__ __forceinline__ float ld_in(const uint16_t* p, long i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float ld_in(const float* p, long i) { return p[i]; }

__device__ __forceinline__ floatx4 mfma16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 zero_frag() {
  uint4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

// 8 consecutive bf16 values (16-byte aligned) from LDS.
__device__ __forceinline__ bf16x8 frag_bf16(const uint16_t* p) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

// 8 consecutive fp32 values (16-byte aligned) split into hi and lo bf16 parts.
__device__ __forceinline__ void frag_split(const float* p, bf16x8& hi, bf16x8& lo) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  uint4 H, Lo;
  split_pair(a.x, a.y, H.x, Lo.x);
  split_pair(a.z, a.w, H.y, Lo.y);
  split_pair(b.x, b.y, H.z, Lo.z);
  split_pair(b.z, b.w, H.w, Lo.w);
  hi = __builtin_bit_cast(bf16x8, H);
  lo = __builtin_bit_cast(bf16x8, Lo);
}

// Sum over the `width` lanes of an aligned lane group (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = WIDTH / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, WIDTH);
  return v;
}

}  // namespace falcon
