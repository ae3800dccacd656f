// falcon_mma.h - MFMA tile helpers of the chunk kernels: split-bf16 operand
// fragments and a 16x16 output tile product over a K range.
//
// Fragment convention (v_mfma_f32_16x16x32_bf16, wave64) and the split-bf16
// scheme are described in falcon_device.h.  An operand "row" is K-contiguous in
// LDS; fa(r, k) / fb(r, k) return the 8-wide fragment of row r at k.
#pragma once
#include "falcon_device.h"

namespace falcon {

struct HL {
  bf16x8 hi, lo;
};

__device__ __forceinline__ HL hl_zero() {
  HL z;
  z.hi = zero_frag();
  z.lo = zero_frag();
  return z;
}
__device__ __forceinline__ HL hl_pair(const uint16_t* hi, const uint16_t* lo) {
  HL f;
  f.hi = frag_bf16(hi);
  f.lo = frag_bf16(lo);
  return f;
}
__device__ __forceinline__ HL hl_bf16(const uint16_t* p) {
  HL f;
  f.hi = frag_bf16(p);
  f.lo = zero_frag();
  return f;
}
__device__ __forceinline__ HL hl_f32(const float* p) {
  HL f;
  frag_split(p, f.hi, f.lo);
  return f;
}
// 8 fp32 values (in registers) -> split fragment
__device__ __forceinline__ HL hl_vals(const float* v) {
  uint4 H, Lo;
  split_pair(v[0], v[1], H.x, Lo.x);
  split_pair(v[2], v[3], H.y, Lo.y);
  split_pair(v[4], v[5], H.z, Lo.z);
  split_pair(v[6], v[7], H.w, Lo.w);
  HL f;
  f.hi = __builtin_bit_cast(bf16x8, H);
  f.lo = __builtin_bit_cast(bf16x8, Lo);
  return f;
}

__device__ __forceinline__ void split1(float x, uint16_t& h, uint16_t& l) {
  const uint32_t hb = f32_to_bf16_bits(x);
  h = (uint16_t)hb;
  l = (uint16_t)f32_to_bf16_bits(x - __uint_as_float(hb << 16));
}

// 4 consecutive fp32 -> 4 hi and 4 lo bf16 stored with one 8-byte write each.
__device__ __forceinline__ void store_split4(uint16_t* hi, uint16_t* lo, const float* v) {
  uint2 H, Lo;
  split_pair(v[0], v[1], H.x, Lo.x);
  split_pair(v[2], v[3], H.y, Lo.y);
  *reinterpret_cast<uint2*>(hi) = H;
  *reinterpret_cast<uint2*>(lo) = Lo;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// acc[m][n] += sum_{k<K} A[m][k] B[n][k] for one 16x16 tile; fa(r, k) / fb(r, k)
// return the fragment of operand row r (0..15) at k (multiple of 8).  AX / BX:
// the operand is an exact bf16 value (its lo part is zero; pass skipped).
// The split passes (and, for exact operands, alternate k steps) accumulate into
// independent registers so consecutive MFMAs do not wait on each other; the
// partial sums are added at the end (fixed order, deterministic).
template <bool AX, bool BX, class FA, class FB>
__device__ __forceinline__ floatx4 mma_nt(floatx4 acc, int K, FA&& fa, FB&& fb) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int kq = (lane >> 4) * 8;
  const bool whole = (K & 31) == 0;      // every lane's k slot is in range
  floatx4 c1 = {0.f, 0.f, 0.f, 0.f}, c2 = {0.f, 0.f, 0.f, 0.f};
  int step = 0;
  for (int k0 = 0; k0 < K; k0 += 32, ++step) {
    const int k = k0 + kq;
    const bool in = whole || k < K;
    const HL A = in ? fa(r, k) : hl_zero();
    const HL Bv = in ? fb(r, k) : hl_zero();
    if (AX && BX) {
      if (step & 1) c1 = mfma16(A.hi, Bv.hi, c1);
      else acc = mfma16(A.hi, Bv.hi, acc);
    } else {
      acc = mfma16(A.hi, Bv.hi, acc);
      if (!BX) c1 = mfma16(A.hi, Bv.lo, c1);
      if (!AX) c2 = mfma16(A.lo, Bv.hi, c2);
    }
  }
  return acc + c1 + c2;
}

}  // namespace falcon
