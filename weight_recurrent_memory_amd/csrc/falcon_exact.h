// falcon_exact.h - the recurrence for a block of value rows of one chain, run by
// every thread of a chunk-form workgroup: the exact path of a chain whose decay
// products leave the range of the chunk algebra.
//
// The chunk kernels scale a chunk's unknowns by the decay products
// g_t = prod_{r<=t} a_r, a_r = 1 - eta_r lambda, of the chunk (explainer of arXiv
// 2608.27763, section 核心方法 §3, chunk-parallel form; 163.com article, section
// 02 (1) for the decay).  When some |g_t| leaves [2^-100, 2^100] or some |a_t| is
// below 2^-24 (strong forgetting: eta_t lambda near 1, or a decay far beyond 1 in
// magnitude) those scalings leave the float range; the kernel then notes it,
// keeps the chain's state untouched and, after its chunk loop, recomputes the
// workgroup's rows of that chain here, one token at a time in fp32 (the
// recurrent form, explainer §3), overwriting o and writing S_out.
//
// Per step, for every window sample j: r_j = s_i . x_j (pre-update state),
// e_j = y_{j,i} - r_j (y_{j,i} for the inner-product family);
// s_i <- a_i s_i + eta_i sum_j e_j x_j; o_{t,i} = s_i . q_t.  A row is owned by
// DK/4 consecutive threads holding 4 state columns each.
#pragma once
#include "falcon_device.h"
#include "falcon_launch.h"

namespace falcon {

// Decay-product bounds of the chunk algebra's ordinary path.
constexpr float kChunkGaugeLo = 0x1p-100f;
constexpr float kChunkGaugeHi = 0x1p100f;
constexpr float kChunkDecayLo = 0x1p-24f;

// True when a step's chunk decay product g (inclusive) or its decay a leaves the
// ordinary range (NaN counts as outside).
__device__ __forceinline__ bool gauge_out_of_range(float g, float a) {
  const float ag = __builtin_fabsf(g), aa = __builtin_fabsf(a);
  return !(ag >= kChunkGaugeLo && ag <= kChunkGaugeHi && aa >= kChunkDecayLo);
}

// Rows [row0, row0 + nrows) of chain `chain` (all NTH threads of the workgroup
// call this together; no barrier inside).  MAXW bounds the window.
template <int DK, int NTH, int MAXW>
__device__ __forceinline__ void recurrence_rows_impl(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ kp, const uint16_t* __restrict__ bt, const uint16_t* __restrict__ xh,
    const uint16_t* __restrict__ yh, const float* __restrict__ S0, float* __restrict__ o,
    float* __restrict__ S_out, long L, int dv, int B, int ks, int regression, int beta_kind,
    float beta0, float lambda, float eps, int chain, int row0, int nrows) {
  constexpr int CPT = 4;
  constexpr int TPR = DK / CPT;              // threads per row
  constexpr int RPP = NTH / TPR;             // rows per pass
  static_assert(NTH % TPR == 0, "whole rows per pass");
  const long qk_base = (long)chain * L * DK;
  const long v_base = (long)chain * L * dv;
  const int tid = threadIdx.x;
  const int c0 = (tid % TPR) * CPT;
  for (int p0 = 0; p0 < nrows; p0 += RPP) {
    const int rl = p0 + tid / TPR;
    const int row = row0 + rl;
    const bool active = rl < nrows && row < dv;
    const int rowc = active ? row : 0;
    float s[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e)
      s[e] = (S0 && active) ? S0[((long)chain * dv + rowc) * DK + c0 + e] : 0.0f;
    for (long t = 0; t < L; ++t) {
      float xw[MAXW][CPT];
      float yw[MAXW];
      float n = 0.0f;
#pragma unroll
      for (int w = 0; w < MAXW; ++w) {
        const long g = t - w;
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
          float xv = 0.0f;
          if (w < B && g >= ks) xv = ld_in(k, qk_base + (g - ks) * DK + c0 + e);
          else if (w < B && g == 0 && kp) xv = ld_in(kp, (long)chain * DK + c0 + e);
          else if (w < B && g < 0 && xh) xv = ld_in(xh, ((long)chain * (B - 1) + (B - 1) + g) * DK + c0 + e);
          xw[w][e] = xv;
          part += xv * xv;
        }
        n += part;
        float yv = 0.0f;
        if (w < B && g >= 0) yv = ld_in(v, v_base + g * dv + rowc);
        else if (w < B && yh) yv = ld_in(yh, ((long)chain * (B - 1) + (B - 1) + g) * dv + rowc);
        yw[w] = yv;
      }
      n = group_sum<TPR>(n);
      float beta = beta0;
      if (beta_kind == 1) beta = ld_in(bt, (long)chain * L + t);
      else if (beta_kind == 2) beta = ld_in(bt, ((long)chain * L + t) * dv + rowc);
      float eta = beta / (eps + n);
      float decay = 1.0f - eta * lambda;
      if (t == 0 && !kp && ks) {   // fresh sequence: S_0 = 0 and x_1 = 0 leave S_1 = 0
        eta = 0.0f;
        decay = 1.0f;
      }
      float ew[MAXW];
#pragma unroll
      for (int w = 0; w < MAXW; ++w) {
        if (w < B) {
          float r = 0.0f;
          if (regression) {
#pragma unroll
            for (int e = 0; e < CPT; ++e) r += s[e] * xw[w][e];
            r = group_sum<TPR>(r);
          }
          ew[w] = yw[w] - r;
        } else {
          ew[w] = 0.0f;
        }
      }
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        float acc = 0.0f;
#pragma unroll
        for (int w = 0; w < MAXW; ++w) acc += ew[w] * xw[w][e];
        s[e] = decay * s[e] + eta * acc;
      }
      float ov = 0.0f;
#pragma unroll
      for (int e = 0; e < CPT; ++e) ov += s[e] * ld_in(q, qk_base + t * DK + c0 + e);
      ov = group_sum<TPR>(ov);
      if (active && tid % TPR == 0) o[v_base + t * dv + row] = ov;
    }
    if (S_out && active) {
#pragma unroll
      for (int e = 0; e < CPT; ++e) S_out[((long)chain * dv + row) * DK + c0 + e] = s[e];
    }
  }
}

// The same for the chain and rows of a chunk-form workgroup, its SeqArgs read
// again from the kernel's argument segment (SeqArgs must be the kernel's first
// argument): the compiler then need not keep every argument in registers
// through the kernel's main loops for this rarely taken path.
template <int DK, int NTH, int MAXW>
__device__ __forceinline__ void recurrence_rows(int chain, int row0, int nrows) {
#if defined(__HIP_DEVICE_COMPILE__)
  const SeqArgs* ka = reinterpret_cast<const SeqArgs*>(__builtin_amdgcn_kernarg_segment_ptr());
  asm volatile("" : "+s"(ka));
#else
  const SeqArgs* ka = nullptr;   // the host pass generates no device code
#endif
  const SeqArgs& a = *ka;
  recurrence_rows_impl<DK, NTH, MAXW>(
      static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
      static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.k_prev),
      static_cast<const uint16_t*>(a.beta_t), static_cast<const uint16_t*>(a.x_hist),
      static_cast<const uint16_t*>(a.y_hist), a.S0, a.o, a.S_out, a.seqlen, a.dv, a.window,
      a.key_shift, a.regression, a.beta_kind, a.beta, a.lambda, a.eps, chain, row0, nrows);
}

}  // namespace falcon
