// falcon_decode.hip - one decode step of the Falcon recurrence for serving
// (explainer of arXiv 2608.27763, section 核心方法 §3: the recurrent form serves
// inference; 163.com section 01: write first, then read with the updated state).
//
// Per (sequence, head), with x = k_prev (prefix pairing; x = k with same-step
// pairing, which leaves k_prev alone) and y = v:
//   r1 = S x, r2 = S q                     (one read pass over S)
//   e  = y - r1 (regression) or y (inner product)
//   S' = a S + eta e x^T                   (one write pass, in place)
//   o  = a r2 + eta e (x . q)              (= S' q, read-after-write)
//   k_prev <- k
// The step is bound by HBM: S is read once and written once, ~1 flop per byte.
// One workgroup owns one (sequence, head), so the in-place k_prev update cannot
// race with another workgroup.  Each row of S is read by DK/4 lanes with 16-byte
// loads; every lane issues all of its row loads before the first reduction so
// the memory system sees PASSES independent 16-byte requests per lane.
#include "falcon_device.h"
#include "falcon_launch.h"

namespace falcon {
namespace {

// Threads per workgroup: dk/4 lanes per row of S, up to 512 (two passes over
// the rows at dk = dv = 64); measured on 512 x 12 x 64 x 64 with the state
// evicted before each step: 256 threads 39.6 us, 512 threads 38.2 us, 1024
// threads 44.2 us per step.
template <int DK, int DV>
constexpr int dec_threads() { return DV * (DK / 4) < 512 ? DV * (DK / 4) : 512; }

template <typename T, int DK, int DV>
__global__ __launch_bounds__((dec_threads<DK, DV>())) void decode_kernel(DecodeArgs a) {
  constexpr int TPR = DK / 4;                    // lanes per row
  constexpr int RPP = dec_threads<DK, DV>() / TPR;   // rows per pass
  constexpr int PASSES = (DV + RPP - 1) / RPP;
  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);
  const T* __restrict__ bt = static_cast<const T*>(a.beta_t);
  T* __restrict__ kp = static_cast<T*>(a.k_prev);

  const long head = blockIdx.x;                  // sequence * heads + head
  const int rloc = threadIdx.x / TPR;
  const int cg = threadIdx.x % TPR;
  const int c0 = cg * 4;
  float* __restrict__ Sh = a.S + head * (long)DV * DK;

  // Issue the state loads first.
  floatx4 s[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = p * RPP + rloc;
    if (row < DV) s[p] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(Sh + (long)row * DK + c0));
    else s[p] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  float x[4], qq[4];
  const T* xsrc = a.key_shift ? kp : k;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = ld_in(xsrc, head * DK + c0 + e);
    qq[e] = ld_in(q, head * DK + c0 + e);
  }
  float yv[PASSES], bv[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = p * RPP + rloc;
    const int rc = row < DV ? row : 0;
    yv[p] = ld_in(v, head * DV + rc);
    bv[p] = a.beta_kind == 0 ? a.beta
            : (a.beta_kind == 1 ? ld_in(bt, head) : ld_in(bt, head * DV + rc));
  }
  // Every lane has read its slice of k_prev; only now may it be overwritten.
  __syncthreads();
  if (rloc == 0 && a.key_shift) {
#pragma unroll
    for (int e = 0; e < 4; ++e) kp[head * DK + c0 + e] = k[head * DK + c0 + e];
  }
  float n = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
  float xq = x[0] * qq[0] + x[1] * qq[1] + x[2] * qq[2] + x[3] * qq[3];
  n = group_sum<TPR>(n);
  xq = group_sum<TPR>(xq);
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = p * RPP + rloc;
    float r1 = s[p].x * x[0] + s[p].y * x[1] + s[p].z * x[2] + s[p].w * x[3];
    float r2 = s[p].x * qq[0] + s[p].y * qq[1] + s[p].z * qq[2] + s[p].w * qq[3];
    r1 = group_sum<TPR>(r1);
    r2 = group_sum<TPR>(r2);
    const float eta = bv[p] / (a.eps + n);
    const float dec = 1.0f - eta * a.lambda;
    const float e = a.regression ? yv[p] - r1 : yv[p];
    const float w = eta * e;
    floatx4 sn;
    sn.x = dec * s[p].x + w * x[0];
    sn.y = dec * s[p].y + w * x[1];
    sn.z = dec * s[p].z + w * x[2];
    sn.w = dec * s[p].w + w * x[3];
    if (row < DV) {
      __builtin_nontemporal_store(sn, reinterpret_cast<floatx4*>(Sh + (long)row * DK + c0));
      if (cg == 0) a.o[head * DV + row] = dec * r2 + w * xq;
    }
  }
}

// Sliding-window step (Falcon-3/3A): the window is the carried history of
// B-1 samples (oldest first) plus (x, y) = (k_prev, v):
//   n = sum_w ||x_w||^2, r_w = S x_w, e_w = y_w - r_w (or y_w), r2 = S q
//   S' = a S + eta sum_w e_w x_w^T,  o = a r2 + eta sum_w e_w (x_w . q)
// then the history drops its oldest sample and appends (x, y), and k_prev <- k
// (prefix pairing; with same-step pairing x = k and k_prev is not used).
constexpr int kMaxDecWindow = 8;

template <typename T, int DK, int DV>
__global__ __launch_bounds__((dec_threads<DK, DV>())) void decode_window_kernel(DecodeArgs a) {
  constexpr int TPR = DK / 4;
  constexpr int RPP = dec_threads<DK, DV>() / TPR;
  constexpr int PASSES = (DV + RPP - 1) / RPP;
  constexpr int MW = kMaxDecWindow;
  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);
  const T* __restrict__ bt = static_cast<const T*>(a.beta_t);
  T* kp = static_cast<T*>(a.k_prev);
  T* xh = static_cast<T*>(a.x_hist);
  T* yh = static_cast<T*>(a.y_hist);

  const long head = blockIdx.x;
  const int rloc = threadIdx.x / TPR;
  const int cg = threadIdx.x % TPR;
  const int c0 = cg * 4;
  const int B = a.window, NH = B - 1;
  float* __restrict__ Sh = a.S + head * (long)DV * DK;

  floatx4 s[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = p * RPP + rloc;
    if (row < DV) s[p] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(Sh + (long)row * DK + c0));
    else s[p] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const T* xcur = a.key_shift ? static_cast<const T*>(kp) : k;   // this step's x
  float x[MW][4], qq[4];
#pragma unroll
  for (int w = 0; w < MW; ++w)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float xv = 0.0f;
      if (w < NH) xv = ld_in(xh, (head * NH + w) * DK + c0 + e);
      else if (w == NH) xv = ld_in(xcur, head * DK + c0 + e);
      x[w][e] = xv;
    }
#pragma unroll
  for (int e = 0; e < 4; ++e) qq[e] = ld_in(q, head * DK + c0 + e);
  float yv[PASSES][MW], bv[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = p * RPP + rloc;
    const int rc = row < DV ? row : 0;
#pragma unroll
    for (int w = 0; w < MW; ++w) {
      float y = 0.0f;
      if (w < NH) y = ld_in(yh, (head * NH + w) * DV + rc);
      else if (w == NH) y = ld_in(v, head * DV + rc);
      yv[p][w] = y;
    }
    bv[p] = a.beta_kind == 0 ? a.beta : ld_in(bt, head);
  }
  // every lane has read k_prev and the history; only now may they change
  __syncthreads();
  if (rloc == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const long c = c0 + e;
      for (int w = 0; w + 1 < NH; ++w) xh[(head * NH + w) * DK + c] = xh[(head * NH + w + 1) * DK + c];
      xh[(head * NH + NH - 1) * DK + c] = xcur[head * DK + c];
      if (a.key_shift) kp[head * DK + c] = k[head * DK + c];
    }
  }
  float n = 0.0f, xq[MW];
#pragma unroll
  for (int w = 0; w < MW; ++w) {
    n += x[w][0] * x[w][0] + x[w][1] * x[w][1] + x[w][2] * x[w][2] + x[w][3] * x[w][3];
    xq[w] = 0.0f;
    if (w < B) xq[w] = group_sum<TPR>(x[w][0] * qq[0] + x[w][1] * qq[1] + x[w][2] * qq[2] + x[w][3] * qq[3]);
  }
  n = group_sum<TPR>(n);
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = p * RPP + rloc;
    float r2 = s[p].x * qq[0] + s[p].y * qq[1] + s[p].z * qq[2] + s[p].w * qq[3];
    r2 = group_sum<TPR>(r2);
    const float eta = bv[p] / (a.eps + n);
    const float dec = 1.0f - eta * a.lambda;
    float acc[4] = {0.f, 0.f, 0.f, 0.f}, ow = 0.0f;
#pragma unroll
    for (int w = 0; w < MW; ++w) {
      if (w < B) {
        float e = yv[p][w];
        if (a.regression) {
          float r1 = s[p].x * x[w][0] + s[p].y * x[w][1] + s[p].z * x[w][2] + s[p].w * x[w][3];
          e -= group_sum<TPR>(r1);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += e * x[w][c];
        ow += e * xq[w];
      }
    }
    floatx4 sn;
    sn.x = dec * s[p].x + eta * acc[0];
    sn.y = dec * s[p].y + eta * acc[1];
    sn.z = dec * s[p].z + eta * acc[2];
    sn.w = dec * s[p].w + eta * acc[3];
    if (row < DV) {
      __builtin_nontemporal_store(sn, reinterpret_cast<floatx4*>(Sh + (long)row * DK + c0));
      if (cg == 0) {
        a.o[head * DV + row] = dec * r2 + eta * ow;
        for (int w = 0; w + 1 < NH; ++w) yh[(head * NH + w) * DV + row] = yh[(head * NH + w + 1) * DV + row];
        yh[(head * NH + NH - 1) * DV + row] = v[head * DV + row];
      }
    }
  }
}

template <typename T, int DK, int DV>
hipError_t launch3(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((long)a.nseq * a.heads));
  if (a.window > 1)
    hipLaunchKernelGGL((decode_window_kernel<T, DK, DV>), grid, dim3(dec_threads<DK, DV>()), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<T, DK, DV>), grid, dim3(dec_threads<DK, DV>()), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int DK>
hipError_t launch_dv(const DecodeArgs& a, hipStream_t stream) {
  switch (a.dv) {
    case 16: return launch3<T, DK, 16>(a, stream);
    case 32: return launch3<T, DK, 32>(a, stream);
    case 64: return launch3<T, DK, 64>(a, stream);
    case 128: return launch3<T, DK, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_dk(const DecodeArgs& a, hipStream_t stream) {
  switch (a.dk) {
    case 16: return launch_dv<T, 16>(a, stream);
    case 32: return launch_dv<T, 32>(a, stream);
    case 64: return launch_dv<T, 64>(a, stream);
    case 128: return launch_dv<T, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  (void)hipGetLastError();
  if (a.dtype == 0) return launch_dk<uint16_t>(a, stream);
  return launch_dk<float>(a, stream);
}

}  // namespace falcon
