// falcon_recurrent.hip - recurrent form of the Falcon update, one token at a time
// (explainer of arXiv 2608.27763, section 核心方法 §3 "recurrent": O(d^2) per
// step, the inference form).
//
// Work decomposition: one workgroup per (batch*head, block of value rows).  Rows
// of S evolve independently given x_t (the update acts row-wise; Falcon-2's
// per-channel eta touches only its own row), so rows split freely across
// workgroups.  Inside a workgroup a row is owned by DK/4 consecutive lanes, each
// holding 4 state columns in registers; dot products reduce over that lane
// group with cross-lane shuffles.  Per step, for every window sample j:
//   r_j = s_i . x_j (pre-update state), e_j = y_{j,i} - r_j (or y_{j,i} for the
//   inner-product family); s_i <- a_i s_i + eta_i sum_j e_j x_j; o_{t,i} = s_i . q_t.
#include "falcon_device.h"
#include "falcon_launch.h"

namespace falcon {
namespace {

constexpr int kRecThreads = 256;
constexpr int kMaxWindow = 8;

template <typename T, int DK>
__global__ __launch_bounds__(kRecThreads) void recurrent_kernel(SeqArgs a, int rows_per_block) {
  constexpr int CPT = 4;          // state columns per lane
  constexpr int TPR = DK / CPT;   // lanes per row (4..32, divides the wave)
  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);
  const T* __restrict__ kp = static_cast<const T*>(a.k_prev);
  const T* __restrict__ bt = static_cast<const T*>(a.beta_t);
  const T* __restrict__ xh = static_cast<const T*>(a.x_hist);
  const T* __restrict__ yh = static_cast<const T*>(a.y_hist);

  const int chain = blockIdx.x;               // batch * heads + head
  const int rloc = threadIdx.x / TPR;
  const int cg = threadIdx.x % TPR;
  const int row = blockIdx.y * rows_per_block + rloc;
  const bool active = rloc < rows_per_block && row < a.dv;
  const int rowc = active ? row : 0;           // clamped index for loads
  const long L = a.seqlen;
  const long qk_base = (long)chain * L * DK;
  const long v_base = (long)chain * L * a.dv;
  const int c0 = cg * CPT;

  float s[CPT];
#pragma unroll
  for (int e = 0; e < CPT; ++e)
    s[e] = (a.S0 && active) ? a.S0[((long)chain * a.dv + rowc) * DK + c0 + e] : 0.0f;

  const int B = a.window;
  const int ks = a.key_shift;
  for (long t = 0; t < L; ++t) {
    // window samples g = t - w, w = 0..B-1: x_g = k[g-ks] (g >= ks), k_prev or 0
    // (g == 0 < ks); g < 0 is history slot B-1+g when one is carried, else zero
    float xw[kMaxWindow][CPT];
    float yw[kMaxWindow];
    float n = 0.0f;
#pragma unroll
    for (int w = 0; w < kMaxWindow; ++w) {
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
      if (w < B && g >= 0) yv = ld_in(v, v_base + g * a.dv + rowc);
      else if (w < B && yh) yv = ld_in(yh, ((long)chain * (B - 1) + (B - 1) + g) * a.dv + rowc);
      yw[w] = yv;
    }
    n = group_sum<TPR>(n);
    float beta = a.beta;
    if (a.beta_kind == 1) beta = ld_in(bt, (long)chain * L + t);
    else if (a.beta_kind == 2) beta = ld_in(bt, ((long)chain * L + t) * a.dv + rowc);
    float eta = beta / (a.eps + n);
    float decay = 1.0f - eta * a.lambda;
    if (t == 0 && !kp && ks) {  // fresh sequence: S_0 = 0 and x_1 = 0 leave S_1 = 0
      eta = 0.0f;
      decay = 1.0f;
    }
    float ew[kMaxWindow];
#pragma unroll
    for (int w = 0; w < kMaxWindow; ++w) {
      if (w < B) {
        float r = 0.0f;
        if (a.regression) {
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
      for (int w = 0; w < kMaxWindow; ++w) acc += ew[w] * xw[w][e];
      s[e] = decay * s[e] + eta * acc;
    }
    float ov = 0.0f;
#pragma unroll
    for (int e = 0; e < CPT; ++e) ov += s[e] * ld_in(q, qk_base + t * DK + c0 + e);
    ov = group_sum<TPR>(ov);
    if (active && cg == 0) a.o[v_base + t * a.dv + row] = ov;
  }
  if (a.S_out && active) {
#pragma unroll
    for (int e = 0; e < CPT; ++e) a.S_out[((long)chain * a.dv + row) * DK + c0 + e] = s[e];
  }
}

template <typename T, int DK>
hipError_t launch_typed(const SeqArgs& a, hipStream_t stream) {
  constexpr int TPR = DK / 4;
  int rows = kRecThreads / TPR;
  if (rows > a.dv) rows = a.dv;
  dim3 grid(a.batch * a.heads, (a.dv + rows - 1) / rows);
  hipLaunchKernelGGL((recurrent_kernel<T, DK>), grid, dim3(kRecThreads), 0, stream, a, rows);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dk(const SeqArgs& a, hipStream_t stream) {
  switch (a.dk) {
    case 16: return launch_typed<T, 16>(a, stream);
    case 32: return launch_typed<T, 32>(a, stream);
    case 64: return launch_typed<T, 64>(a, stream);
    case 128: return launch_typed<T, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

// The window-1 latest samples after a call, oldest first: slot h holds sample
// s = L - (B-1) + h (0-based steps; sample s pairs x_s with y_s = v_s, x_s =
// k_{s-shift}, x_0 = k_prev or 0 when shift = 1); s < 0 comes from the incoming history slot
// B-1+s (zero without one).  One thread per column walks the slots in
// ascending order: in-place use (out == incoming history) reads slot L+h > h
// before anything at or above slot h has been written.
template <typename T>
__global__ __launch_bounds__(256) void history_out_kernel(SeqArgs a, T* xo, T* yo) {
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);
  const T* __restrict__ kp = static_cast<const T*>(a.k_prev);
  const T* xh = static_cast<const T*>(a.x_hist);
  const T* yh = static_cast<const T*>(a.y_hist);
  const long chain = blockIdx.x;
  const int NH = a.window - 1;
  const long L = a.seqlen;
  for (int c = threadIdx.x; c < a.dk + a.dv; c += blockDim.x) {
    const bool isx = c < a.dk;
    const int col = isx ? c : c - a.dk;
    const int d = isx ? a.dk : a.dv;
    T* out = isx ? xo : yo;
    const T* hin = isx ? xh : yh;
    for (int h = 0; h < NH; ++h) {
      const long s = L - NH + h;
      T val = T(0);
      if (s >= 0) {
        if (!isx) val = v[(chain * L + s) * a.dv + col];
        else if (s >= a.key_shift) val = k[(chain * L + s - a.key_shift) * a.dk + col];
        else if (kp) val = kp[chain * a.dk + col];
      } else if (hin) {
        val = hin[(chain * NH + NH + s) * d + col];
      }
      out[(chain * NH + h) * d + col] = val;
    }
  }
}

}  // namespace

hipError_t launch_history_out(const SeqArgs& a, void* x_out, void* y_out, hipStream_t stream) {
  const dim3 grid((unsigned)((long)a.batch * a.heads));
  if (a.dtype == 0)
    hipLaunchKernelGGL(history_out_kernel<uint16_t>, grid, dim3(256), 0, stream, a,
                       static_cast<uint16_t*>(x_out), static_cast<uint16_t*>(y_out));
  else
    hipLaunchKernelGGL(history_out_kernel<float>, grid, dim3(256), 0, stream, a,
                       static_cast<float*>(x_out), static_cast<float*>(y_out));
  return hipGetLastError();
}

hipError_t launch_recurrent(const SeqArgs& a, hipStream_t stream) {
  (void)hipGetLastError();
  if (a.dtype == 0) return launch_dk<uint16_t>(a, stream);
  return launch_dk<float>(a, stream);
}

}  // namespace falcon
