// falcon_backward.hip - gradients of the window-1 chunk form (Falcon-1/2/1A/2A)
// on gfx950.
//
// The pages give no gradients; the chunk form they describe for training
// (explainer of arXiv 2608.27763, section 核心方法 §3 chunk-parallel; 163.com
// section 02 (2): inside a chunk everything is parallel, only the fixed-size
// state crosses chunks) is differentiated by the chain rule.  Per value row i
// and chunk of c steps starting from state row s0 (0-based steps t, g_t =
// prod_{r<=t} a_r, gm_t = g_{t-1}, zeta = eta / g, G = X X^T, P = lower(Q X^T)):
//   forward   e_t = y_t - gm_t (s0.x_t + sum_{s<t} G_ts z_s)  (inner product: e = y)
//             z = zeta e;  o_t = g_t (q_t.s0 + sum_{s<=t} P_ts z_s);
//             s_end = gC (s0 + sum_s z_s x_s),  gC = g_{c-1}
//   backward  dz_s = sum_{t>=s} P_ts g_t do_t + gC (x_s.ds_end);  de = zeta dz
//             dr_s = de_s - zeta_s sum_{t>s} G_ts w_t,  w_t = gm_t dr_t   (dv = dr)
//             ds0 = gC ds_end + sum_t g_t do_t q_t - sum_t w_t x_t
//             dG_ts = -sum_i w_t z_s (t > s),  dP_ts = sum_i g_t do_t z_s (s <= t)
//             dq_t = sum_i g_t do_t s0 + sum_s dP_ts x_s
//             dx_t = sum_i (gC z_t ds_end - w_t s0) + sum_s (dG_ts + dG_st) x_s
//                    + sum_t' dP_t't q_t' + 2 dn_t x_t
//   scalars   dg_t = do_t o_t / g_t - dzeta_t zeta_t / g_t (+ ds_end.s_end / gC at c-1)
//             (+ the terms through gm_{t+1}); da_r = sum_{t>=r} dg_t g_t / a_r;
//             deta = dzeta / g - lambda da;  dbeta = deta / (eps + n);
//             dn = -sum_i deta eta / (eps + n)
//
// One workgroup (8 waves) per (batch*head) chain holds the whole state and its
// gradient in LDS, so every sum over value rows stays inside the workgroup.  A
// forward sweep over 16-step chunks stores each chunk's starting state in the
// caller's workspace; the backward sweep walks the chunks in reverse, reloads
// that state, recomputes the chunk's forward quantities and carries dS.  Per
// chunk: dk-long dot products (Gram, q.x, S0 x, S0 q, dS x) by all threads;
// the per-row triangular sweeps (forward solve, its transpose, the scalar
// chain) on one lane per value row; then the sums over rows (dG, dP, dn) and
// the dk-wide products (dq, dx, dS) by all threads.  Arithmetic is fp32.
#include "falcon_device.h"
#include "falcon_launch.h"

namespace falcon {
namespace {

constexpr int BC = 16;        // chunk length of the backward
constexpr int BNT = 512;

template <int DK, int DV>
struct BwdLds {
  float S[DV][DK + 4];        // chunk-start state
  float dS[DV][DK + 4];       // gradient of the chunk-end state
  float X[BC][DK + 4];        // keys x_t (shifted)
  float Q[BC][DK + 4];
  float Y[BC][DV + 4];        // values
  float dO[BC][DV + 4];
  float bt[BC][DV];           // gain per step and row
  float nrm[BC];
  float G[BC][BC + 1];
  float P[BC][BC + 1];
  float XS[BC][DV + 4];       // s0_i . x_t
  float QS[BC][DV + 4];       // s0_i . q_t
  float XdS[BC][DV + 4];      // ds_i . x_t
  float sds[DV];              // s0_i . ds_i
  float Z[BC][DV + 4];
  float W[BC][DV + 4];        // gm_t dr_t
  float GD[BC][DV + 4];       // g_t do_t
  float DE[BC][DV + 4];       // d eta
  float ETA[BC][DV + 4];
  float gC[DV];
  float dG[BC][BC + 1];
  float dP[BC][BC + 1];
  float dn[BC];
};

__device__ __forceinline__ float dot4(const float4 a, const float4 b, float acc) {
  acc = __builtin_fmaf(a.x, b.x, acc);
  acc = __builtin_fmaf(a.y, b.y, acc);
  acc = __builtin_fmaf(a.z, b.z, acc);
  return __builtin_fmaf(a.w, b.w, acc);
}

// sum_k a[k] b[k] over n floats (n % 4 == 0), both 16-byte aligned in LDS
__device__ __forceinline__ float row_dot(const float* a, const float* b, int n) {
  float acc = 0.0f;
  for (int k = 0; k < n; k += 4)
    acc = dot4(*reinterpret_cast<const float4*>(a + k), *reinterpret_cast<const float4*>(b + k), acc);
  return acc;
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(BNT) void backward_kernel(BwdArgs a) {
  using SM = BwdLds<DK, DV>;
  __shared__ __align__(16) SM sm;
  const T* __restrict__ qg = static_cast<const T*>(a.q);
  const T* __restrict__ kg = static_cast<const T*>(a.k);
  const T* __restrict__ vg = static_cast<const T*>(a.v);
  const T* __restrict__ kpg = static_cast<const T*>(a.k_prev);
  const T* __restrict__ bg = static_cast<const T*>(a.beta_t);
  const int tid = threadIdx.x;
  const long chain = blockIdx.x;
  const long L = a.seqlen;
  const int nch = (int)((L + BC - 1) / BC);
  const int ks = a.key_shift;
  const bool fresh = ks == 1 && kpg == nullptr;
  const long qk_base = chain * L * DK;
  const long v_base = chain * L * DV;
  float* __restrict__ ws = a.workspace + chain * (long)nch * DV * DK;

  // ---- loaders ----
  auto load_chunk = [&](long t0, int c, bool with_q) {
    for (int idx = tid; idx < BC * DK; idx += BNT) {
      const int t = idx / DK, kk = idx % DK;
      const long g = t0 + t;
      float xv = 0.0f, qv = 0.0f;
      if (t < c) {
        if (g >= ks) xv = ld_in(kg, qk_base + (g - ks) * DK + kk);
        else if (kpg) xv = ld_in(kpg, chain * DK + kk);
        if (with_q) qv = ld_in(qg, qk_base + g * DK + kk);
      }
      sm.X[t][kk] = xv;
      sm.Q[t][kk] = qv;
    }
    for (int idx = tid; idx < BC * DV; idx += BNT) {
      const int t = idx / DV, i = idx % DV;
      const long g = t0 + t;
      float yv = 0.0f, dov = 0.0f, bv = 0.0f;
      if (t < c) {
        yv = ld_in(vg, v_base + g * DV + i);
        if (with_q) dov = a.dO[v_base + g * DV + i];
        bv = a.beta_kind == 0 ? a.beta
             : (a.beta_kind == 1 ? ld_in(bg, chain * L + g) : ld_in(bg, v_base + g * DV + i));
      }
      sm.Y[t][i] = yv;
      sm.dO[t][i] = dov;
      sm.bt[t][i] = bv;
    }
  };
  auto norms = [&]() {
    if (tid < BC) sm.nrm[tid] = row_dot(&sm.X[tid][0], &sm.X[tid][0], DK);
  };
  // per-row scalars of the chunk: eta, a, g (inclusive), gm, zeta; padded steps
  // and the fresh sequence's first step: eta = 0, a = 1
  auto row_scalars = [&](int i, long t0, int c, float (&eta)[BC], float (&av)[BC], float (&g)[BC],
                         float (&gm)[BC], float (&zeta)[BC]) {
    float gp = 1.0f;
#pragma unroll
    for (int t = 0; t < BC; ++t) {
      float e = 0.0f;
      if (t < c && !(fresh && t0 + t == 0)) e = sm.bt[t][i] / (a.eps + sm.nrm[t]);
      eta[t] = e;
      av[t] = 1.0f - e * a.lambda;
      gm[t] = gp;
      gp *= av[t];
      g[t] = gp;
      zeta[t] = e / gp;
    }
  };
  // forward solve of row i: z (and e, h)
  auto row_solve = [&](int i, const float (&gm)[BC], const float (&zeta)[BC], float (&e)[BC],
                       float (&z)[BC], float (&h)[BC]) {
#pragma unroll
    for (int t = 0; t < BC; ++t) {
      float hs = 0.0f;
      if (a.regression) {
#pragma unroll
        for (int s = 0; s < t; ++s) hs = __builtin_fmaf(sm.G[t][s], z[s], hs);
        e[t] = sm.Y[t][i] - gm[t] * (sm.XS[t][i] + hs);
      } else {
        e[t] = sm.Y[t][i];
      }
      h[t] = hs;
      z[t] = zeta[t] * e[t];
    }
  };

  // ================= forward sweep: chunk-start states =================
  for (int idx = tid; idx < DV * DK; idx += BNT) {
    const int i = idx / DK, kk = idx % DK;
    sm.S[i][kk] = a.S0 ? a.S0[(chain * DV + i) * DK + kk] : 0.0f;
  }
  for (int ci = 0; ci < nch; ++ci) {
    const long t0 = (long)ci * BC;
    const int c = (int)((L - t0) < BC ? (L - t0) : BC);
    load_chunk(t0, c, false);
    __syncthreads();
    for (int idx = tid; idx < DV * DK; idx += BNT) ws[(long)ci * DV * DK + idx] = sm.S[idx / DK][idx % DK];
    norms();
    if (a.regression) {
      for (int idx = tid; idx < BC * BC + BC * DV; idx += BNT) {
        if (idx < BC * BC) {
          const int t = idx / BC, s = idx % BC;
          sm.G[t][s] = s < t ? row_dot(&sm.X[t][0], &sm.X[s][0], DK) : 0.0f;
        } else {
          const int t = (idx - BC * BC) / DV, i = (idx - BC * BC) % DV;
          sm.XS[t][i] = row_dot(&sm.X[t][0], &sm.S[i][0], DK);
        }
      }
    }
    __syncthreads();
    if (tid < DV) {
      const int i = tid;
      float eta[BC], av[BC], g[BC], gm[BC], zeta[BC], e[BC], z[BC], h[BC];
      row_scalars(i, t0, c, eta, av, g, gm, zeta);
      row_solve(i, gm, zeta, e, z, h);
#pragma unroll
      for (int t = 0; t < BC; ++t) sm.Z[t][i] = z[t];
      sm.gC[i] = g[BC - 1];
    }
    __syncthreads();
    // S <- gC (S + Z^T X)
    for (int idx = tid; idx < DV * (DK / 4); idx += BNT) {
      const int i = idx / (DK / 4), k4 = 4 * (idx % (DK / 4));
      float4 acc = *reinterpret_cast<const float4*>(&sm.S[i][k4]);
#pragma unroll
      for (int t = 0; t < BC; ++t) {
        const float zv = sm.Z[t][i];
        const float4 xv = *reinterpret_cast<const float4*>(&sm.X[t][k4]);
        acc.x = __builtin_fmaf(zv, xv.x, acc.x);
        acc.y = __builtin_fmaf(zv, xv.y, acc.y);
        acc.z = __builtin_fmaf(zv, xv.z, acc.z);
        acc.w = __builtin_fmaf(zv, xv.w, acc.w);
      }
      const float gc = sm.gC[i];
      *reinterpret_cast<float4*>(&sm.S[i][k4]) = make_float4(gc * acc.x, gc * acc.y, gc * acc.z, gc * acc.w);
    }
    __syncthreads();
  }

  // ================= backward sweep =================
  for (int idx = tid; idx < DV * DK; idx += BNT) {
    const int i = idx / DK, kk = idx % DK;
    sm.dS[i][kk] = a.dS_L ? a.dS_L[(chain * DV + i) * DK + kk] : 0.0f;
  }
  if (ks == 1) {   // k_{L-1} only leaves the call as k_last
    for (int kk = tid; kk < DK; kk += BNT)
      a.dk[qk_base + (L - 1) * DK + kk] = a.dk_last ? a.dk_last[chain * DK + kk] : 0.0f;
  }
  for (int ci = nch - 1; ci >= 0; --ci) {
    const long t0 = (long)ci * BC;
    const int c = (int)((L - t0) < BC ? (L - t0) : BC);
    load_chunk(t0, c, true);
    for (int idx = tid; idx < DV * DK; idx += BNT) sm.S[idx / DK][idx % DK] = ws[(long)ci * DV * DK + idx];
    __syncthreads();
    // ---- dk-long products ----
    norms();
    for (int idx = tid; idx < 2 * BC * BC + 3 * BC * DV + DV; idx += BNT) {
      if (idx < BC * BC) {
        const int t = idx / BC, s = idx % BC;
        sm.G[t][s] = (a.regression && s < t) ? row_dot(&sm.X[t][0], &sm.X[s][0], DK) : 0.0f;
      } else if (idx < 2 * BC * BC) {
        const int t = (idx - BC * BC) / BC, s = (idx - BC * BC) % BC;
        sm.P[t][s] = s <= t ? row_dot(&sm.Q[t][0], &sm.X[s][0], DK) : 0.0f;
      } else if (idx < 2 * BC * BC + 3 * BC * DV) {
        const int r = idx - 2 * BC * BC;
        const int which = r / (BC * DV), t = (r % (BC * DV)) / DV, i = r % DV;
        if (which == 0) sm.XS[t][i] = row_dot(&sm.X[t][0], &sm.S[i][0], DK);
        else if (which == 1) sm.QS[t][i] = row_dot(&sm.Q[t][0], &sm.S[i][0], DK);
        else sm.XdS[t][i] = row_dot(&sm.X[t][0], &sm.dS[i][0], DK);
      } else {
        const int i = idx - 2 * BC * BC - 3 * BC * DV;
        sm.sds[i] = row_dot(&sm.S[i][0], &sm.dS[i][0], DK);
      }
    }
    __syncthreads();
    // ---- per-row sweeps ----
    if (tid < DV) {
      const int i = tid;
      float eta[BC], av[BC], g[BC], gm[BC], zeta[BC], e[BC], z[BC], h[BC];
      row_scalars(i, t0, c, eta, av, g, gm, zeta);
      row_solve(i, gm, zeta, e, z, h);
      const float gc = g[BC - 1];
      float gdo[BC], dg[BC], dz[BC], dzeta[BC], w[BC], dr[BC];
      float dgc = sm.sds[i];
#pragma unroll
      for (int t = 0; t < BC; ++t) {
        float oh = sm.QS[t][i];
#pragma unroll
        for (int s = 0; s <= t; ++s) oh = __builtin_fmaf(sm.P[t][s], z[s], oh);
        const float dov = sm.dO[t][i];
        gdo[t] = g[t] * dov;
        dg[t] = dov * oh;
        dgc = __builtin_fmaf(z[t], sm.XdS[t][i], dgc);
      }
#pragma unroll
      for (int s = 0; s < BC; ++s) {
        float acc = gc * sm.XdS[s][i];
#pragma unroll
        for (int t = s; t < BC; ++t) acc = __builtin_fmaf(sm.P[t][s], gdo[t], acc);
        dz[s] = acc;
        dzeta[s] = acc * e[s];
      }
      if (a.regression) {
#pragma unroll
        for (int s = BC - 1; s >= 0; --s) {
          float gs = 0.0f;
#pragma unroll
          for (int t = s + 1; t < BC; ++t) gs = __builtin_fmaf(sm.G[t][s], w[t], gs);
          dr[s] = zeta[s] * dz[s] - zeta[s] * gs;
          w[s] = gm[s] * dr[s];
          dzeta[s] -= e[s] * gs;
        }
        // terms through gm_t = g_{t-1} (t >= 1)
#pragma unroll
        for (int t = 1; t < BC; ++t) dg[t - 1] -= dr[t] * (h[t] + sm.XS[t][i]);
      } else {
#pragma unroll
        for (int s = 0; s < BC; ++s) {
          dr[s] = zeta[s] * dz[s];
          w[s] = 0.0f;
        }
      }
      float deta[BC];
#pragma unroll
      for (int t = 0; t < BC; ++t) {
        deta[t] = dzeta[t] / g[t];
        dg[t] -= dzeta[t] * zeta[t] / g[t];
      }
      dg[BC - 1] += dgc;
      float suf = 0.0f;
#pragma unroll
      for (int r = BC - 1; r >= 0; --r) {
        suf = __builtin_fmaf(dg[r], g[r], suf);
        deta[r] -= a.lambda * (suf / av[r]);
        if (r >= c || (fresh && t0 + r == 0)) deta[r] = 0.0f;
      }
#pragma unroll
      for (int t = 0; t < BC; ++t) {
        sm.Z[t][i] = z[t];
        sm.W[t][i] = w[t];
        sm.GD[t][i] = gdo[t];
        sm.DE[t][i] = deta[t];
        sm.ETA[t][i] = eta[t];
        if (t < c) {
          a.dv[v_base + (t0 + t) * DV + i] = dr[t];
          if (a.dbeta_t && a.beta_kind == 2)
            a.dbeta_t[v_base + (t0 + t) * DV + i] = deta[t] / (a.eps + sm.nrm[t]);
        }
      }
      sm.gC[i] = gc;
    }
    __syncthreads();
    // ---- sums over value rows ----
    for (int idx = tid; idx < 2 * BC * BC + BC; idx += BNT) {
      if (idx < BC * BC) {
        const int t = idx / BC, s = idx % BC;
        sm.dG[t][s] = (a.regression && s < t) ? -row_dot(&sm.W[t][0], &sm.Z[s][0], DV) : 0.0f;
      } else if (idx < 2 * BC * BC) {
        const int t = (idx - BC * BC) / BC, s = (idx - BC * BC) % BC;
        sm.dP[t][s] = s <= t ? row_dot(&sm.GD[t][0], &sm.Z[s][0], DV) : 0.0f;
      } else {
        const int t = idx - 2 * BC * BC;
        const float den = a.eps + sm.nrm[t];
        sm.dn[t] = -row_dot(&sm.DE[t][0], &sm.ETA[t][0], DV) / den;
        if (a.dbeta_t && a.beta_kind == 1 && t < c) {
          float sde = 0.0f;
          for (int i = 0; i < DV; ++i) sde += sm.DE[t][i];
          a.dbeta_t[chain * L + t0 + t] = sde / den;
        }
      }
    }
    __syncthreads();
    // ---- dq, dx (rows t, four columns per thread) ----
    for (int idx = tid; idx < 2 * BC * (DK / 4); idx += BNT) {
      const bool isq = idx < BC * (DK / 4);
      const int r = isq ? idx : idx - BC * (DK / 4);
      const int t = r / (DK / 4), k4 = 4 * (r % (DK / 4));
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      auto fma4 = [&](float cf, const float* row) {
        const float4 v4 = *reinterpret_cast<const float4*>(row + k4);
        acc.x = __builtin_fmaf(cf, v4.x, acc.x);
        acc.y = __builtin_fmaf(cf, v4.y, acc.y);
        acc.z = __builtin_fmaf(cf, v4.z, acc.z);
        acc.w = __builtin_fmaf(cf, v4.w, acc.w);
      };
      if (isq) {
        // dq_t = sum_i g_t do_t s0_i + sum_s dP_ts x_s
        for (int i = 0; i < DV; ++i) fma4(sm.GD[t][i], &sm.S[i][0]);
#pragma unroll
        for (int s = 0; s < BC; ++s) fma4(sm.dP[t][s], &sm.X[s][0]);
        if (t < c) *reinterpret_cast<float4*>(&a.dq[qk_base + (t0 + t) * DK + k4]) = acc;
      } else {
        // dx_t = sum_i (gC_i z_t ds_i - w_t s0_i) + sum_s (dG_ts + dG_st) x_s
        //        + sum_t' dP_t't q_t' + 2 dn_t x_t
        for (int i = 0; i < DV; ++i) {
          fma4(sm.gC[i] * sm.Z[t][i], &sm.dS[i][0]);
          fma4(-sm.W[t][i], &sm.S[i][0]);
        }
#pragma unroll
        for (int s = 0; s < BC; ++s) {
          fma4(sm.dG[t][s] + sm.dG[s][t], &sm.X[s][0]);
          fma4(sm.dP[s][t], &sm.Q[s][0]);
        }
        fma4(2.0f * sm.dn[t], &sm.X[t][0]);
        const long j = t0 + t - ks;    // x_t = k_j
        if (t < c) {
          if (j >= 0) {
            if (ks == 0 && j == L - 1 && a.dk_last) {
              const float4 dl = *reinterpret_cast<const float4*>(&a.dk_last[chain * DK + k4]);
              acc.x += dl.x; acc.y += dl.y; acc.z += dl.z; acc.w += dl.w;
            }
            *reinterpret_cast<float4*>(&a.dk[qk_base + j * DK + k4]) = acc;
          } else if (a.dk_prev) {
            *reinterpret_cast<float4*>(&a.dk_prev[chain * DK + k4]) = acc;
          }
        }
      }
    }
    __syncthreads();
    // ---- dS <- gC dS + sum_t g_t do_t q_t - sum_t w_t x_t (in place, per element) ----
    for (int idx = tid; idx < DV * (DK / 4); idx += BNT) {
      const int i = idx / (DK / 4), k4 = 4 * (idx % (DK / 4));
      const float gc = sm.gC[i];
      const float4 d0 = *reinterpret_cast<const float4*>(&sm.dS[i][k4]);
      float4 acc = make_float4(gc * d0.x, gc * d0.y, gc * d0.z, gc * d0.w);
#pragma unroll
      for (int t = 0; t < BC; ++t) {
        const float cq = sm.GD[t][i], cx = -sm.W[t][i];
        const float4 qv = *reinterpret_cast<const float4*>(&sm.Q[t][k4]);
        const float4 xv = *reinterpret_cast<const float4*>(&sm.X[t][k4]);
        acc.x = __builtin_fmaf(cq, qv.x, __builtin_fmaf(cx, xv.x, acc.x));
        acc.y = __builtin_fmaf(cq, qv.y, __builtin_fmaf(cx, xv.y, acc.y));
        acc.z = __builtin_fmaf(cq, qv.z, __builtin_fmaf(cx, xv.z, acc.z));
        acc.w = __builtin_fmaf(cq, qv.w, __builtin_fmaf(cx, xv.w, acc.w));
      }
      *reinterpret_cast<float4*>(&sm.dS[i][k4]) = acc;
    }
    __syncthreads();
  }
  if (a.dS0) {
    for (int idx = tid; idx < DV * DK; idx += BNT)
      a.dS0[(chain * DV + idx / DK) * DK + idx % DK] = sm.dS[idx / DK][idx % DK];
  }
}

template <typename T, int DK, int DV>
hipError_t launch_bwd3(const BwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((backward_kernel<T, DK, DV>), dim3((unsigned)((long)a.batch * a.heads)),
                     dim3(BNT), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int DK>
hipError_t launch_bwd_dv(const BwdArgs& a, hipStream_t stream) {
  switch (a.ndv) {
    case 16: return launch_bwd3<T, DK, 16>(a, stream);
    case 32: return launch_bwd3<T, DK, 32>(a, stream);
    case 64: return launch_bwd3<T, DK, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_bwd_dk(const BwdArgs& a, hipStream_t stream) {
  switch (a.ndk) {
    case 16: return launch_bwd_dv<T, 16>(a, stream);
    case 32: return launch_bwd_dv<T, 32>(a, stream);
    case 64: return launch_bwd_dv<T, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t backward_workspace_bytes(int batch, int heads, long seqlen, int dk, int dv) {
  const long nch = (seqlen + BC - 1) / BC;
  return (size_t)batch * heads * nch * dv * dk * sizeof(float);
}

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
  (void)hipGetLastError();
  if (a.dtype == 0) return launch_bwd_dk<uint16_t>(a, stream);
  return launch_bwd_dk<float>(a, stream);
}

}  // namespace falcon
