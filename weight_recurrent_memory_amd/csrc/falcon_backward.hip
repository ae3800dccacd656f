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
// then, with gains shared by the value rows, one wave forms the scalars and
// T = A^-1 and the waves share E = T R, its transpose dR = T^T dE and the
// per-step sums over rows that feed the scalar chain; with per-channel gains A
// differs per row and the sweeps run on one lane per value row.  Last the sums
// over rows (dG, dP, dn) and the dk-wide products (dq, dx, dS).  Every product
// is a 16x16 output tile on the fp32 matrix cores (v_mfma_f32_16x16x4_f32,
// exact fp32 products): with the K index of step j of a 16-wide block taken as
// 4 (lane / 16) + j, a lane feeds four steps from one 16-byte LDS read where
// the operand is contiguous in K.  Arithmetic is fp32 throughout.
#include "falcon_device.h"
#include "falcon_launch.h"

namespace falcon {
namespace {

constexpr int BC = 16;        // chunk length of the backward
constexpr int BNT = 512;
constexpr int BNW = BNT / 64;

template <int DK, int DV>
struct BwdLds {
  float S[DV][DK + 4];        // chunk-start state
  float dS[DV][DK + 4];       // gradient of the chunk-end state
  float X[BC][DK + 4];        // keys x_t (shifted)
  float Q[BC][DK + 4];
  float Y[BC][DV + 4];        // values
  float dO[BC][DV + 4];
  float bt[BC][DV];           // per-channel gain per step and row
  float bts[BC];              // shared gain per step
  float nrm[BC];
  float G[BC][BC + 4];        // strictly lower
  float P[BC][BC + 4];        // lower incl. diagonal
  float Tm[BC][BC + 4];       // A^-1 (shared gains)
  float XS[BC][DV + 4];       // s0_i . x_t
  float QS[BC][DV + 4];       // s0_i . q_t
  float XdS[BC][DV + 4];      // ds_i . x_t
  float sds[DV];              // s0_i . ds_i
  float E[BC][DV + 4];        // residuals (shared gains)
  float dZ[BC][DV + 4];
  float H[BC][DV + 4];        // sum_{s<t} G_ts z_s
  float Z[BC][DV + 4];
  float W[BC][DV + 4];        // gm_t dr_t (regression), 0 (inner product)
  float GD[BC][DV + 4];       // g_t do_t
  float DE[BC][DV + 4];       // d eta (per channel)
  float ETA[BC][DV + 4];
  float dxp[BC][DK + 4];      // partial dx
  float gC[DV];
  float sv[5][BC];            // shared scalars: eta, a, g, gm, zeta
  float part[4][DV / 16][BC];  // per row tile: sums over its 16 rows (dO o/g, z XdS, dgm, dzeta)
  float dG[BC][BC + 4];
  float dP[BC][BC + 4];
  float dn[BC];
};

// workgroup barrier that orders LDS only: global stores issued before it may
// still be in flight (nothing in the workgroup reads them back before a full
// __syncthreads)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// acc + (g of lane N of the same 16-lane row) * r: one DPP multiply-add; g comes
// straight from LDS (never written by the vector ALU, so no DPP wait states)
template <int N>
__device__ __forceinline__ float fmac_bcast(float acc, float g, float r) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(g), "v"(r), "i"(N));
  return acc;
}
// forward substitution x_M = rhs_M - om_M acc_M, acc_r += g_M[r] zs_M x_M
// (r > M), steps M.. of a 16-unknown system; lane m of a 16-lane row holds g_m[]
template <int M>
__device__ __forceinline__ void sweep16(float (&rhs)[16], float (&acc)[16], const float (&g)[16], const float (&om)[16],
                                        const float (&zs)[16]) {
  rhs[M] = __builtin_fmaf(-om[M], acc[M], rhs[M]);
  const float xm = zs[M] * rhs[M];
#pragma unroll
  for (int r = M + 1; r < 16; ++r) acc[r] = fmac_bcast<M>(acc[r], g[r], xm);
  if constexpr (M < 15) sweep16<M + 1>(rhs, acc, g, om, zs);
}
// v times the v of lane - N in the same 16-lane row (lanes whose source is
// outside the row keep v: the DPP bounds rule disables them)
template <int N>
__device__ __forceinline__ float row_shr_mul(float v) {
  asm("s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shr:%1 row_mask:0xf bank_mask:0xf" : "+v"(v) : "i"(N));
  return v;
}
template <int N>
__device__ __forceinline__ float row_shr_fill(float v, float fill) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill), __builtin_bit_cast(int, v),
                                                             0x110 + N, 0xF, 0xF, false));
}

// raw 16-byte register images of four elements (converted only when stored
// to LDS, so that a load in flight is not waited for at its issue)
__device__ __forceinline__ uint4 ldraw(const uint16_t* p, long i) {
  const uint2 w = *reinterpret_cast<const uint2*>(p + i);
  return make_uint4(w.x, w.y, 0u, 0u);
}
__device__ __forceinline__ uint4 ldraw(const float* p, long i) {
  return *reinterpret_cast<const uint4*>(p + i);
}
__device__ __forceinline__ float4 cvt4(uint4 r, const uint16_t*) {
  return make_float4(bf16_to_f32((uint16_t)(r.x & 0xFFFFu)), bf16_to_f32((uint16_t)(r.x >> 16)),
                     bf16_to_f32((uint16_t)(r.y & 0xFFFFu)), bf16_to_f32((uint16_t)(r.y >> 16)));
}
__device__ __forceinline__ float4 cvt4(uint4 r, const float*) {
  return make_float4(__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z), __uint_as_float(r.w));
}
__device__ __forceinline__ float4 ld4(const uint16_t* p, long i) {
  const uint2 w = *reinterpret_cast<const uint2*>(p + i);
  return make_float4(bf16_to_f32((uint16_t)(w.x & 0xFFFFu)), bf16_to_f32((uint16_t)(w.x >> 16)),
                     bf16_to_f32((uint16_t)(w.y & 0xFFFFu)), bf16_to_f32((uint16_t)(w.y >> 16)));
}
__device__ __forceinline__ float4 ld4(const float* p, long i) {
  return *reinterpret_cast<const float4*>(p + i);
}
__device__ __forceinline__ float4 f4(const float* p) { return *reinterpret_cast<const float4*>(p); }
// four consecutive rows r..r+3 of column c
template <int LD>
__device__ __forceinline__ float4 col4(const float (*m)[LD], int r, int c) {
  return make_float4(m[r][c], m[r + 1][c], m[r + 2][c], m[r + 3][c]);
}
__device__ __forceinline__ float dot4(const float4 a, const float4 b, float acc) {
  acc = __builtin_fmaf(a.x, b.x, acc);
  acc = __builtin_fmaf(a.y, b.y, acc);
  acc = __builtin_fmaf(a.z, b.z, acc);
  return __builtin_fmaf(a.w, b.w, acc);
}
__device__ __forceinline__ floatx4 mfma4(const float4 a, const float4 b, floatx4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
}
// acc (a 16x16 tile: lane l holds rows 4 (l / 16) + r, column l % 16) +=
// sum_{k < K} A(m, k) B(k, n); fa(m, k) / fb(k, n) return elements k..k+3
template <int K, class FA, class FB>
__device__ __forceinline__ floatx4 mtile(floatx4 acc, int lane, FA fa, FB fb) {
  const int mn = lane & 15, k4 = 4 * (lane >> 4);
#pragma unroll
  for (int kb = 0; kb < K; kb += 16) acc = mfma4(fa(mn, kb + k4), fb(kb + k4, mn), acc);
  return acc;
}

template <typename T, int DK, int DV, bool PERROW>
__global__ __launch_bounds__(BNT) void backward_kernel(BwdArgs a) {
  using SM = BwdLds<DK, DV>;
  constexpr int GX = BC * DK / 4, GY = BC * DV / 4, GS = DV * DK / 4;
  constexpr int NIB = DV / 16, NKB = DK / 16;     // row and column tiles
  __shared__ __align__(16) SM sm;
  const T* __restrict__ qg = static_cast<const T*>(a.q);
  const T* __restrict__ kg = static_cast<const T*>(a.k);
  const T* __restrict__ vg = static_cast<const T*>(a.v);
  const T* __restrict__ kpg = static_cast<const T*>(a.k_prev);
  const T* __restrict__ bg = static_cast<const T*>(a.beta_t);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int mn = lane & 15, rq = 4 * (lane >> 4);   // tile column, first tile row of the lane
  const long chain = blockIdx.x;
  const long L = a.seqlen;
  const int nch = (int)((L + BC - 1) / BC);
  const int ks = a.key_shift;
  const bool fresh = ks == 1 && kpg == nullptr;
  const long qk_base = chain * L * DK;
  const long v_base = chain * L * DV;
  // workspace per chunk: start state, S0 x, Gram, (shared gains) T and scalars
  constexpr int WS_XS = DV * DK, WS_G = WS_XS + BC * DV, WS_T = WS_G + BC * BC;
  constexpr int WS_SV = WS_T + BC * BC, WS_CHUNK = WS_SV + 5 * BC;
  float* __restrict__ ws = a.workspace + chain * (long)nch * WS_CHUNK;
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // ---- chunk inputs: issue_chunk starts every global load of a chunk into
  // registers (bwd: also q, dO and the chunk's workspace record: start state,
  // S0 x, Gram, T, scalars); commit_chunk stores them to LDS.  A chunk's loads
  // are issued one chunk ahead, so they fly while the previous chunk computes.
  constexpr int NG = 2 * GX + 2 * GY + (PERROW ? GY : 0) + WS_CHUNK / 4;
  constexpr int NPER = (NG + BNT - 1) / BNT;
  // buffer resources (per chain; a range-checked load past the end, or at the
  // parked offset, returns 0), so every load is issued unconditionally
  constexpr int BUF_WORD3 = 0x00020000;
  constexpr uint32_t PARKED = 0xC0000000u;
  constexpr uint32_t ES = sizeof(T);
  auto rsrc = [](const void* base, long bytes) __attribute__((always_inline)) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, BUF_WORD3);
  };
  const auto rsk = rsrc(kg + qk_base, L * DK * ES);
  const auto rsq = rsrc(qg + qk_base, L * DK * ES);
  const auto rsv = rsrc(vg + v_base, L * DV * ES);
  const auto rsdo = rsrc(a.dO + v_base, L * DV * 4);
  const auto rsb = PERROW ? rsrc(bg + v_base, L * DV * ES)
                         : (a.beta_kind == 1 ? rsrc(bg + chain * L, L * ES) : rsrc(vg, 0));
  const auto rsws = rsrc(ws, (long)nch * WS_CHUNK * 4);
  auto ldr_t = [&](__amdgpu_buffer_rsrc_t r, uint32_t off) __attribute__((always_inline)) {
    if constexpr (sizeof(T) == 2) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
      return make_uint4(v[0], v[1], 0u, 0u);
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
      return make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  auto ldr_f = [&](__amdgpu_buffer_rsrc_t r, uint32_t off) __attribute__((always_inline)) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  auto issue_chunk = [&](uint4 (&val)[NPER], uint32_t& bval, int ci, bool bwd) {
    const long t0 = (long)ci * BC;
    const int c = (int)((L - t0) < BC ? (L - t0) : BC);
#pragma unroll
    for (int u = 0; u < NPER; ++u) {
      const int g = tid + u * BNT;
      uint4 v;
      if (g < 2 * GX) {
        const int r = g < GX ? g : g - GX;
        const int t = r / (DK / 4), k4 = 4 * (r % (DK / 4));
        const long st = t0 + t;
        if (g < GX) {   // x_t = k_{t - ks}; the carried key x_0 is put in at commit
          const bool in = t < c && st >= ks;
          v = ldr_t(rsk, in ? (uint32_t)(((st - ks) * DK + k4) * ES) : PARKED);
        } else {
          v = ldr_t(rsq, (bwd && t < c) ? (uint32_t)((st * DK + k4) * ES) : PARKED);
        }
      } else if (g < 2 * GX + 2 * GY + (PERROW ? GY : 0)) {
        const int r0 = g - 2 * GX;
        const int which = r0 / GY, r = r0 % GY;
        const int t = r / (DV / 4), i4 = 4 * (r % (DV / 4));
        const long st = t0 + t;
        const bool in = t < c;
        if (which == 0) v = ldr_t(rsv, in ? (uint32_t)((st * DV + i4) * ES) : PARKED);
        else if (which == 1) v = ldr_f(rsdo, (in && bwd) ? (uint32_t)((st * DV + i4) * 4) : PARKED);
        else v = ldr_t(rsb, in ? (uint32_t)((st * DV + i4) * ES) : PARKED);
      } else {
        const int e = 4 * (g - (NG - WS_CHUNK / 4));
        v = ldr_f(rsws, (bwd && g < NG) ? (uint32_t)(((long)ci * WS_CHUNK + e) * 4) : PARKED);
      }
      val[u] = v;
    }
    bval = 0u;
    if (!PERROW && a.beta_kind == 1)
      bval = __builtin_amdgcn_raw_buffer_load_b16(rsb, (tid < c && tid < BC) ? (uint32_t)((t0 + tid) * ES) : PARKED, 0, 0);
  };
  auto commit_chunk = [&](const uint4 (&val)[NPER], uint32_t bval, int ci, bool bwd) {
#pragma unroll
    for (int u = 0; u < NPER; ++u) {
      const int g = tid + u * BNT;
      if (g < 2 * GX) {
        const int r = g < GX ? g : g - GX;
        const int t = r / (DK / 4), k4 = 4 * (r % (DK / 4));
        *reinterpret_cast<float4*>(g < GX ? &sm.X[t][k4] : &sm.Q[t][k4]) = cvt4(val[u], kg);
      } else if (g < 2 * GX + 2 * GY + (PERROW ? GY : 0)) {
        const int r0 = g - 2 * GX;
        const int which = r0 / GY, r = r0 % GY;
        const int t = r / (DV / 4), i4 = 4 * (r % (DV / 4));
        if (which == 0) *reinterpret_cast<float4*>(&sm.Y[t][i4]) = cvt4(val[u], vg);
        else if (which == 1) *reinterpret_cast<float4*>(&sm.dO[t][i4]) = cvt4(val[u], a.dO);
        else *reinterpret_cast<float4*>(&sm.bt[t][i4]) = cvt4(val[u], bg);
      } else if (g < NG) {
        const float4 v = cvt4(val[u], a.dO);
        if (bwd) {
          const int e = 4 * (g - (NG - WS_CHUNK / 4));
          float* dst;
          if (e < WS_XS) dst = &sm.S[e / DK][e % DK];
          else if (e < WS_G) dst = &sm.XS[(e - WS_XS) / DV][(e - WS_XS) % DV];
          else if (e < WS_T) dst = &sm.G[(e - WS_G) / BC][(e - WS_G) % BC];
          else if (e < WS_SV) dst = &sm.Tm[(e - WS_T) / BC][(e - WS_T) % BC];
          else dst = &sm.sv[(e - WS_SV) / BC][(e - WS_SV) % BC];
          *reinterpret_cast<float4*>(dst) = v;
        }
      }
    }
    if (!PERROW && tid < BC) {
      float b = a.beta;
      if (a.beta_kind == 1) {
        if constexpr (sizeof(T) == 2) b = bf16_to_f32((uint16_t)bval);
        else b = 0.0f;   // fp32 gains take the 4-byte path below
      }
      sm.bts[tid] = b;
    }
    if constexpr (sizeof(T) == 4) {
      if (!PERROW && a.beta_kind == 1 && tid < BC) {
        const long t0 = (long)ci * BC;
        sm.bts[tid] = t0 + tid < L ? ld_in(bg, chain * L + t0 + tid) : 0.0f;
      }
    }
    if (ci == 0 && ks == 1 && kpg && tid < DK / 4)   // the carried key is x_0
      *reinterpret_cast<float4*>(&sm.X[0][4 * tid]) = ld4(kpg, chain * DK + 4 * tid);
  };
  auto nrm_and = [&]() {
    if (tid < BC) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < DK; k += 4) acc = dot4(f4(&sm.X[tid][k]), f4(&sm.X[tid][k]), acc);
      sm.nrm[tid] = acc;
    }
  };
  // forward sweep: Gram (strictly lower) and S0 x tiles, also into the workspace
  auto gram_tile = [&](float* wsc) {
    const floatx4 acc = mtile<DK>(zero4, lane, [&](int m, int k) { return f4(&sm.X[m][k]); },
                                  [&](int k, int n) { return f4(&sm.X[n][k]); });
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = rq + r, s2 = mn;
      const float gv = (a.regression && s2 < t) ? acc[r] : 0.0f;
      sm.G[t][s2] = gv;
      wsc[WS_G + t * BC + s2] = gv;
    }
  };
  auto xs_tile = [&](int ib, float* wsc) {
    const floatx4 acc = mtile<DK>(zero4, lane, [&](int m, int k) { return f4(&sm.X[m][k]); },
                                  [&](int k, int n) { return f4(&sm.S[16 * ib + n][k]); });
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = rq + r, i = 16 * ib + mn;
      sm.XS[t][i] = acc[r];
      wsc[WS_XS + t * DV + i] = acc[r];
    }
  };
  // shared gains, one wave (lane t of each 16-lane row): eta, a, g, gm, zeta,
  // and T = A^-1, A_ts = [t==s] + gm_t G_ts zeta_s (s < t), column j on lane j
  auto shared_scalars_and_inverse = [&](long t0, int c, float* wsc) {
    const int t = lane & 15;
    float eta = 0.0f;
    if (t < c && !(fresh && t0 + t == 0)) eta = sm.bts[t] / (a.eps + sm.nrm[t]);
    const float av = 1.0f - eta * a.lambda;
    float g = av;
    g = row_shr_mul<1>(g);
    g = row_shr_mul<2>(g);
    g = row_shr_mul<4>(g);
    g = row_shr_mul<8>(g);
    const float gm = row_shr_fill<1>(g, 1.0f);
    const float zeta = eta / g;
    if (lane < 16) {
      sm.sv[0][t] = eta;
      sm.sv[1][t] = av;
      sm.sv[2][t] = g;
      sm.sv[3][t] = gm;
      sm.sv[4][t] = zeta;
    }
    // lane m holds column m of the strictly lower Gram; column j of T on lane j:
    // x_r = [r == j] - gm_r sum_{s<r} G_rs zeta_s x_s
    float gcol[BC], om[BC], zs[BC], rhs[BC], acc[BC];
#pragma unroll
    for (int r = 0; r < BC; ++r) {
      gcol[r] = sm.G[r][t];
      om[r] = sm.sv[3][r];
      zs[r] = sm.sv[4][r];
      rhs[r] = r == t ? 1.0f : 0.0f;
      acc[r] = 0.0f;
    }
    sweep16<0>(rhs, acc, gcol, om, zs);
    if (lane < 16) {
#pragma unroll
      for (int r = 0; r < BC; ++r) {
        sm.Tm[r][t] = rhs[r];
        wsc[WS_T + r * BC + t] = rhs[r];
      }
      wsc[WS_SV + t] = eta;
      wsc[WS_SV + BC + t] = av;
      wsc[WS_SV + 2 * BC + t] = g;
      wsc[WS_SV + 3 * BC + t] = gm;
      wsc[WS_SV + 4 * BC + t] = zeta;
    }
  };
  // E = T R with R = Y - gm XS (regression; T = I and R = Y for the inner
  // product), Z = zeta E: row tiles ib on waves 0..NIB-1
  auto shared_residual_tile = [&](int ib) {
    {
      floatx4 acc = zero4;
      if (a.regression) {
        acc = mtile<BC>(zero4, lane, [&](int m, int k) { return f4(&sm.Tm[m][k]); },
                        [&](int k, int n) {
                          const int i = 16 * ib + n;
                          return make_float4(sm.Y[k][i] - sm.sv[3][k] * sm.XS[k][i],
                                             sm.Y[k + 1][i] - sm.sv[3][k + 1] * sm.XS[k + 1][i],
                                             sm.Y[k + 2][i] - sm.sv[3][k + 2] * sm.XS[k + 2][i],
                                             sm.Y[k + 3][i] - sm.sv[3][k + 3] * sm.XS[k + 3][i]);
                        });
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = sm.Y[rq + r][16 * ib + mn];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = rq + r, i = 16 * ib + mn;
        sm.E[t][i] = acc[r];
        sm.Z[t][i] = sm.sv[4][t] * acc[r];
      }
    }
  };
  // backward sweep: q.x (lower incl. diagonal), S0 q, dS x tiles, (shared gains)
  // E = T R tiles; s0.ds, the key norms and g_t do_t on the vector ALU
  auto bwd_products = [&]() {
    const int ntile = 1 + 2 * NIB + (PERROW ? 0 : NIB);
    for (int tt = wave; tt < ntile; tt += BNW) {
      if (tt == 0) {
        const floatx4 acc = mtile<DK>(zero4, lane, [&](int m, int k) { return f4(&sm.Q[m][k]); },
                                      [&](int k, int n) { return f4(&sm.X[n][k]); });
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.P[rq + r][mn] = mn <= rq + r ? acc[r] : 0.0f;
      } else if (tt < 1 + 2 * NIB) {
        const int kind = (tt - 1) / NIB, ib = (tt - 1) % NIB;
        const floatx4 acc = mtile<DK>(zero4, lane, [&](int m, int k) { return f4(kind == 0 ? &sm.Q[m][k] : &sm.X[m][k]); },
                                      [&](int k, int n) { return f4(kind == 1 ? &sm.dS[16 * ib + n][k] : &sm.S[16 * ib + n][k]); });
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (kind == 0) sm.QS[rq + r][16 * ib + mn] = acc[r];
          else sm.XdS[rq + r][16 * ib + mn] = acc[r];
        }
      } else {
        shared_residual_tile(tt - 1 - 2 * NIB);
      }
    }
    nrm_and();
    if (tid >= BNT - DV) {
      const int i = tid - (BNT - DV);
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < DK; k += 4) acc = dot4(f4(&sm.S[i][k]), f4(&sm.dS[i][k]), acc);
      sm.sds[i] = acc;
    }
    if (!PERROW) {
      for (int idx = tid; idx < BC * DV; idx += BNT)
        sm.GD[idx / DV][idx % DV] = sm.sv[2][idx / DV] * sm.dO[idx / DV][idx % DV];
    }
  };
  // sum over the 16 columns of a tile row (lanes of one 16-lane row), written
  // by the row's first lane
  auto tile_row_sums = [&](float (&dst)[BC], const float (&v)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float s2 = group_sum<16>(v[r]);
      if (mn == 0) dst[rq + r] = s2;
    }
  };
  // per-channel: scalars of row i (eta, a, g, gm, zeta)
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
  // per-channel: forward solve of row i
  auto row_solve = [&](int i, const float (&gm)[BC], const float (&zeta)[BC], float (&e)[BC],
                       float (&z)[BC], float (&h)[BC]) {
#pragma unroll
    for (int t = 0; t < BC; ++t) {
      float hs = 0.0f;
      if (a.regression) {
#pragma unroll
        for (int s2 = 0; s2 < t; ++s2) hs = __builtin_fmaf(sm.G[t][s2], z[s2], hs);
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
  uint4 pre[NPER];
  uint32_t pre_b;
  issue_chunk(pre, pre_b, 0, false);
  for (int ci = 0; ci < nch; ++ci) {
    const long t0 = (long)ci * BC;
    const int c = (int)((L - t0) < BC ? (L - t0) : BC);
    commit_chunk(pre, pre_b, ci, false);
    lds_barrier();
    if (ci + 1 < nch) issue_chunk(pre, pre_b, ci + 1, false);
    // record the chunk for the backward sweep: start state (all threads); wave 0:
    // Gram, key norms and (shared gains) scalars and T; waves 1..NIB: S0 x tiles
    float* __restrict__ wsc = ws + (long)ci * WS_CHUNK;
    for (int idx = tid; idx < GS; idx += BNT) {
      const int e = 4 * idx;
      *reinterpret_cast<float4*>(wsc + e) = *reinterpret_cast<const float4*>(&sm.S[e / DK][e % DK]);
    }
    if (wave == 0) {
      if (a.regression) gram_tile(wsc);
      else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sm.G[rq + r][mn] = 0.0f;
          wsc[WS_G + (rq + r) * BC + mn] = 0.0f;
        }
      }
      nrm_and();
      if (!PERROW) shared_scalars_and_inverse(t0, c, wsc);
    } else if (wave <= NIB) {
      xs_tile(wave - 1, wsc);
    }
    lds_barrier();
    if constexpr (!PERROW) {
      if (wave < NIB) shared_residual_tile(wave);
      if (tid < DV) sm.gC[tid] = sm.sv[2][BC - 1];
    } else {
      if (tid < DV) {
        const int i = tid;
        float eta[BC], av[BC], g[BC], gm[BC], zeta[BC], e[BC], z[BC], h[BC];
        row_scalars(i, t0, c, eta, av, g, gm, zeta);
        row_solve(i, gm, zeta, e, z, h);
#pragma unroll
        for (int t = 0; t < BC; ++t) sm.Z[t][i] = z[t];
        sm.gC[i] = g[BC - 1];
      }
    }
    lds_barrier();
    // S <- gC (S + Z^T X): tiles (ib, kb)
    for (int tt = wave; tt < NIB * NKB; tt += BNW) {
      const int ib = tt / NKB, kb = tt % NKB;
      floatx4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = sm.S[16 * ib + rq + r][16 * kb + mn];
      acc = mtile<BC>(acc, lane, [&](int m, int k) { return col4(sm.Z, k, 16 * ib + m); },
                      [&](int k, int n) { return col4(sm.X, k, 16 * kb + n); });
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ib + rq + r;
        sm.S[i][16 * kb + mn] = sm.gC[i] * acc[r];
      }
    }
    lds_barrier();
  }

  // the workspace records written above are read back by other threads below
  __syncthreads();
  // ================= backward sweep =================
  for (int idx = tid; idx < DV * DK; idx += BNT) {
    const int i = idx / DK, kk = idx % DK;
    sm.dS[i][kk] = a.dS_L ? a.dS_L[(chain * DV + i) * DK + kk] : 0.0f;
  }
  if (ks == 1) {   // k_{L-1} only leaves the call as k_last
    for (int kk = tid; kk < DK; kk += BNT)
      a.dk[qk_base + (L - 1) * DK + kk] = a.dk_last ? a.dk_last[chain * DK + kk] : 0.0f;
  }
  issue_chunk(pre, pre_b, nch - 1, true);
  for (int ci = nch - 1; ci >= 0; --ci) {
    const long t0 = (long)ci * BC;
    const int c = (int)((L - t0) < BC ? (L - t0) : BC);
    commit_chunk(pre, pre_b, ci, true);
    lds_barrier();
    if (ci > 0) issue_chunk(pre, pre_b, ci - 1, true);
    bwd_products();
    lds_barrier();
    if constexpr (!PERROW) {
      // ---- gains shared by the rows: matrix form ----
      // H = L(G) Z;  o/g = QS + P Z (sum over rows of dO o/g);  dZ = P^T GD + gC XdS
      // (and the sum over rows of Z XdS): tiles (kind, ib)
      {
        const float gc = sm.sv[2][BC - 1];
        for (int tt = wave; tt < 3 * NIB; tt += BNW) {
          const int kind = tt / NIB, ib = tt % NIB;
          floatx4 acc;
          float v[4];
          if (kind == 0) {
            acc = mtile<BC>(zero4, lane, [&](int m, int k) { return f4(&sm.G[m][k]); },
                            [&](int k, int n) { return col4(sm.Z, k, 16 * ib + n); });
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.H[rq + r][16 * ib + mn] = acc[r];
          } else if (kind == 1) {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = sm.QS[rq + r][16 * ib + mn];
            acc = mtile<BC>(acc, lane, [&](int m, int k) { return f4(&sm.P[m][k]); },
                            [&](int k, int n) { return col4(sm.Z, k, 16 * ib + n); });
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = sm.dO[rq + r][16 * ib + mn] * acc[r];
            tile_row_sums(sm.part[0][ib], v);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = gc * sm.XdS[rq + r][16 * ib + mn];
            acc = mtile<BC>(acc, lane, [&](int m, int k) { return col4(sm.P, k, m); },
                            [&](int k, int n) { return col4(sm.GD, k, 16 * ib + n); });
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = rq + r, i = 16 * ib + mn;
              sm.dZ[t][i] = acc[r];
              v[r] = sm.Z[t][i] * sm.XdS[t][i];
            }
            tile_row_sums(sm.part[1][ib], v);
          }
        }
      }
      lds_barrier();
      // dR = T^T (zeta dZ); W = gm dR (regression); dv = dR; sum over rows of -dR (H + XS)
      if (wave < NIB) {
        const int ib = wave;
        floatx4 acc = mtile<BC>(zero4, lane, [&](int m, int k) { return col4(sm.Tm, k, m); },
                                [&](int k, int n) {
                                  const int i = 16 * ib + n;
                                  return make_float4(sm.sv[4][k] * sm.dZ[k][i], sm.sv[4][k + 1] * sm.dZ[k + 1][i],
                                                     sm.sv[4][k + 2] * sm.dZ[k + 2][i], sm.sv[4][k + 3] * sm.dZ[k + 3][i]);
                                });
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s2 = rq + r, i = 16 * ib + mn;
          const float dr = acc[r];
          sm.W[s2][i] = a.regression ? sm.sv[3][s2] * dr : 0.0f;
          if (s2 < c) a.dv[v_base + (t0 + s2) * DV + i] = dr;
          v[r] = a.regression ? -dr * (sm.H[s2][i] + sm.XS[s2][i]) : 0.0f;
        }
        tile_row_sums(sm.part[2][ib], v);
      }
      lds_barrier();
      // sum over rows of E (dZ - L(G)^T W); dG = -L(W Z^T); dP = lower(GD Z^T)
      for (int tt = wave; tt < NIB + 2; tt += BNW) {
        if (tt < NIB) {
          const int ib = tt;
          const floatx4 acc = mtile<BC>(zero4, lane, [&](int m, int k) { return col4(sm.G, k, m); },
                                        [&](int k, int n) { return col4(sm.W, k, 16 * ib + n); });
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int s2 = rq + r, i = 16 * ib + mn;
            v[r] = sm.E[s2][i] * (sm.dZ[s2][i] - acc[r]);
          }
          tile_row_sums(sm.part[3][ib], v);
        } else {
          const bool dg = tt == NIB;
          const floatx4 acc = mtile<DV>(zero4, lane, [&](int m, int k) { return f4(dg ? &sm.W[m][k] : &sm.GD[m][k]); },
                                        [&](int k, int n) { return f4(&sm.Z[n][k]); });
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = rq + r, s2 = mn;
            if (dg) sm.dG[t][s2] = (a.regression && s2 < t) ? -acc[r] : 0.0f;
            else sm.dP[t][s2] = s2 <= t ? acc[r] : 0.0f;
          }
        }
      }
      lds_barrier();
      // scalar chain (one wave, lane t of each 16-lane row)
      if (wave == 0) {
        const int t = lane & 15;
        const float g = sm.sv[2][t], zeta = sm.sv[4][t], eta = sm.sv[0][t];
        float sdgo = 0.0f, szx = 0.0f, sdzeta = 0.0f;
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) {
          sdgo += sm.part[0][ib][t];
          szx += sm.part[1][ib][t];
          sdzeta += sm.part[3][ib][t];
        }
        float sdgm_next = 0.0f;
        if (t + 1 < BC) {
#pragma unroll
          for (int ib = 0; ib < NIB; ++ib) sdgm_next += sm.part[2][ib][t + 1];
        }
        float dgc = szx;
        for (int i = t; i < DV; i += 16) dgc += sm.sds[i];
        dgc = group_sum<16>(dgc);
        float dg = sdgo - sdzeta * zeta / g + sdgm_next;
        if (t == BC - 1) dg += dgc;
        float suf = dg * g;
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) {
          const float o = __shfl_down(suf, d, 16);
          if (t + d < 16) suf += o;
        }
        float deta = sdzeta / g - a.lambda * (suf / sm.sv[1][t]);
        if (t >= c || (fresh && t0 + t == 0)) deta = 0.0f;
        const float den = a.eps + sm.nrm[t];
        if (lane < 16) {
          sm.dn[t] = -deta * eta / den;
          if (a.dbeta_t && t < c) a.dbeta_t[chain * L + t0 + t] = deta / den;
        }
        if (tid < DV) sm.gC[tid] = sm.sv[2][BC - 1];
      }
      lds_barrier();
    } else {
      // ---- per-channel gains: one lane per value row ----
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
          for (int s2 = 0; s2 <= t; ++s2) oh = __builtin_fmaf(sm.P[t][s2], z[s2], oh);
          const float dov = sm.dO[t][i];
          gdo[t] = g[t] * dov;
          dg[t] = dov * oh;
          dgc = __builtin_fmaf(z[t], sm.XdS[t][i], dgc);
        }
#pragma unroll
        for (int s2 = 0; s2 < BC; ++s2) {
          float acc = gc * sm.XdS[s2][i];
#pragma unroll
          for (int t = s2; t < BC; ++t) acc = __builtin_fmaf(sm.P[t][s2], gdo[t], acc);
          dz[s2] = acc;
          dzeta[s2] = acc * e[s2];
        }
        if (a.regression) {
#pragma unroll
          for (int s2 = BC - 1; s2 >= 0; --s2) {
            float gs = 0.0f;
#pragma unroll
            for (int t = s2 + 1; t < BC; ++t) gs = __builtin_fmaf(sm.G[t][s2], w[t], gs);
            dr[s2] = zeta[s2] * dz[s2] - zeta[s2] * gs;
            w[s2] = gm[s2] * dr[s2];
            dzeta[s2] -= e[s2] * gs;
          }
          // terms through gm_t = g_{t-1} (t >= 1)
#pragma unroll
          for (int t = 1; t < BC; ++t) dg[t - 1] -= dr[t] * (h[t] + sm.XS[t][i]);
        } else {
#pragma unroll
          for (int s2 = 0; s2 < BC; ++s2) {
            dr[s2] = zeta[s2] * dz[s2];
            w[s2] = 0.0f;
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
            if (a.dbeta_t) a.dbeta_t[v_base + (t0 + t) * DV + i] = deta[t] / (a.eps + sm.nrm[t]);
          }
        }
        sm.gC[i] = gc;
      }
      lds_barrier();
      // ---- sums over value rows: dG, dP (matrix cores), dn ----
      for (int tt = wave; tt < 2; tt += BNW) {
        const bool dg = tt == 0;
        const floatx4 acc = mtile<DV>(zero4, lane, [&](int m, int k) { return f4(dg ? &sm.W[m][k] : &sm.GD[m][k]); },
                                      [&](int k, int n) { return f4(&sm.Z[n][k]); });
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = rq + r, s2 = mn;
          if (dg) sm.dG[t][s2] = (a.regression && s2 < t) ? -acc[r] : 0.0f;
          else sm.dP[t][s2] = s2 <= t ? acc[r] : 0.0f;
        }
      }
      if (tid >= BNT - BC) {
        const int t = tid - (BNT - BC);
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < DV; k += 4) acc = dot4(f4(&sm.DE[t][k]), f4(&sm.ETA[t][k]), acc);
        sm.dn[t] = -acc / (a.eps + sm.nrm[t]);
      }
      lds_barrier();
    }
    // ---- dq and dx, column tiles kb: waves 0..NKB-1 take dq and the gC z ds part
    // of dx (to LDS); waves NKB..2NKB-1 the rest of dx, completed after the barrier
    floatx4 dxr = zero4;
    const bool dxw = wave >= NKB && wave < 2 * NKB;
    if (wave < NKB) {
      const int kb = wave;
      // dq_t = sum_i g_t do_t s0_i + sum_s dP_ts x_s
      floatx4 acc = mtile<DV>(zero4, lane, [&](int m, int k) { return f4(&sm.GD[m][k]); },
                              [&](int k, int n) { return col4(sm.S, k, 16 * kb + n); });
      acc = mtile<BC>(acc, lane, [&](int m, int k) { return f4(&sm.dP[m][k]); },
                      [&](int k, int n) { return col4(sm.X, k, 16 * kb + n); });
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = rq + r;
        if (t < c) a.dq[qk_base + (t0 + t) * DK + 16 * kb + mn] = acc[r];
      }
      // sum_i gC_i z_t ds_i
      acc = mtile<DV>(zero4, lane, [&](int m, int k) {
                        const float4 z4 = f4(&sm.Z[m][k]);
                        const float4 g4 = f4(&sm.gC[k]);
                        return make_float4(g4.x * z4.x, g4.y * z4.y, g4.z * z4.z, g4.w * z4.w);
                      },
                      [&](int k, int n) { return col4(sm.dS, k, 16 * kb + n); });
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.dxp[rq + r][16 * kb + mn] = acc[r];
    } else if (dxw) {
      const int kb = wave - NKB;
      // -sum_i w_t s0_i + sum_s (dG_ts + dG_st) x_s + sum_t' dP_t't q_t'
      dxr = mtile<DV>(zero4, lane, [&](int m, int k) {
                        const float4 w4 = f4(&sm.W[m][k]);
                        return make_float4(-w4.x, -w4.y, -w4.z, -w4.w);
                      },
                      [&](int k, int n) { return col4(sm.S, k, 16 * kb + n); });
      dxr = mtile<BC>(dxr, lane, [&](int m, int k) {
                        return make_float4(sm.dG[m][k] + sm.dG[k][m], sm.dG[m][k + 1] + sm.dG[k + 1][m],
                                           sm.dG[m][k + 2] + sm.dG[k + 2][m], sm.dG[m][k + 3] + sm.dG[k + 3][m]);
                      },
                      [&](int k, int n) { return col4(sm.X, k, 16 * kb + n); });
      dxr = mtile<BC>(dxr, lane, [&](int m, int k) { return col4(sm.dP, k, m); },
                      [&](int k, int n) { return col4(sm.Q, k, 16 * kb + n); });
    }
    lds_barrier();
    if (dxw) {
      const int kb = wave - NKB;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = rq + r, kk = 16 * kb + mn;
        float v = dxr[r] + sm.dxp[t][kk] + 2.0f * sm.dn[t] * sm.X[t][kk];
        const long j = t0 + t - ks;    // x_t = k_j
        if (t < c) {
          if (j >= 0) {
            if (ks == 0 && j == L - 1 && a.dk_last) v += a.dk_last[chain * DK + kk];
            a.dk[qk_base + j * DK + kk] = v;
          } else if (a.dk_prev) {
            a.dk_prev[chain * DK + kk] = v;
          }
        }
      }
    }
    // ---- dS <- gC dS + sum_t g_t do_t q_t - sum_t w_t x_t: tiles (ib, kb); every
    // reader of dS finished before the barrier above ----
    for (int tt = wave; tt < NIB * NKB; tt += BNW) {
      const int ib = tt / NKB, kb = tt % NKB;
      floatx4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ib + rq + r;
        acc[r] = sm.gC[i] * sm.dS[i][16 * kb + mn];
      }
      acc = mtile<BC>(acc, lane, [&](int m, int k) { return col4(sm.GD, k, 16 * ib + m); },
                      [&](int k, int n) { return col4(sm.Q, k, 16 * kb + n); });
      acc = mtile<BC>(acc, lane, [&](int m, int k) {
                        const float4 w4 = col4(sm.W, k, 16 * ib + m);
                        return make_float4(-w4.x, -w4.y, -w4.z, -w4.w);
                      },
                      [&](int k, int n) { return col4(sm.X, k, 16 * kb + n); });
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.dS[16 * ib + rq + r][16 * kb + mn] = acc[r];
    }
    lds_barrier();
  }
  if (a.dS0) {
    for (int idx = tid; idx < DV * DK; idx += BNT)
      a.dS0[(chain * DV + idx / DK) * DK + idx % DK] = sm.dS[idx / DK][idx % DK];
  }
}

template <typename T, int DK, int DV>
hipError_t launch_bwd3(const BwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((long)a.batch * a.heads));
  if (a.beta_kind == 2)
    hipLaunchKernelGGL((backward_kernel<T, DK, DV, true>), grid, dim3(BNT), 0, stream, a);
  else
    hipLaunchKernelGGL((backward_kernel<T, DK, DV, false>), grid, dim3(BNT), 0, stream, a);
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
  // per chunk: start state, S0 x, Gram, T, five per-step scalars (fp32)
  const long nch = (seqlen + BC - 1) / BC;
  const long per_chunk = (long)dv * dk + (long)BC * dv + 2L * BC * BC + 5L * BC;
  return (size_t)batch * heads * nch * per_chunk * sizeof(float);
}

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
  (void)hipGetLastError();
  if (a.dtype == 0) return launch_bwd_dk<uint16_t>(a, stream);
  return launch_bwd_dk<float>(a, stream);
}

}  // namespace falcon
