// falcon_backward.hip - gradients of the chunk form (every variant; window 1, or
// sliding windows of 2..8 samples for Falcon-3/3A) on gfx950.
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
// One workgroup (8 waves) per (batch*head) chain and slice of up to 32 value rows
// holds that slice of the state and its gradient in LDS; the sums over value rows
// (dq, dk, a per-token gain's gradient) are partial per slice and a second kernel
// adds them in slice order.  Windows: the unknowns are (step, window slot) pairs,
// 16 per chunk of floor(16 / window) steps, with the same per-row sweeps.  A
// forward sweep over 16-step chunks stores each chunk's starting state in the
// caller's workspace; the backward sweep walks the chunks in reverse, reloads
// that state, recomputes the chunk's forward quantities and carries dS.  Per
// chunk: dk-long dot products (Gram, q.x, S0 x, S0 q, dS x) on the matrix
// cores; then each value row runs its own triangular sweeps (forward for z,
// transposed for dr) and its scalar chain on one 16-lane row, lane t = step t,
// with DPP broadcasts and shifts in place of LDS round trips, so shared,
// per-token and per-channel gains take the same path.  Last the sums over rows
// (dG, dP, dn) and the dk-wide products (dq, dx, dS).  Every product is a 16x16
// output tile on the fp32 matrix cores (v_mfma_f32_16x16x4_f32, exact fp32
// products): with the K index of step j of a 16-wide block taken as
// 4 (lane / 16) + j, a lane feeds four steps from one 16-byte LDS read where
// the operand is contiguous in K.  The chunk-start records (state, S0 x, Gram)
// written by the forward sweep come back through the workspace.  Arithmetic is
// fp32 throughout.
#include "falcon_device.h"
#include "falcon_exact.h"
#include "falcon_launch.h"
#include "falcon_mma.h"

namespace falcon {
namespace {

constexpr int BC = 16;        // chunk length of the backward
constexpr int BNT = 512;
constexpr int BNW = BNT / 64;

template <int DK, int RB, int BW>
struct BwdLds {
  static constexpr int WR = BW > 1 ? BC : 1;     // rows of the window-only arrays
  static constexpr int WH = BW > 1 ? BW - 1 : 1;
  static constexpr int KP = DK + 4, VP = RB + 4, BP = BC + 4;   // fp32 row pitches
  float S[RB][KP];        // chunk-start state
  float dS[RB][KP];       // gradient of the chunk-end state
  float X[BC][KP];        // key tile: samples t0 - (B-1) + k (shifted keys)
  float Q[BC][KP];
  float Y[BC][VP];        // values
  float dO[BC][VP];
  float bt[BC][RB];           // gain per step and row
  float nrm[BC];              // squared norms of the key tile rows
  float nsum[BC];             // per step: window sums of the squared norms
  float XU[WR][KP];       // window: the key of each unknown (step, slot)
  float DR[WR][VP];       // window: d y per unknown
  float dxh[2][WH][DK];       // window: d x of the samples before the chunk (to the next one)
  float dyh[2][WH][RB];
  float G[BC][BP];        // strictly lower
  float P[BC][BP];        // lower incl. diagonal
  float XS[BC][VP];       // s0_i . x_t
  float QS[BC][VP];       // s0_i . q_t
  float XdS[BC][VP];      // ds_i . x_t
  float sds[RB];              // s0_i . ds_i
  float E[BC][VP];        // residuals
  float dZ[BC][VP];
  float H[BC][VP];        // sum_{s<t} G_ts z_s
  float Z[BC][VP];
  float W[BC][VP];        // gm_t dr_t (regression), 0 (inner product)
  float GD[BC][VP];       // g_t do_t
  float DE[BC][VP];       // d eta
  float DGO[BC][VP];      // do_t (o_t / g_t)
  float ETA[BC][VP];
  float dxp[BC][KP];      // partial dx
  float gC[RB];
  float dG[BC][BP];
  float dP[BC][BP];
  float dn[BC];
  int bad;                // some chunk's decay products left the range
};

// workgroup barrier that orders LDS only: global stores issued before it may
// still be in flight (nothing in the workgroup reads them back before a full
// __syncthreads)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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

// acc + g * (v of lane N of the same 16-lane row) with v just written by the
// vector ALU (the nop gives the two wait states a DPP read of it needs)
template <int N>
__device__ __forceinline__ float fmac_bcast_nop(float acc, float v, float g) {
  asm("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(acc) : "v"(v), "v"(g), "i"(N));
  return acc;
}
// v of lane 15 of the same 16-lane row on every lane of the row
__device__ __forceinline__ float row_last(float v) {
  float r;
  asm("s_nop 1\n\tv_mov_b32_dpp %0, %1 row_newbcast:15 row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(v));
  return r;
}
template <int N>
__device__ __forceinline__ float row_shl_fill(float v, float fill) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill), __builtin_bit_cast(int, v),
                                                             0x100 + N, 0xF, 0xF, false));
}
// Per-row sweeps, one value row per 16-lane row, lane t = step t of the chunk.
// Forward: e_t = y_t - gm_t (xs_t + acc_t), z_t = zeta_t e_t with acc_t =
// sum_{s<t} G_ts z_s; every lane forms its candidate z and step M takes lane M's
// (grow = the lane's Gram row, zero at and above the diagonal).
// With a window the lanes are unknowns and the BW unknowns of one step do not
// couple (their Gram entries are zero), so the pivots of a step share one
// candidate: a sweep has ceil(16 / BW) dependent stages of BW multiply-adds, in
// pivot order as before.
template <int M, int E>   // acc += v(lane m) g[m], m = M .. E-1
__device__ __forceinline__ void fmacs_up(float& acc, float v, const float (&g)[16]) {
  acc = fmac_bcast_nop<M>(acc, v, g[M]);
  if constexpr (M + 1 < E) fmacs_up<M + 1, E>(acc, v, g);
}
template <int M, int E>   // the same for m = E-1 down to M
__device__ __forceinline__ void fmacs_down(float& acc, float v, const float (&g)[16]) {
  acc = fmac_bcast_nop<E - 1>(acc, v, g[E - 1]);
  if constexpr (E - 1 > M) fmacs_down<M, E - 1>(acc, v, g);
}
template <int BW, int S>
__device__ __forceinline__ void fsweep(float& acc, const float (&grow)[16], float y, float xs, float gm, float zeta) {
  constexpr int M = BW * S, E = M + BW < 16 ? M + BW : 16;
  const float zc = zeta * (y - gm * (xs + acc));
  fmacs_up<M, E>(acc, zc, grow);
  if constexpr (E < 16) fsweep<BW, S + 1>(acc, grow, y, xs, gm, zeta);
}
// Transposed: dr_s = zeta_s (dz_s - acc2_s), w_s = gm_s dr_s with acc2_s =
// sum_{t>s} G_ts w_t, pivots 15 .. 0 (gcol = the lane's Gram column)
template <int BW, int S>
__device__ __forceinline__ void bsweep(float& acc2, const float (&gcol)[16], float dz, float gm, float zeta) {
  constexpr int M = BW * S, E = M + BW < 16 ? M + BW : 16;
  const float wc = gm * zeta * (dz - acc2);
  fmacs_down<M, E>(acc2, wc, gcol);
  if constexpr (S > 0) bsweep<BW, S - 1>(acc2, gcol, dz, gm, zeta);
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

template <typename T, int DK, int RB, int BW>
__global__ __launch_bounds__(BNT) void backward_kernel(BwdArgs a) {
  using SM = BwdLds<DK, RB, BW>;
  // unknowns u = BW s + w (step s of the chunk, window slot w) on the 16 lanes of a
  // row; the chunk has NS steps and a key tile of NK rows (the BW-1 samples
  // before it, then its own); the key of u is tile row kt(u) = BW-1 + s - w.  When
  // BW does not divide 16 the lanes past the last step (u >= NU, all in step NS)
  // are idle: their keys are zero, so every quantity they hold stays 0.
  constexpr int NS = BC / BW, NK = BW - 1 + NS, NU = BW * NS;
  static_assert(BW >= 1 && BW <= 8, "window 1..8");
  constexpr int GX = BC * DK / 4, GY = BC * RB / 4, GS = RB * DK / 4;
  constexpr int NIB = RB / 16, NKB = DK / 16;     // row and column tiles
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
  // workgroup = (chain, slice of RB value rows); the slices of a chain share an XCD
  const int dvf = a.ndv, nrg = dvf / RB;
  long chain;
  int rg;
  {
    const int b = blockIdx.x;
    const int nchain = a.batch * a.heads;
    if (nchain % 8 == 0) {
      const int xcd = b & 7, slot = b >> 3;
      chain = xcd + 8 * (slot / nrg);
      rg = slot % nrg;
    } else {
      chain = b / nrg;
      rg = b % nrg;
    }
  }
  const int i0 = rg * RB;                          // first value row of the slice
  const long L = a.seqlen;
  const int nch = (int)((L + NS - 1) / NS);
  const int ks = a.key_shift;
  const bool fresh = ks == 1 && kpg == nullptr;
  const long qk_base = chain * L * DK;
  const long v_base = chain * L * dvf;
  // workspace per chunk: start state, S0 x, Gram
  constexpr int WS_XS = RB * DK, WS_G = WS_XS + BC * RB, WS_CHUNK = WS_G + BC * BC;
  float* __restrict__ ws = a.workspace + (chain * nrg + rg) * (long)nch * WS_CHUNK;
  // cross-row sums (dq, dk, dk_prev, per-token dbeta): with several slices each
  // writes its partial sums to the workspace (after the chunk records) and a
  // second kernel adds them in slice order; with one slice, straight to the outputs
  const long BH = (long)a.batch * a.heads;
  float* __restrict__ part = a.workspace + BH * nrg * (long)nch * WS_CHUNK;
  const bool split = nrg > 1;
  float* __restrict__ oq = split ? part + rg * (BH * L * DK) : a.dq;
  float* __restrict__ ok = split ? part + (nrg + rg) * (BH * L * DK) : a.dk;
  float* __restrict__ okp = split ? (a.dk_prev ? part + 2 * nrg * (BH * L * DK) + rg * (BH * DK) : nullptr) : a.dk_prev;
  float* __restrict__ odb = split ? ((a.dbeta_t && a.beta_kind == 1)
                                         ? part + 2 * nrg * (BH * L * DK) + nrg * (BH * DK) + rg * (BH * L)
                                         : nullptr)
                                 : a.dbeta_t;
  const float* __restrict__ dkl = split ? nullptr : a.dk_last;   // with slices, added by the sum kernel
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  // the keys as the unknowns see them (window 1: the tile itself)
  float (*XU)[SM::KP] = BW == 1 ? sm.X : sm.XU;
  const float* nsum = BW == 1 ? sm.nrm : sm.nsum;

  // ---- chunk inputs: issue_chunk starts every global load of a chunk into
  // registers (bwd: also q, dO and the chunk's workspace record: start state,
  // S0 x, Gram); commit_chunk stores them to LDS.  A chunk's loads
  // are issued one chunk ahead, so they fly while the previous chunk computes.
  constexpr int NG = 2 * GX + 2 * GY + GY + WS_CHUNK / 4;
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
  const auto rsv = rsrc(vg + v_base, L * dvf * ES);
  const auto rsdo = rsrc(a.dO + v_base, L * dvf * 4);
  const auto rsb = a.beta_kind == 2 ? rsrc(bg + v_base, L * dvf * ES)
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
  auto issue_chunk = [&](uint4 (&val)[NPER], int ci, bool bwd) {
    const long t0 = (long)ci * NS;
    const int c = (int)((L - t0) < NS ? (L - t0) : NS);
#pragma unroll
    for (int u = 0; u < NPER; ++u) {
      const int g = tid + u * BNT;
      uint4 v;
      if (g < 2 * GX) {
        const int r = g < GX ? g : g - GX;
        const int t = r / (DK / 4), k4 = 4 * (r % (DK / 4));
        const long st = t0 + t;
        if (g < GX) {   // tile row t: sample j, x_j = k_{j - ks}; the carried key x_0 is put in at commit
          const long j = t0 - (BW - 1) + t;
          const bool in = t < NK && j >= ks && j < L;
          v = ldr_t(rsk, in ? (uint32_t)(((j - ks) * DK + k4) * ES) : PARKED);
        } else {
          v = ldr_t(rsq, (bwd && t < c) ? (uint32_t)((st * DK + k4) * ES) : PARKED);
        }
      } else if (g < 2 * GX + 2 * GY + GY) {
        const int r0 = g - 2 * GX;
        const int which = r0 / GY, r = r0 % GY;
        const int t = r / (RB / 4), i4 = 4 * (r % (RB / 4));
        const long st = t0 + t;
        const bool in = t < c;
        const long j = t0 - (BW - 1) + t;     // values: tile row t is sample j
        if (which == 0) v = ldr_t(rsv, (t < NK && j >= 0 && j < L) ? (uint32_t)((j * dvf + i0 + i4) * ES) : PARKED);
        else if (which == 1) v = ldr_f(rsdo, (in && bwd) ? (uint32_t)((st * dvf + i0 + i4) * 4) : PARKED);
        else if (a.beta_kind == 2) v = ldr_t(rsb, in ? (uint32_t)((st * dvf + i0 + i4) * ES) : PARKED);
        else if (a.beta_kind == 1) {   // per-token gain of step t, for every row
          uint32_t b;
          if constexpr (sizeof(T) == 2) b = __builtin_amdgcn_raw_buffer_load_b16(rsb, in ? (uint32_t)(st * ES) : PARKED, 0, 0);
          else b = __builtin_amdgcn_raw_buffer_load_b32(rsb, in ? (uint32_t)(st * ES) : PARKED, 0, 0);
          v = make_uint4(b, 0u, 0u, 0u);
        } else {
          v = make_uint4(0u, 0u, 0u, 0u);
        }
      } else {
        const int e = 4 * (g - (NG - WS_CHUNK / 4));
        v = ldr_f(rsws, (bwd && g < NG) ? (uint32_t)(((long)ci * WS_CHUNK + e) * 4) : PARKED);
      }
      val[u] = v;
    }
  };
  auto commit_chunk = [&](const uint4 (&val)[NPER], int ci, bool bwd) {
    // the carried key is x_0: tile row BW-1 of chunk 0, and a halo row of the
    // next chunks while the window still reaches sample 0 (windows above NS + 1);
    // written by the thread that owns the row's piece
    const int r0 = (ks == 1 && kpg) ? BW - 1 - ci * NS : -1;
#pragma unroll
    for (int u = 0; u < NPER; ++u) {
      const int g = tid + u * BNT;
      if (g < 2 * GX) {
        const int r = g < GX ? g : g - GX;
        const int t = r / (DK / 4), k4 = 4 * (r % (DK / 4));
        if (g < GX && t == r0) *reinterpret_cast<float4*>(&sm.X[t][k4]) = ld4(kpg, chain * DK + k4);
        else *reinterpret_cast<float4*>(g < GX ? &sm.X[t][k4] : &sm.Q[t][k4]) = cvt4(val[u], kg);
      } else if (g < 2 * GX + 2 * GY + GY) {
        const int r0 = g - 2 * GX;
        const int which = r0 / GY, r = r0 % GY;
        const int t = r / (RB / 4), i4 = 4 * (r % (RB / 4));
        if (which == 0) *reinterpret_cast<float4*>(&sm.Y[t][i4]) = cvt4(val[u], vg);
        else if (which == 1) *reinterpret_cast<float4*>(&sm.dO[t][i4]) = cvt4(val[u], a.dO);
        else {
          float4 b4;
          if (a.beta_kind == 2) {
            b4 = cvt4(val[u], bg);
          } else {
            float b = a.beta;
            if (a.beta_kind == 1) {
              if constexpr (sizeof(T) == 2) b = bf16_to_f32((uint16_t)val[u].x);
              else b = __uint_as_float(val[u].x);
            }
            b4 = make_float4(b, b, b, b);
          }
          *reinterpret_cast<float4*>(&sm.bt[t][i4]) = b4;
        }
      } else if (g < NG) {
        const float4 v = cvt4(val[u], a.dO);
        if (bwd) {
          const int e = 4 * (g - (NG - WS_CHUNK / 4));
          float* dst;
          if (e < WS_XS) dst = &sm.S[e / DK][e % DK];
          else if (e < WS_G) dst = &sm.XS[(e - WS_XS) / RB][(e - WS_XS) % RB];
          else dst = &sm.G[(e - WS_G) / BC][(e - WS_G) % BC];
          *reinterpret_cast<float4*>(dst) = v;
        }
      }
    }
  };
  // after a commit: the unknowns' keys (window) and, on wave 0, the tile's
  // squared norms and their window sums per step
  auto gather = [&]() {
    if constexpr (BW > 1) {
      for (int idx = tid; idx < BC * DK / 4; idx += BNT) {
        const int u = idx / (DK / 4), k4 = 4 * (idx % (DK / 4));
        const int s = u / BW, w = u % BW;
        *reinterpret_cast<float4*>(&sm.XU[u][k4]) =
            u < NU ? f4(&sm.X[BW - 1 + s - w][k4]) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    // key norms; with window 1 on wave BNW - 2, which has no product tile in
    // either sweep (the windowed gather above needs a barrier first anyway)
    constexpr int GT0 = BW == 1 ? 64 * (BNW - 2) : 0;
    if (tid >= GT0 && tid < GT0 + BC) {
      const int t = tid - GT0;
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < DK; k += 4) acc = dot4(f4(&sm.X[t][k]), f4(&sm.X[t][k]), acc);
      sm.nrm[t] = acc;
      if constexpr (BW > 1) {
        wave_sync();
        float n = 0.0f;
#pragma unroll
        for (int w = 0; w < BW; ++w) n += t < NS ? sm.nrm[BW - 1 + t - w] : 0.0f;
        sm.nsum[t] = n;
      }
    }
  };
  // forward sweep: Gram (strictly lower) and S0 x tiles, also into the workspace
  auto gram_tile = [&](float* wsc) {
    const floatx4 acc = mtile<DK>(zero4, lane, [&](int m, int k) { return f4(&XU[m][k]); },
                                  [&](int k, int n) { return f4(&XU[n][k]); });
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = rq + r, s2 = mn;   // unknowns: only earlier steps couple
      const float gv = (a.regression && s2 / BW < t / BW) ? acc[r] : 0.0f;
      sm.G[t][s2] = gv;
      wsc[WS_G + t * BC + s2] = gv;
    }
  };
  auto xs_tile = [&](int ib, float* wsc) {
    const floatx4 acc = mtile<DK>(zero4, lane, [&](int m, int k) { return f4(&XU[m][k]); },
                                  [&](int k, int n) { return f4(&sm.S[16 * ib + n][k]); });
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = rq + r, i = 16 * ib + mn;
      sm.XS[t][i] = acc[r];
      wsc[WS_XS + t * RB + i] = acc[r];
    }
  };
  // backward sweep: q.x (lower incl. diagonal), S0 q, dS x tiles; s0.ds and the
  // key norms on the vector ALU
  auto bwd_products = [&]() {
    const int ntile = 1 + 2 * NIB;
    for (int tt = wave; tt < ntile; tt += BNW) {
      if (tt == 0) {
        const floatx4 acc = mtile<DK>(zero4, lane, [&](int m, int k) { return f4(&sm.Q[m][k]); },
                                      [&](int k, int n) { return f4(&XU[n][k]); });
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.P[rq + r][mn] = mn / BW <= rq + r ? acc[r] : 0.0f;   // [step][unknown]
      } else {
        const int kind = (tt - 1) / NIB, ib = (tt - 1) % NIB;
        const floatx4 acc = mtile<DK>(zero4, lane, [&](int m, int k) { return f4(kind == 0 ? &sm.Q[m][k] : &XU[m][k]); },
                                      [&](int k, int n) { return f4(kind == 1 ? &sm.dS[16 * ib + n][k] : &sm.S[16 * ib + n][k]); });
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (kind == 0) sm.QS[rq + r][16 * ib + mn] = acc[r];
          else sm.XdS[rq + r][16 * ib + mn] = acc[r];
        }
      }
    }
    if (tid >= BNT - RB) {
      const int i = tid - (BNT - RB);
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < DK; k += 4) acc = dot4(f4(&sm.S[i][k]), f4(&sm.dS[i][k]), acc);
      sm.sds[i] = acc;
    }
  };
  // lane u of the 16-lane row of value row i (unknown u, step s = u / BW): eta,
  // a, g (prefix product by DPP row shifts over the lanes, each step's factor
  // entering once, on its slot-0 lane), gm = g_{s-1}, zeta
  struct RowScal { float eta, av, g, gm, zeta; };
  auto row_scal_dpp = [&](int i, long t0, int c) __attribute__((always_inline)) {
    const int u = lane & 15, s = u / BW;
    RowScal r;
    r.eta = 0.0f;
    if (s < c && !(fresh && t0 + s == 0)) r.eta = sm.bt[s][i] / (a.eps + nsum[s]);
    r.av = 1.0f - r.eta * a.lambda;
    float g = (u % BW == 0) ? r.av : 1.0f;
    g = row_shr_mul<1>(g);
    g = row_shr_mul<2>(g);
    g = row_shr_mul<4>(g);
    g = row_shr_mul<8>(g);
    r.g = g;
    if constexpr (BW == 1) {
      r.gm = row_shr_fill<1>(g, 1.0f);
    } else {   // g at the last lane of the previous step
      const float gp = __shfl(g, (lane & 48) | ((s * BW + 15) & 15));
      r.gm = s == 0 ? 1.0f : gp;
    }
    r.zeta = r.eta / g;
    if (gauge_out_of_range(g, r.av)) sm.bad = 1;
    return r;
  };
  // forward sweep of value row i (lane t): z (and for the backward e, h, eta,
  // g do) into LDS, gC
  auto row_forward = [&](int i, const RowScal& r, bool bwd) __attribute__((always_inline)) {
    const int t = lane & 15;   // unknown
    const int s = t / BW;
    const float y = sm.Y[BW - 1 + s - t % BW][i], xs = sm.XS[t][i];
    float acc = 0.0f;
    if (a.regression) {
      float grow[16];
#pragma unroll
      for (int m = 0; m < 16; ++m) grow[m] = sm.G[t][m];
      fsweep<BW, 0>(acc, grow, y, xs, r.gm, r.zeta);
    }
    const float e = a.regression ? y - r.gm * (xs + acc) : y;
    sm.Z[t][i] = r.zeta * e;
    if (bwd) {
      sm.E[t][i] = e;
      sm.H[t][i] = acc;
      if (t % BW == 0) {   // step quantities
        sm.ETA[s][i] = r.eta;
        sm.GD[s][i] = r.g * sm.dO[s][i];
      }
    }
    const float gc = row_last(r.g);
    if (t == 0) sm.gC[i] = gc;
  };
  // ================= forward sweep: chunk-start states =================
  // LDS starts as zeros: rows of the last, partial chunk that the sweeps read
  // without writing (padded steps, idle window lanes) then hold zeros, not
  // whatever an earlier workgroup left there
  for (int idx = tid; idx < (int)(sizeof(SM) / sizeof(float)); idx += BNT) reinterpret_cast<float*>(&sm)[idx] = 0.0f;
  __syncthreads();
  for (int idx = tid; idx < RB * DK; idx += BNT) {
    const int i = idx / DK, kk = idx % DK;
    sm.S[i][kk] = a.S0 ? a.S0[(chain * dvf + i0 + i) * DK + kk] : 0.0f;
  }
  uint4 pre[NPER];
  issue_chunk(pre, 0, false);
  for (int ci = 0; ci < nch; ++ci) {
    const long t0 = (long)ci * NS;
    const int c = (int)((L - t0) < NS ? (L - t0) : NS);
    commit_chunk(pre, ci, false);
    lds_barrier();
    if (ci + 1 < nch) issue_chunk(pre, ci + 1, false);
    if constexpr (BW > 1) {
      gather();
      lds_barrier();
    }
    // record the chunk for the backward sweep: start state (all threads); wave 0:
    // Gram and key norms; waves 1..NIB: S0 x tiles
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
    } else if (wave <= NIB) {
      xs_tile(wave - 1, wsc);
    }
    if constexpr (BW == 1) gather();
    lds_barrier();
    for (int i = 4 * wave + (lane >> 4); i < RB; i += 4 * BNW) row_forward(i, row_scal_dpp(i, t0, c), false);
    lds_barrier();
    // S <- gC (S + Z^T X): tiles (ib, kb)
    for (int tt = wave; tt < NIB * NKB; tt += BNW) {
      const int ib = tt / NKB, kb = tt % NKB;
      floatx4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = sm.S[16 * ib + rq + r][16 * kb + mn];
      acc = mtile<BC>(acc, lane, [&](int m, int k) { return col4(sm.Z, k, 16 * ib + m); },
                      [&](int k, int n) { return col4(XU, k, 16 * kb + n); });
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
  for (int idx = tid; idx < RB * DK; idx += BNT) {
    const int i = idx / DK, kk = idx % DK;
    sm.dS[i][kk] = a.dS_L ? a.dS_L[(chain * dvf + i0 + i) * DK + kk] : 0.0f;
  }
  if (ks == 1 && !split) {   // k_{L-1} only leaves the call as k_last
    for (int kk = tid; kk < DK; kk += BNT)
      a.dk[qk_base + (L - 1) * DK + kk] = a.dk_last ? a.dk_last[chain * DK + kk] : 0.0f;
  }
  if constexpr (BW > 1) {   // no later chunk: nothing carried into the last one
    for (int idx = tid; idx < 2 * (BW - 1) * DK; idx += BNT) (&sm.dxh[0][0][0])[idx] = 0.0f;
    for (int idx = tid; idx < 2 * (BW - 1) * RB; idx += BNT) (&sm.dyh[0][0][0])[idx] = 0.0f;
  }
  issue_chunk(pre, nch - 1, true);
  for (int ci = nch - 1; ci >= 0; --ci) {
    const long t0 = (long)ci * NS;
    const int c = (int)((L - t0) < NS ? (L - t0) : NS);
    commit_chunk(pre, ci, true);
    lds_barrier();
    if (ci > 0) issue_chunk(pre, ci - 1, true);
    if constexpr (BW > 1) {
      gather();
      lds_barrier();
    } else {
      gather();   // the key norms
    }
    bwd_products();
    lds_barrier();
    // ---- per-row sweeps on 16-lane DPP rows, shared products on the matrix cores ----
    for (int i = 4 * wave + (lane >> 4); i < RB; i += 4 * BNW) row_forward(i, row_scal_dpp(i, t0, c), true);
    lds_barrier();
    // o/g = QS + P Z (kept as do o/g), dZ = P^T GD + gC XdS: tiles (kind, ib)
    for (int tt = wave; tt < 2 * NIB; tt += BNW) {
      const int kind = tt / NIB, ib = tt % NIB;
      floatx4 acc;
      if (kind == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = sm.QS[rq + r][16 * ib + mn];
        acc = mtile<BC>(acc, lane, [&](int m, int k) { return f4(&sm.P[m][k]); },
                        [&](int k, int n) { return col4(sm.Z, k, 16 * ib + n); });
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.DGO[rq + r][16 * ib + mn] = sm.dO[rq + r][16 * ib + mn] * acc[r];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = sm.gC[16 * ib + mn] * sm.XdS[rq + r][16 * ib + mn];
        acc = mtile<BC>(acc, lane, [&](int m, int k) { return col4(sm.P, k, m); },
                        [&](int k, int n) { return col4(sm.GD, k, 16 * ib + n); });
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.dZ[rq + r][16 * ib + mn] = acc[r];
      }
    }
    lds_barrier();
    // transposed sweep and the scalar chain of each row (lane t of its 16-lane row)
    for (int i = 4 * wave + (lane >> 4); i < RB; i += 4 * BNW) {
      const int t = lane & 15;
      const RowScal r = row_scal_dpp(i, t0, c);
      const float dz = sm.dZ[t][i], e = sm.E[t][i];
      float acc2 = 0.0f;
      if (a.regression) {
        float gcol[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) gcol[m] = sm.G[m][t];
        bsweep<BW, 15 / BW>(acc2, gcol, dz, r.gm, r.zeta);
      }
      const float dr = r.zeta * (dz - acc2);
      const float w = a.regression ? r.gm * dr : 0.0f;
      float dzeta = e * (dz - acc2);
      float dgm = a.regression ? -dr * (sm.H[t][i] + sm.XS[t][i]) : 0.0f;
      const int s = t / BW;
      if constexpr (BW > 1) {   // step sums over the step's window slots (lanes of a group)
        if constexpr (BW == 2 || BW == 4) {
          dzeta += __shfl_xor(dzeta, 1);
          dgm += __shfl_xor(dgm, 1);
          if constexpr (BW == 4) {
            dzeta += __shfl_xor(dzeta, 2);
            dgm += __shfl_xor(dgm, 2);
          }
        } else {   // gather from the group, in slot order
          const int g0 = (lane & 48) | (s < NS ? s * BW : 0);
          float sz = 0.0f, sg = 0.0f;
#pragma unroll
          for (int w = 0; w < BW; ++w) {
            sz += __shfl(dzeta, g0 + w);
            sg += __shfl(dgm, g0 + w);
          }
          dzeta = s < NS ? sz : 0.0f;   // idle lanes
          dgm = s < NS ? sg : 0.0f;
        }
      }
      // d gC: s0.ds + sum_t z_t (x_t . ds), a row sum
      float zx = sm.Z[t][i] * sm.XdS[t][i];
      zx += row_shr_fill<1>(zx, 0.0f);
      zx += row_shr_fill<2>(zx, 0.0f);
      zx += row_shr_fill<4>(zx, 0.0f);
      zx += row_shr_fill<8>(zx, 0.0f);
      const float dgc = row_last(zx) + sm.sds[i];
      // dgm of the next step (gm_{s+1} = g_s) is BW lanes up
      float dg = sm.DGO[s][i] - dzeta * r.zeta / r.g + row_shl_fill<BW>(dgm, 0.0f);
      if (s == NS - 1) dg += dgc;
      // suffix sums over steps s' >= s of dg g (one lane per step, its last slot)
      float suf = (t % BW == BW - 1) ? dg * r.g : 0.0f;
      suf += row_shl_fill<1>(suf, 0.0f);
      suf += row_shl_fill<2>(suf, 0.0f);
      suf += row_shl_fill<4>(suf, 0.0f);
      suf += row_shl_fill<8>(suf, 0.0f);
      float deta = dzeta / r.g - a.lambda * (suf / r.av);
      if (s >= c || (fresh && t0 + s == 0)) deta = 0.0f;
      sm.W[t][i] = w;
      if (t % BW == 0) sm.DE[s][i] = deta;
      if constexpr (BW == 1) {
        if (t < c) {
          a.dv[v_base + (t0 + t) * dvf + i0 + i] = dr;
          if (a.dbeta_t && a.beta_kind == 2) a.dbeta_t[v_base + (t0 + t) * dvf + i0 + i] = deta / (a.eps + sm.nrm[t]);
        }
      } else {
        sm.DR[t][i] = dr;   // d y of the unknown's sample, summed per sample below
      }
    }
    lds_barrier();
    // ---- sums over value rows: dG, dP (matrix cores), dn ----
    for (int tt = wave; tt < 2; tt += BNW) {
      const bool dg = tt == 0;
      const floatx4 acc = mtile<RB>(zero4, lane, [&](int m, int k) { return f4(dg ? &sm.W[m][k] : &sm.GD[m][k]); },
                                    [&](int k, int n) { return f4(&sm.Z[n][k]); });
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = rq + r, s2 = mn;
        if (dg) sm.dG[t][s2] = (a.regression && s2 / BW < t / BW) ? -acc[r] : 0.0f;
        else sm.dP[t][s2] = s2 / BW <= t ? acc[r] : 0.0f;   // [step][unknown]
      }
    }
    if (tid >= BNT - BC) {
      const int t = tid - (BNT - BC);
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < RB; k += 4) acc = dot4(f4(&sm.DE[t][k]), f4(&sm.ETA[t][k]), acc);
      sm.dn[t] = -acc / (a.eps + nsum[t]);   // per step
      if (odb && a.beta_kind == 1 && t < c) {   // a per-token gain feeds every row
        float sde = 0.0f;
#pragma unroll
        for (int k = 0; k < RB; k += 4) {
          const float4 d4 = f4(&sm.DE[t][k]);
          sde += d4.x + d4.y + d4.z + d4.w;
        }
        odb[chain * L + t0 + t] = sde / (a.eps + nsum[t]);
      }
    }
    lds_barrier();
    // ---- dq and dx by column tiles kb ----
    // dx of unknown t, column kk: to the key's gradient (window 1) or to LDS for the
    // per-sample sums (windows)
    auto dx_out = [&](int t, int kk, float v) __attribute__((always_inline)) {
      if constexpr (BW == 1) {
        const long j = t0 + t - ks;    // x_t = k_j
        if (t < c) {
          if (j >= 0) {
            if (ks == 0 && j == L - 1 && dkl) v += dkl[chain * DK + kk];
            ok[qk_base + j * DK + kk] = v;
          } else if (okp) {
            okp[chain * DK + kk] = v;
          }
        }
      } else {
        sm.dxp[t][kk] = v;   // d x of the unknown's key, summed per sample below
      }
    };
    auto dq_tile = [&](int kb) __attribute__((always_inline)) {
      // dq_t = sum_i g_t do_t s0_i + sum_s dP_ts x_s
      floatx4 acc = mtile<RB>(zero4, lane, [&](int m, int k) { return f4(&sm.GD[m][k]); },
                              [&](int k, int n) { return col4(sm.S, k, 16 * kb + n); });
      acc = mtile<BC>(acc, lane, [&](int m, int k) { return f4(&sm.dP[m][k]); },
                      [&](int k, int n) { return col4(XU, k, 16 * kb + n); });
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = rq + r;
        if (t < c) oq[qk_base + (t0 + t) * DK + 16 * kb + mn] = acc[r];
      }
    };
    auto dx_gz = [&](int kb) __attribute__((always_inline)) {   // sum_i gC_i z_t ds_i
      return mtile<RB>(zero4, lane, [&](int m, int k) {
                         const float4 z4 = f4(&sm.Z[m][k]);
                         const float4 g4 = f4(&sm.gC[k]);
                         return make_float4(g4.x * z4.x, g4.y * z4.y, g4.z * z4.z, g4.w * z4.w);
                       },
                       [&](int k, int n) { return col4(sm.dS, k, 16 * kb + n); });
    };
    // -sum_i w_t s0_i + sum_s (dG_ts + dG_st) x_s + sum_t' dP_t't q_t'
    auto dx_rest = [&](int kb, floatx4 acc) __attribute__((always_inline)) {
      acc = mtile<RB>(acc, lane, [&](int m, int k) {
                        const float4 w4 = f4(&sm.W[m][k]);
                        return make_float4(-w4.x, -w4.y, -w4.z, -w4.w);
                      },
                      [&](int k, int n) { return col4(sm.S, k, 16 * kb + n); });
      acc = mtile<BC>(acc, lane, [&](int m, int k) {
                        return make_float4(sm.dG[m][k] + sm.dG[k][m], sm.dG[m][k + 1] + sm.dG[k + 1][m],
                                           sm.dG[m][k + 2] + sm.dG[k + 2][m], sm.dG[m][k + 3] + sm.dG[k + 3][m]);
                      },
                      [&](int k, int n) { return col4(XU, k, 16 * kb + n); });
      return mtile<BC>(acc, lane, [&](int m, int k) { return col4(sm.dP, k, m); },
                       [&](int k, int n) { return col4(sm.Q, k, 16 * kb + n); });
    };
    if constexpr (2 * NKB <= BNW) {
      // waves 0..NKB-1: dq and the gC z ds part of dx (to LDS); waves NKB..2NKB-1:
      // the rest of dx, completed after the barrier
      floatx4 dxr = zero4;
      const bool dxw = wave >= NKB && wave < 2 * NKB;
      if (wave < NKB) {
        dq_tile(wave);
        const floatx4 acc = dx_gz(wave);
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.dxp[rq + r][16 * wave + mn] = acc[r];
      } else if (dxw) {
        dxr = dx_rest(wave - NKB, zero4);
      }
      lds_barrier();
      if (dxw) {
        const int kb = wave - NKB;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = rq + r, kk = 16 * kb + mn;
          dx_out(t, kk, dxr[r] + sm.dxp[t][kk] + 2.0f * sm.dn[t / BW] * XU[t][kk]);
        }
      }
    } else {
      // every wave takes whole column tiles (dk = 128)
      for (int kb = wave; kb < NKB; kb += BNW) {
        dq_tile(kb);
        const floatx4 acc = dx_rest(kb, dx_gz(kb));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = rq + r, kk = 16 * kb + mn;
          dx_out(t, kk, acc[r] + 2.0f * sm.dn[t / BW] * XU[t][kk]);
        }
      }
      lds_barrier();
    }
    // ---- dS <- gC dS + sum_t g_t do_t q_t - sum_t w_t x_t: tiles (ib, kb); every
    // reader of dS finished before the barrier above ----
    constexpr bool SPLITX = 2 * NKB <= BNW;   // waves NKB..2NKB-1 finish dx above
    const int widx = (SPLITX && wave >= 2 * NKB) ? wave - NKB : wave;
    const int nwk = SPLITX ? BNW - NKB : BNW;
    for (int tt = (SPLITX && wave >= NKB && wave < 2 * NKB) ? NIB * NKB : widx; tt < NIB * NKB; tt += nwk) {
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
                      [&](int k, int n) { return col4(XU, k, 16 * kb + n); });
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.dS[16 * ib + rq + r][16 * kb + mn] = acc[r];
    }
    lds_barrier();
    if constexpr (BW > 1) {
      // d x and d y per sample: the sum over the unknowns that hold it (slot w of
      // step k - (BW-1) + w for tile row k).  The tile's first BW-1 rows are samples
      // of earlier chunks: their sums go to the previous chunk, which adds them to
      // its rows NS .. NS+BW-2 (double-buffered by chunk parity); when BW-1 > NS some
      // of those rows are again before that chunk and travel on.  Nothing here is
      // touched by the next chunk's commit.
      const int cur = ci & 1, nxt = (ci + 1) & 1;
      for (int idx = tid; idx < NK * DK; idx += BNT) {
        const int k = idx / DK, kk = idx % DK;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < BW; ++w) {
          const int st = k - (BW - 1) + w;
          if (st >= 0 && st < NS) v += sm.dxp[BW * st + w][kk];
        }
        if (k >= NS) v += sm.dxh[nxt][k - NS][kk];   // carried from the chunk after
        if (k < BW - 1) {
          sm.dxh[cur][k][kk] = v;                    // on to the chunk before
        } else {
          const long j = t0 - (BW - 1) + k;     // sample; x_j = k_{j - ks}
          if (j < L) {
            if (j - ks >= 0) {
              if (ks == 0 && j == L - 1 && dkl) v += dkl[chain * DK + kk];
              ok[qk_base + (j - ks) * DK + kk] = v;
            } else if (okp) {
              okp[chain * DK + kk] = v;
            }
          }
        }
      }
      for (int idx = tid; idx < NK * RB; idx += BNT) {
        const int k = idx / RB, i = idx % RB;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < BW; ++w) {
          const int st = k - (BW - 1) + w;
          if (st >= 0 && st < NS) v += sm.DR[BW * st + w][i];
        }
        if (k >= NS) v += sm.dyh[nxt][k - NS][i];
        if (k < BW - 1) {
          sm.dyh[cur][k][i] = v;
        } else {
          const long j = t0 - (BW - 1) + k;
          if (j < L) a.dv[v_base + j * dvf + i0 + i] = v;
        }
      }
    }
  }
  if (a.dS0) {
    for (int idx = tid; idx < RB * DK; idx += BNT)
      a.dS0[(chain * dvf + i0 + idx / DK) * DK + idx % DK] = sm.dS[idx / DK][idx % DK];
  }
  // A chunk whose decay products left the range of the chunk algebra: the
  // chain's gradients are not computed; every output this workgroup writes for
  // the chain (its value rows, and the chain's dq, dk, dk_prev and per-token
  // dbeta, or its slice's partial sums of them, which the sum kernel adds) is
  // set to NaN instead.
  __syncthreads();
  if (sm.bad) {
    const float nan = __builtin_nanf("");
    for (long e = tid; e < L * RB; e += BNT) {
      a.dv[v_base + (e / RB) * dvf + i0 + e % RB] = nan;
      if (a.dbeta_t && a.beta_kind == 2) a.dbeta_t[v_base + (e / RB) * dvf + i0 + e % RB] = nan;
    }
    for (long e = tid; e < L * DK; e += BNT) {
      oq[qk_base + e] = nan;
      // k_{L-1} only leaves the call as k_last (previous-key pairing): its
      // gradient is dk_last, written above, whatever the chain
      if (!(ks == 1 && e / DK == L - 1)) ok[qk_base + e] = nan;
    }
    if (okp)
      for (int e = tid; e < DK; e += BNT) okp[chain * DK + e] = nan;
    if (odb && a.beta_kind == 1)
      for (long e = tid; e < L; e += BNT) odb[chain * L + e] = nan;
    if (a.dS0)
      for (int idx = tid; idx < RB * DK; idx += BNT) a.dS0[(chain * dvf + i0 + idx / DK) * DK + idx % DK] = nan;
  }
}

// Sum of the slices' partial dq, dk, dk_prev and per-token dbeta, in slice order
// (deterministic); dk_last enters here: k_{L-1} is k_last itself with the previous
// pairing, an input key of the last sample with the same-step pairing.
__global__ __launch_bounds__(256) void backward_sum_kernel(BwdArgs a, int nrg, const float* part) {
  const long BH = (long)a.batch * a.heads, L = a.seqlen;
  const int DK = a.ndk;
  const long nq = BH * L * DK;
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  const long nkp = a.dk_prev ? BH * DK : 0;
  const long nb = (a.dbeta_t && a.beta_kind == 1) ? BH * L : 0;
  if (e < nq) {
    float q = 0.0f, k = 0.0f;
    for (int r = 0; r < nrg; ++r) {
      q += part[r * nq + e];
      k += part[(nrg + r) * nq + e];
    }
    const long chain = e / (L * DK), t = (e / DK) % L, kk = e % DK;
    if (t == L - 1) {
      const float dl = a.dk_last ? a.dk_last[chain * DK + kk] : 0.0f;
      k = a.key_shift ? dl : k + dl;
    }
    a.dq[e] = q;
    a.dk[e] = k;
  } else if (e < nq + nkp) {
    const long f = e - nq;
    float v = 0.0f;
    for (int r = 0; r < nrg; ++r) v += part[2 * nrg * nq + r * (BH * DK) + f];
    a.dk_prev[f] = v;
  } else if (e < nq + nkp + nb) {
    const long f = e - nq - nkp;
    float v = 0.0f;
    for (int r = 0; r < nrg; ++r) v += part[2 * nrg * nq + nrg * (BH * DK) + r * (BH * L) + f];
    a.dbeta_t[f] = v;
  }
}

// value rows per workgroup (a head's rows are split over dv / RB workgroups):
// 32, so that every per-row sweep is one pass of the 32 sixteen-lane rows of the
// eight waves (64 rows take two passes of latency-bound DPP chains, 16 leave half
// the waves idle and double the partial sums); fewer when dv is smaller
__host__ __device__ constexpr int bwd_rows(int dk, int dv) { return (void)dk, dv < 32 ? dv : 32; }

template <typename T, int DK, int RB>
hipError_t launch_bwd_rb(const BwdArgs& a, hipStream_t stream) {
  const int nrg = a.ndv / RB;
  const dim3 grid((unsigned)((long)a.batch * a.heads * nrg));
  if (a.window == 1) hipLaunchKernelGGL((backward_kernel<T, DK, RB, 1>), grid, dim3(BNT), 0, stream, a);
  else if (a.window == 2) hipLaunchKernelGGL((backward_kernel<T, DK, RB, 2>), grid, dim3(BNT), 0, stream, a);
  else if (a.window == 3) hipLaunchKernelGGL((backward_kernel<T, DK, RB, 3>), grid, dim3(BNT), 0, stream, a);
  else if (a.window == 4) hipLaunchKernelGGL((backward_kernel<T, DK, RB, 4>), grid, dim3(BNT), 0, stream, a);
  else if (a.window == 5) hipLaunchKernelGGL((backward_kernel<T, DK, RB, 5>), grid, dim3(BNT), 0, stream, a);
  else if (a.window == 6) hipLaunchKernelGGL((backward_kernel<T, DK, RB, 6>), grid, dim3(BNT), 0, stream, a);
  else if (a.window == 7) hipLaunchKernelGGL((backward_kernel<T, DK, RB, 7>), grid, dim3(BNT), 0, stream, a);
  else if (a.window == 8) hipLaunchKernelGGL((backward_kernel<T, DK, RB, 8>), grid, dim3(BNT), 0, stream, a);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nrg == 1) return e;
  const long BH = (long)a.batch * a.heads;
  const long ns = BC / a.window, nch = (a.seqlen + ns - 1) / ns;
  const float* part = a.workspace + BH * nrg * nch * ((long)RB * DK + (long)BC * RB + (long)BC * BC);
  const long n = BH * a.seqlen * DK + (a.dk_prev ? BH * DK : 0) + ((a.dbeta_t && a.beta_kind == 1) ? BH * a.seqlen : 0);
  hipLaunchKernelGGL(backward_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a, nrg, part);
  return hipGetLastError();
}

template <typename T, int DK>
hipError_t launch_bwd_dk2(const BwdArgs& a, hipStream_t stream) {
  switch (bwd_rows(DK, a.ndv)) {
    case 16: return launch_bwd_rb<T, DK, 16>(a, stream);
    case 32: return launch_bwd_rb<T, DK, 32>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_bwd_dk(const BwdArgs& a, hipStream_t stream) {
  switch (a.ndk) {
    case 16: return launch_bwd_dk2<T, 16>(a, stream);
    case 32: return launch_bwd_dk2<T, 32>(a, stream);
    case 64: return launch_bwd_dk2<T, 64>(a, stream);
    case 128: return launch_bwd_dk2<T, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t backward_workspace_bytes(int batch, int heads, long seqlen, int dk, int dv, int window) {
  // per slice of value rows (bwd_rows) and chunk of floor(16 / window) steps: start state,
  // S0 x, Gram (fp32); with several slices per chain also their partial dq, dk,
  // dk_prev and per-token dbeta (the larger of what any call may need)
  const long ns = BC / window;
  const long nch = (seqlen + ns - 1) / ns;
  const long RB = bwd_rows(dk, dv), nrg = dv / RB, BH = (long)batch * heads;
  const long records = BH * nrg * nch * (RB * dk + (long)BC * RB + (long)BC * BC);
  const long partials = nrg > 1 ? nrg * BH * (2 * seqlen * dk + dk + seqlen) : 0;
  return (size_t)(records + partials) * sizeof(float);
}

size_t backward_chain_bytes(long seqlen, int dk, int dv, int window, int dtype) {
  // the kernel reads a chain's q, k, v, gains, dO and workspace record through
  // 32-bit buffer ranges; the largest of them
  const long es = dtype == 0 ? 2 : 4;
  const long ns = BC / window, nch = (seqlen + ns - 1) / ns, RB = bwd_rows(dk, dv);
  long m = seqlen * dk * es;
  m = m > seqlen * dv * 4 ? m : seqlen * dv * 4;
  const long rec = nch * (RB * dk + (long)BC * RB + (long)BC * BC) * 4;
  return (size_t)(m > rec ? m : rec);
}

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
  (void)hipGetLastError();
  if (a.dtype == 0) return launch_bwd_dk<uint16_t>(a, stream);
  return launch_bwd_dk<float>(a, stream);
}

}  // namespace falcon
