// falcon_chunk_w1.hip - chunk-parallel Falcon forward for window 1 (Falcon-1,
// -2, -1A, -2A), software-pipelined across chunks on gfx950.
//
// Method and algebra: explainer of arXiv 2608.27763, section 核心方法 §3
// (chunk-parallel form) and the 163.com article, section 02 (2) (only the
// fixed-size state passes between chunks; Gram / WY representation with a
// batched triangular solve).  With window 1 the unknowns of a chunk are the
// residuals e_t = y_t - S_{t-1} x_t, t = 0..C-1, and (per value row)
//   g_t = prod_{r<=t} a_r, zeta_t = eta_t / g_t, z_t = zeta_t e_t,
//   e_t + g_{t-1} sum_{s<t} (x_t . x_s) z_s = y_t - g_{t-1} S0 x_t   (regression)
//   z_t = zeta_t y_t                                                  (inner product)
//   o_t = g_t (S0 q_t + sum_{s<=t} (q_t . x_s) z_s)
//   S_C = g_{C-1} (S0 + sum_s z_s x_s^T)
//
// Why a separate kernel: everything that does not depend on the incoming
// state S0 (Gram, q.x, decay products, the triangular factors) can be computed
// one chunk ahead.  Each iteration c therefore runs, between three workgroup
// barriers, the state-dependent chain of chunk c next to the state-independent
// preparation of chunk c+1, so the serial pieces (the solve on two waves, the
// diagonal-block inverses on one wave) overlap with matrix-core work of the
// other waves instead of idling them:
//   phase 1  commit chunk c+1's prefetched q/k/v/beta to LDS (second buffer)
//            and issue chunk c+2's global loads; keys of chunk c transposed;
//            S0 x_t and S0 q_t (kept in registers for the readout);
//            off-diagonal solve blocks M_bj of chunk c; per-row scalars (Falcon-2)
//   phase 2  solve of chunk c (shared eta: one wave per 16-row block, next to
//            Gram, q.x and scalars of chunk c+1; per-channel eta: one value row
//            per 16-lane row on every wave)
//   phase 3  readout and state carry of chunk c  ||  diagonal-block inverses
//            of chunk c+1 (shared eta) or its Gram and q.x (per-channel eta)
// One workgroup = 8 wave64 = one (batch*head) chain x 32 value rows.
#include "falcon_device.h"
#include "falcon_exact.h"
#include "falcon_launch.h"
#include "falcon_mma.h"

namespace falcon {
namespace {

// v of lane - N within the same 16-lane row (DPP row_shr); lanes whose source
// lies outside the row return `fill`
template <int N>
__device__ __forceinline__ float row_shr(float v, float fill) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill), __builtin_bit_cast(int, v),
                                                             0x110 + N, 0xF, 0xF, false));
}

// g times the g of lane - N within the same 16-lane row; lanes whose source lies
// outside the row are disabled by the DPP bounds rule and keep g (the nop gives
// the two wait states a DPP read needs after a VALU write)
template <int N>
__device__ __forceinline__ float row_shr_mul(float g) {
  asm("s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shr:%1 row_mask:0xf bank_mask:0xf" : "+v"(g) : "i"(N));
  return g;
}

// acc + g * (v of lane N of the same 16-lane row); the nop gives the two wait
// states a DPP read needs after a VALU write of v
template <int N>
__device__ __forceinline__ float fmac_bcast(float acc, float v, float g) {
  asm("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(acc) : "v"(v), "v"(g), "i"(N));
  return acc;
}

// Per-channel forward substitution, step M onwards, for the row held by one
// 16-lane row: lane l owns the unknowns u = l + 16 j, with partial sums
// acc[j] = sum_{m<M} Gs[u][m] z_m and g[j][m] = Gs[u][m] (zero for m >= u).
// z_M is formed on every lane and taken from lane M mod 16, its owner.
template <int NS, int M>
__device__ __forceinline__ void row_sweep(float (&acc)[NS], const float (&g)[NS][16 * NS], const float (&rp)[NS],
                                          const float (&gm)[NS], const float (&ze)[NS]) {
  constexpr int J = M / 16;
  const float z = ze[J] * __builtin_fmaf(-gm[J], acc[J], rp[J]);
#pragma unroll
  for (int j = J; j < NS; ++j) acc[j] = fmac_bcast<M % 16>(acc[j], z, g[j][M]);
  if constexpr (M + 1 < 16 * NS) row_sweep<NS, M + 1>(acc, g, rp, gm, ze);
}

constexpr int RB = 16;
constexpr int NRB = 2;
constexpr int RW = RB * NRB;
constexpr int NW = 8;
constexpr int NT = 64 * NW;

template <int DK, int CS, bool REG, bool PERROW>
struct W1Lds {
  static constexpr int NB = CS / 16;
  static constexpr int SCB = PERROW ? 1 : 2;   // scalar buffers (shared eta: double)
  static constexpr int SR = PERROW ? RW : 1;   // scalar rows
  struct Split {
    uint16_t hi[RW][CS + 8];
    uint16_t lo[RW][CS + 8];
  };
  union Slot {               // keys of a chunk; once consumed, that chunk's z
    uint16_t X[CS][DK + 8];
    Split ZT;
  };
  Slot slot[2];
  uint16_t Q[2][CS][DK + 8];
  uint16_t XT[DK][CS + 8];           // keys of the current chunk, transposed
  uint16_t YT[2][RW][CS + 8];        // values (bf16 bits), transposed
  uint16_t BT[PERROW ? 2 : 1][PERROW ? RW : 1][CS];   // per-channel beta (bf16 bits)
  float beta[2][CS];                 // shared beta (fp32)
  float nrm[2][CS];
  float S[RW][DK + 4];
  uint16_t Shi[RW][DK + 8];
  uint16_t Slo[RW][DK + 8];
  float XS[REG ? RW : 1][CS + 4];    // S0 x_t
  float GT[REG ? CS : 1][CS + 4];    // shared eta: Gram transposed; per-channel: Gram
  uint16_t Phi[2][CS][CS + 8];       // masked q.x, split
  uint16_t Plo[2][CS][CS + 8];
  uint16_t SAhi[(REG && !PERROW) ? NB : 1][16][CS + 8];   // [T_bb | -M_b0 | ...]
  uint16_t SAlo[(REG && !PERROW) ? NB : 1][16][CS + 8];
  alignas(16) float gam[SCB][SR][CS];
  alignas(16) float gm1[SCB][SR][CS];
  alignas(16) float zeta[SCB][SR][CS];
  int bad;                           // some chunk's decay products left the range
};

struct W1Geom {
  int nrbg;
  int remap;
  int nchunks;
};

template <int DK, int CS, bool REG, bool PERROW>
__global__ __launch_bounds__(NT) void chunk_w1_kernel(SeqArgs a, W1Geom geo) {
  using SM = W1Lds<DK, CS, REG, PERROW>;
  constexpr int NB = CS / 16, NTT = CS / 16, NKT = DK / 16, VPR = DK / 8;
  constexpr int KV = (CS * VPR + NT - 1) / NT;
  constexpr int YV = (CS * (RW / 8) + NT - 1) / NT;
  __shared__ __align__(16) SM sm;

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(a.v);
  const uint16_t* __restrict__ kpg = static_cast<const uint16_t*>(a.k_prev);
  const uint16_t* __restrict__ bg = static_cast<const uint16_t*>(a.beta_t);

  int chain, rbg;
  {
    const int b = blockIdx.x;
    if (geo.remap) {   // the row-block groups of one chain share an XCD (and its L2)
      const int xcd = b & 7, slot = b >> 3;
      chain = xcd + 8 * (slot / geo.nrbg);
      rbg = slot % geo.nrbg;
    } else {
      chain = b / geo.nrbg;
      rbg = b % geo.nrbg;
    }
  }
  const int dv = a.dv;
  const int i0 = rbg * RW;
  const int nrb = (dv - i0) >= RW ? NRB : 1;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const long L = a.seqlen;
  const long qk_base = (long)chain * L * DK;
  const long v_base = (long)chain * L * dv;
  const int nchunks = geo.nchunks;

  // ---------------- prefetch registers (one chunk ahead of the commit) ----------------
  // Loads land in registers that nothing reads before the next commit, so the
  // compiler issues them without waiting (no widening or merging after a load).
  uint4 pk[KV], pq[KV], py[YV];
  uint4 pbc[PERROW ? YV : 1];     // per-channel beta, same tiling as v
  uint32_t pbt = 0;               // per-token beta of step tid (tid < CS)
  auto prefetch = [&](int cidx) __attribute__((always_inline)) {
    const long t0 = (long)cidx * CS;
    const int c = (int)((L - t0) < CS ? (L - t0) : CS);
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int idx = tid + v * NT;
      const int t = idx / VPR, kv = idx % VPR;
      uint4 kval = {0u, 0u, 0u, 0u}, qval = {0u, 0u, 0u, 0u};
      if (idx < CS * VPR && t < c) {
        const long g = t0 + t;   // key x_g = k_{g-s}; with s = 1, x_0 = k_prev or 0
        if (g >= a.key_shift) kval = *reinterpret_cast<const uint4*>(kg + qk_base + (g - a.key_shift) * DK + kv * 8);
        else if (kpg) kval = *reinterpret_cast<const uint4*>(kpg + (long)chain * DK + kv * 8);
        qval = *reinterpret_cast<const uint4*>(qg + qk_base + g * DK + kv * 8);
      }
      pk[v] = kval;
      pq[v] = qval;
    }
#pragma unroll
    for (int v = 0; v < YV; ++v) {
      const int idx = tid + v * NT;
      const int t = idx / (RW / 8), h = idx % (RW / 8);
      uint4 val = {0u, 0u, 0u, 0u};
      if (idx < CS * (RW / 8) && t < c && i0 + h * 8 < dv)
        val = *reinterpret_cast<const uint4*>(vg + v_base + (t0 + t) * dv + i0 + h * 8);
      py[v] = val;
    }
    if (PERROW) {
#pragma unroll
      for (int v = 0; v < YV; ++v) {
        const int idx = tid + v * NT;
        const int t = idx / (RW / 8), h = idx % (RW / 8);
        uint4 val = {0u, 0u, 0u, 0u};
        if (idx < CS * (RW / 8) && t < c && i0 + h * 8 < dv)
          val = *reinterpret_cast<const uint4*>(bg + ((long)chain * L + t0 + t) * dv + i0 + h * 8);
        pbc[v] = val;
      }
    } else {
      pbt = 0;
      if (a.beta_kind == 1 && tid < c) pbt = (uint32_t)bg[(long)chain * L + t0 + tid];
    }
  };
  auto commit = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int idx = tid + v * NT;
      const uint4 val = pk[v];
      const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
      float part = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_to_f32((uint16_t)(w4[e] & 0xFFFFu));
        const float hi = bf16_to_f32((uint16_t)(w4[e] >> 16));
        part += lo * lo + hi * hi;
      }
      part = group_sum<VPR>(part);
      if (idx < CS * VPR) {
        const int t = idx / VPR, kv = idx % VPR;
        *reinterpret_cast<uint4*>(&sm.slot[s].X[t][kv * 8]) = val;
        *reinterpret_cast<uint4*>(&sm.Q[s][t][kv * 8]) = pq[v];
        if (kv == 0) sm.nrm[s][t] = part;
      }
    }
#pragma unroll
    for (int v = 0; v < YV; ++v) {
      const int idx = tid + v * NT;
      if (idx < CS * (RW / 8)) {
        const int t = idx / (RW / 8), h = idx % (RW / 8);
        const uint4 val = py[v];
        const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sm.YT[s][h * 8 + 2 * e][t] = (uint16_t)(w4[e] & 0xFFFFu);
          sm.YT[s][h * 8 + 2 * e + 1][t] = (uint16_t)(w4[e] >> 16);
        }
      }
    }
    if (PERROW) {
#pragma unroll
      for (int v = 0; v < YV; ++v) {
        const int idx = tid + v * NT;
        if (idx < CS * (RW / 8)) {
          const int t = idx / (RW / 8), h = idx % (RW / 8);
          const uint4 val = pbc[v];
          const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sm.BT[s][h * 8 + 2 * e][t] = (uint16_t)(w4[e] & 0xFFFFu);
            sm.BT[s][h * 8 + 2 * e + 1][t] = (uint16_t)(w4[e] >> 16);
          }
        }
      }
    } else if (tid < CS) {
      sm.beta[s][tid] = a.beta_kind == 0 ? a.beta : bf16_to_f32((uint16_t)pbt);
    }
  };

  // eta_t = beta_t / (eps + ||x_t||^2), a_t = 1 - eta_t lambda; padded steps and
  // the fresh-sequence first step (x_1 = 0 on S_0 = 0) take eta = 0, a = 1.
  // One wave per row of scalars; lane = step; prefix product by a wave scan.
  auto scalars = [&](int s, int cidx, int dst, int row, int wv) __attribute__((always_inline)) {
    (void)wv;
    const long t0 = (long)cidx * CS;
    const int c = (int)((L - t0) < CS ? (L - t0) : CS);
    const int t = lane;
    const bool live = t < c && !(t0 + t == 0 && kpg == nullptr && a.key_shift);
    float eta = 0.0f, dec = 1.0f;
    if (live) {
      const float bv = PERROW ? bf16_to_f32(sm.BT[s][row][t]) : sm.beta[s][t];
      eta = bv / (a.eps + sm.nrm[s][t]);
      dec = 1.0f - eta * a.lambda;
    }
    float gsc = dec;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float o = __shfl_up(gsc, d, 64);
      if (lane >= d) gsc *= o;
    }
    float gprev = __shfl_up(gsc, 1, 64);
    if (lane == 0) gprev = 1.0f;
    if (__builtin_amdgcn_ballot_w64(t < CS && gauge_out_of_range(gsc, dec)) != 0 && lane == 0) sm.bad = 1;
    if (t < CS) {
      sm.gam[dst][row][t] = gsc;
      sm.gm1[dst][row][t] = gprev;
      sm.zeta[dst][row][t] = eta / gsc;
    }
  };

  // Per-channel scalars of NC groups of 64/CS rows, group k = rows r0 + k rstep
  // + lane / CS (lane = row slot x CS + step): prefix products by DPP row shifts
  // (16-lane rows), the upper half of a 32-step row times the lower half's total.
  // All loads first, then the scans, then the stores: LDS stores in between
  // would keep the compiler from issuing the later loads early.
  auto scalars_rows = [&](auto nc_tag, int s, int cidx, int dst, int r0, int rstep) __attribute__((always_inline)) {
    static_assert(!PERROW || CS == 16 || CS == 32, "per-channel sub-chunks of 16 or 32 steps");
    constexpr int NC = decltype(nc_tag)::value;
    const long t0 = (long)cidx * CS;
    const int c = (int)((L - t0) < CS ? (L - t0) : CS);
    const int t = lane % CS, rl = lane / CS;
    const bool live = t < c && !(t0 + t == 0 && kpg == nullptr && a.key_shift);
    const float rn = __builtin_amdgcn_rcpf(a.eps + sm.nrm[s][t]);
    float eta[NC], g[NC], dec[NC];
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const float bv = bf16_to_f32(sm.BT[s][r0 + k * rstep + rl][t]);
      eta[k] = live ? bv * rn : 0.0f;
      g[k] = __builtin_fmaf(-eta[k], a.lambda, 1.0f);
      dec[k] = g[k];
    }
#pragma unroll
    for (int k = 0; k < NC; ++k) g[k] = row_shr_mul<1>(g[k]);
#pragma unroll
    for (int k = 0; k < NC; ++k) g[k] = row_shr_mul<2>(g[k]);
#pragma unroll
    for (int k = 0; k < NC; ++k) g[k] = row_shr_mul<4>(g[k]);
#pragma unroll
    for (int k = 0; k < NC; ++k) g[k] = row_shr_mul<8>(g[k]);
    bool out_of_range = false;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      float fill = 1.0f;
      if constexpr (CS == 32) {
        const float tA = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g[k]), 15));
        const float tB = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g[k]), 47));
        const float tot = lane < 32 ? tA : tB;
        if ((lane & 31) >= 16) g[k] *= tot;
        fill = (lane & 31) == 16 ? tot : 1.0f;
      }
      const float gprev = row_shr<1>(g[k], fill);
      out_of_range |= gauge_out_of_range(g[k], dec[k]);
      const int row = r0 + k * rstep + rl;
      sm.gam[dst][row][t] = g[k];
      sm.gm1[dst][row][t] = gprev;
      sm.zeta[dst][row][t] = eta[k] * __builtin_amdgcn_rcpf(g[k]);
    }
    if (__builtin_amdgcn_ballot_w64(out_of_range) != 0 && lane == 0) sm.bad = 1;
  };

  // Per-channel residual solve of the chunk in slot s: value row 4 wave + lg on
  // the 16-lane row lg, right-hand sides r_u = y_u - g_{u-1} (S0 x_u), and the
  // per-channel Gram (strictly lower, zero at and above the diagonal) held per
  // lane; once the sweep has passed step u the partial sum of u no longer
  // changes, so each lane forms its own z_u from it at the end.
  auto row_solve = [&](int s, typename SM::Split* zt) __attribute__((always_inline)) {
    constexpr int NS = CS / 16;
    const int i = 4 * wave + lg;
    float g[NS][CS], rp[NS], gm[NS], ze[NS], acc[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
#pragma unroll
      for (int m = 0; m < 16 * (j + 1); m += 4) {
        const float4 gv = *reinterpret_cast<const float4*>(&sm.GT[lr + 16 * j][m]);
        g[j][m] = gv.x; g[j][m + 1] = gv.y; g[j][m + 2] = gv.z; g[j][m + 3] = gv.w;
      }
      const int u = lr + 16 * j;
      gm[j] = sm.gm1[0][i][u];
      ze[j] = sm.zeta[0][i][u];
      rp[j] = bf16_to_f32(sm.YT[s][i][u]) - gm[j] * sm.XS[i][u];
      acc[j] = 0.0f;
    }
    row_sweep<NS, 0>(acc, g, rp, gm, ze);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const float z = ze[j] * __builtin_fmaf(-gm[j], acc[j], rp[j]);
      split1(z, zt->hi[i][lr + 16 * j], zt->lo[i][lr + 16 * j]);
    }
  };

  // Gram (regression) and q.x tiles of slot s: lower triangle of 16x16 tiles.
  constexpr int NLT = NTT * (NTT + 1) / 2;
  auto gram_tile = [&](int s, int tt) __attribute__((always_inline)) {
    int ti = 0;
    while ((ti + 1) * (ti + 2) / 2 <= tt) ++ti;
    const int tj = tt - ti * (ti + 1) / 2;
    // output rows = the index that is contiguous in GT, so a lane stores a float4:
    // shared eta keeps Gs^T[u'][u] (rows u = tile ti), per-channel Gs[u][u'] (rows u' = tj)
    const int ra = PERROW ? tj : ti, rb2 = PERROW ? ti : tj;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mma_nt<true, true>(acc, DK,
        [&](int r, int k) { return hl_bf16(&sm.slot[s].X[16 * ra + r][k]); },
        [&](int r, int k) { return hl_bf16(&sm.slot[s].X[16 * rb2 + r][k]); });
    const int col = 16 * rb2 + lr;           // the other index
    float gv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * ra + 4 * lg + e;
      const int u = PERROW ? col : row, u2 = PERROW ? row : col;   // Gs[u][u'], u' < u
      gv[e] = (u2 < u) ? acc[e] : 0.0f;
    }
    *reinterpret_cast<float4*>(&sm.GT[col][16 * ra + 4 * lg]) = make_float4(gv[0], gv[1], gv[2], gv[3]);
  };
  auto qx_tile = [&](int s, int tt) __attribute__((always_inline)) {
    int ti = 0;
    while ((ti + 1) * (ti + 2) / 2 <= tt) ++ti;
    const int tj = tt - ti * (ti + 1) / 2;     // step tile ti, key tile tj <= ti
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mma_nt<true, true>(acc, DK,
        [&](int r, int k) { return hl_bf16(&sm.slot[s].X[16 * tj + r][k]); },
        [&](int r, int k) { return hl_bf16(&sm.Q[s][16 * ti + r][k]); });
    const int t = 16 * ti + lr;
    float pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int u = 16 * tj + 4 * lg + e;
      pv[e] = (u <= t) ? acc[e] : 0.0f;
    }
    store_split4(&sm.Phi[s][t][16 * tj + 4 * lg], &sm.Plo[s][t][16 * tj + 4 * lg], pv);
  };
  // 16x16 diagonal-block inverses T_bb = Gamma_- (I + Gs D)^-1 Gamma_-^{-1},
  // D = diag(zeta_m g_{m-1}); one wave, lane = 16 b + column.
  auto diag_inverse = [&](int sc) __attribute__((always_inline)) {
    const int bb = (lane >> 4) < NB ? (lane >> 4) : 0;
    const int cc = lane & 15;
    const int u0 = 16 * bb;
    float gmv[16], dm[16], acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      gmv[r] = sm.gm1[sc][0][u0 + r];
      dm[r] = sm.zeta[sc][0][u0 + r] * gmv[r];
      acc[r] = (r == cc) ? 1.0f : 0.0f;
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const float sv = dm[m] * acc[m];
      const float* grow = &sm.GT[u0 + m][u0];   // Gs^T[u_m][u_r] = Gs[r][m]
#pragma unroll
      for (int r = m + 1; r < 16; ++r) acc[r] -= grow[r] * sv;
    }
    if ((lane >> 4) < NB) {
      const float inv_c = 1.0f / sm.gm1[sc][0][u0 + cc];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        split1(gmv[r] * acc[r] * inv_c, sm.SAhi[bb][r][cc], sm.SAlo[bb][r][cc]);
    }
  };

  // ---------------- prologue: state, chunk 0 ----------------
  if (tid == 0) sm.bad = 0;
  for (int idx = tid; idx < RW * DK; idx += NT) {
    const int i = idx / DK, kk = idx % DK;
    float sv = 0.0f;
    if (a.S0 && i0 + i < dv) sv = a.S0[((long)chain * dv + i0 + i) * DK + kk];
    sm.S[i][kk] = sv;
    split1(sv, sm.Shi[i][kk], sm.Slo[i][kk]);
  }
  prefetch(0);
  commit(0);
  if (nchunks > 1) prefetch(1);
  __syncthreads();
  for (int task = wave; task < (REG ? 2 : 1) * NLT; task += NW) {
    if (task < NLT) qx_tile(0, task);
    else gram_tile(0, task - NLT);
  }
  if (!PERROW && wave == NW - 1) scalars(0, 0, 0, 0, wave);
  __syncthreads();
  if (REG && !PERROW && wave == NW - 1) diag_inverse(0);
  __syncthreads();

  // The readout of chunk c is stored during phase 1 of chunk c+1, after that
  // phase's commit and prefetch: global stores share the in-order
  // vector-memory counter with the loads, so a store issued shortly before a
  // commit would make the commit wait for the store's completion.
  float4 opend = make_float4(0.f, 0.f, 0.f, 0.f);
  float* optr = nullptr;
  for (int ci = 0; ci < nchunks; ++ci) {
    const int cur = ci & 1, nxt = cur ^ 1;
    const bool has_next = ci + 1 < nchunks;
    const long t0 = (long)ci * CS;
    const int cval = (int)((L - t0) < CS ? (L - t0) : CS);
    const int sc = PERROW ? 0 : cur;          // scalar buffer of chunk ci

    // ================= phase 1 =================
    if (has_next) commit(nxt);
    if (has_next && ci + 2 < nchunks) prefetch(ci + 2);
    if (optr) *reinterpret_cast<float4*>(optr) = opend;
    optr = nullptr;
    // keys of chunk ci transposed (carry operand)
    // (8 keys x 4 columns per thread: 8-byte reads, 16-byte writes)
    for (int idx = tid; idx < (DK / 4) * (CS / 8); idx += NT) {
      const int c4 = idx % (DK / 4), j8 = idx / (DK / 4);
      uint2 rw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) rw[e] = *reinterpret_cast<const uint2*>(&sm.slot[cur].X[8 * j8 + e][4 * c4]);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t a0 = (cc < 2) ? rw[2 * e].x : rw[2 * e].y;
          const uint32_t a1 = (cc < 2) ? rw[2 * e + 1].x : rw[2 * e + 1].y;
          w[e] = (cc & 1) ? ((a0 >> 16) | (a1 & 0xFFFF0000u)) : ((a0 & 0xFFFFu) | (a1 << 16));
        }
        *reinterpret_cast<uint4*>(&sm.XT[4 * c4 + cc][8 * j8]) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    // S0 q_t tiles stay in the registers of the wave that reads them out in phase 3
    constexpr int NQ = NRB * NTT;
    floatx4 qacc = {0.f, 0.f, 0.f, 0.f};
    if (wave < NQ) {
      const int rbk = wave / NTT, tt = wave % NTT;
      if (rbk < nrb)
        qacc = mma_nt<false, true>(qacc, DK,
            [&](int r, int k) { return hl_pair(&sm.Shi[16 * rbk + r][k], &sm.Slo[16 * rbk + r][k]); },
            [&](int r, int k) { return hl_bf16(&sm.Q[cur][16 * tt + r][k]); });
    }
    {
      constexpr int NXS = REG ? NRB * NTT : 0;
      constexpr int NM = (REG && !PERROW) ? NB * (NB - 1) / 2 : 0;
      for (int task = (wave + NQ) % NW; task < NXS + NM; task += NW) {
        if (task < NXS) {
          const int rbk = task / NTT, tj = task % NTT;
          if (rbk >= nrb) continue;
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          acc = mma_nt<true, false>(acc, DK,
              [&](int r, int k) { return hl_bf16(&sm.slot[cur].X[16 * tj + r][k]); },
              [&](int r, int k) { return hl_pair(&sm.Shi[16 * rbk + r][k], &sm.Slo[16 * rbk + r][k]); });
          *reinterpret_cast<float4*>(&sm.XS[16 * rbk + lr][16 * tj + 4 * lg]) =
              make_float4(acc[0], acc[1], acc[2], acc[3]);
        } else {
          // M_bj = T_bb diag(g_{t-1})_b Gs_bj (negated next to T_bb)
          const int mt = task - NXS;
          int bb = 1;
          while (bb * (bb + 1) / 2 <= mt) ++bb;
          const int jb = mt - bb * (bb - 1) / 2;
          // computed transposed: M^T[u'][r] = sum_m g_{m-1} Gs[m][u'] T_bb[r][m]
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          acc = mma_nt<false, false>(acc, 16,
              [&](int r, int k) {
                const float4 g0 = *reinterpret_cast<const float4*>(&sm.GT[16 * jb + r][16 * bb + k]);
                const float4 g1 = *reinterpret_cast<const float4*>(&sm.GT[16 * jb + r][16 * bb + k + 4]);
                const float4 m0 = *reinterpret_cast<const float4*>(&sm.gm1[sc][0][16 * bb + k]);
                const float4 m1 = *reinterpret_cast<const float4*>(&sm.gm1[sc][0][16 * bb + k + 4]);
                const float v[8] = {g0.x * m0.x, g0.y * m0.y, g0.z * m0.z, g0.w * m0.w,
                                    g1.x * m1.x, g1.y * m1.y, g1.z * m1.z, g1.w * m1.w};
                return hl_vals(v);
              },
              [&](int r, int k) { return hl_pair(&sm.SAhi[bb][r][k], &sm.SAlo[bb][r][k]); });
          const float mv[4] = {-acc[0], -acc[1], -acc[2], -acc[3]};
          store_split4(&sm.SAhi[bb][lr][16 * (jb + 1) + 4 * lg], &sm.SAlo[bb][lr][16 * (jb + 1) + 4 * lg], mv);
        }
      }
    }
    if constexpr (PERROW) {
      if (wave >= NW - 4) {
        constexpr int RPC = 64 / CS;     // rows per 64 lanes
        scalars_rows(std::integral_constant<int, RW / (4 * RPC)>{}, cur, ci, 0, RPC * (wave - (NW - 4)), 4 * RPC);
      }
    }
    __syncthreads();

    // ================= phase 2 =================
    typename SM::Split* const zt = &sm.slot[cur].ZT;   // keys of ci are consumed
    if (REG) {
      if (!PERROW && wave < nrb) {
        const int ib = 16 * wave;
        {
          for (int bb = 0; bb < NB; ++bb) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_nt<false, false>(acc, 16 * (bb + 1),
                [&](int r, int k) { return hl_pair(&sm.SAhi[bb][r][k], &sm.SAlo[bb][r][k]); },
                [&](int r, int k) {
                  if (k < 16) {
                    // right-hand side r_u = y_u - g_{u-1} (S0 x_u), formed on the fly
                    const int u = 16 * bb + k;
                    const uint4 yb = *reinterpret_cast<const uint4*>(&sm.YT[cur][ib + r][u]);
                    const uint32_t yw[4] = {yb.x, yb.y, yb.z, yb.w};
                    const float4 x0 = *reinterpret_cast<const float4*>(&sm.XS[ib + r][u]);
                    const float4 x1 = *reinterpret_cast<const float4*>(&sm.XS[ib + r][u + 4]);
                    const float4 m0 = *reinterpret_cast<const float4*>(&sm.gm1[sc][0][u]);
                    const float4 m1 = *reinterpret_cast<const float4*>(&sm.gm1[sc][0][u + 4]);
                    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                    const float gm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                      const uint16_t yv = (e & 1) ? (uint16_t)(yw[e >> 1] >> 16) : (uint16_t)(yw[e >> 1] & 0xFFFFu);
                      v[e] = bf16_to_f32(yv) - gm[e] * xs[e];
                    }
                    return hl_vals(v);
                  }
                  return hl_pair(&zt->hi[ib + r][k - 16], &zt->lo[ib + r][k - 16]);
                });
            const float4 zf = *reinterpret_cast<const float4*>(&sm.zeta[sc][0][16 * bb + 4 * lg]);
            const float z[4] = {zf.x * acc[0], zf.y * acc[1], zf.z * acc[2], zf.w * acc[3]};
            store_split4(&zt->hi[ib + lr][16 * bb + 4 * lg], &zt->lo[ib + lr][16 * bb + 4 * lg], z);
            wave_sync();
          }
        }
      }
      if constexpr (PERROW) {
        if (wave < 4 * nrb) row_solve(cur, zt);
      }
    } else {
      // inner-product family: z_t = zeta_t y_t
      for (int idx = tid; idx < RW * CS; idx += NT) {
        const int i = idx / CS, t = idx % CS;
        const float zv = sm.zeta[sc][PERROW ? i : 0][t] * bf16_to_f32(sm.YT[cur][i][t]);
        split1(zv, zt->hi[i][t], zt->lo[i][t]);
      }
    }
    if (has_next && !(REG && PERROW)) {
      // state-independent preparation of chunk ci+1 on the waves not solving
      const int w0 = REG ? NRB : 0;
      const int nws = NW - w0;
      constexpr int NG2 = (REG && !PERROW) ? NLT : 0;   // per-channel Gram waits for phase 3
      if (wave >= w0) {
        for (int task = wave - w0; task < NLT + NG2; task += nws) {
          if (task < NLT) qx_tile(nxt, task);
          else gram_tile(nxt, task - NLT);
        }
      }
      if (!PERROW && wave == NW - 1) scalars(nxt, ci + 1, nxt, 0, wave);
    }
    __syncthreads();

    // ================= phase 3 =================
    if (wave < NQ) {
      const int rbk = wave / NTT, tt = wave % NTT;
      if (rbk < nrb) {
        const int ib = 16 * rbk;
        floatx4 acc = mma_nt<false, false>(qacc, 16 * (tt + 1),
            [&](int r, int k) { return hl_pair(&zt->hi[ib + r][k], &zt->lo[ib + r][k]); },
            [&](int r, int k) { return hl_pair(&sm.Phi[cur][16 * tt + r][k], &sm.Plo[cur][16 * tt + r][k]); });
        const int t = 16 * tt + lr;
        if (t < cval) {
          float ov[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = sm.gam[sc][PERROW ? ib + 4 * lg + e : 0][t] * acc[e];
          opend = make_float4(ov[0], ov[1], ov[2], ov[3]);
          optr = a.o + v_base + (t0 + t) * dv + i0 + ib + 4 * lg;
        }
      }
    }
    {
      // carry tiles, dealt so the diagonal-inverse wave gets the fewest
      constexpr int NC = NRB * NKT;
      for (int task = wave; task < NC; task += NW) {
        const int rbk = task / NKT, tk = task % NKT;
        if (rbk >= nrb) continue;
        const int ib = 16 * rbk;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_nt<true, false>(acc, CS,
            [&](int r, int k) { return hl_bf16(&sm.XT[16 * tk + r][k]); },
            [&](int r, int k) { return hl_pair(&zt->hi[ib + r][k], &zt->lo[ib + r][k]); });
        // lane holds S_new[i][k..k+3] for i = ib + lr, k = 16 tk + 4 lg
        const int i = ib + lr, k0 = 16 * tk + 4 * lg;
        const float gC = sm.gam[sc][PERROW ? i : 0][CS - 1];
        const float4 so = *reinterpret_cast<const float4*>(&sm.S[i][k0]);
        const float sn[4] = {gC * (so.x + acc[0]), gC * (so.y + acc[1]), gC * (so.z + acc[2]),
                             gC * (so.w + acc[3])};
        *reinterpret_cast<float4*>(&sm.S[i][k0]) = make_float4(sn[0], sn[1], sn[2], sn[3]);
        store_split4(&sm.Shi[i][k0], &sm.Slo[i][k0], sn);
      }
    }
    if (has_next) {
      if (REG && !PERROW && wave == NW - 1) diag_inverse(nxt);
      if (REG && PERROW) {
        // Gram of chunk ci+1 on waves 0-2 and its q.x on waves 4-6 (the solve
        // of phase 2 occupies every wave)
        for (int task = wave & 3; task < NLT; task += 4) {
          if (wave >= 4) qx_tile(nxt, task);
          else gram_tile(nxt, task);
        }
      }
    }
    __syncthreads();
  }
  if (optr) *reinterpret_cast<float4*>(optr) = opend;
  if (a.S_out && !sm.bad) {
    for (int idx = tid; idx < RW * DK; idx += NT) {
      const int i = idx / DK, kk = idx % DK;
      if (i0 + i < dv) a.S_out[((long)chain * dv + i0 + i) * DK + kk] = sm.S[i][kk];
    }
  }
  // a chain whose decay products left the range of the chunk algebra: its rows
  // again, exactly, by the recurrence (S_out was left untouched above)
  __syncthreads();
  if (sm.bad) recurrence_rows<DK, NT, 1>(chain, i0, dv - i0 < RW ? dv - i0 : RW);
}

template <int DK, int CS, bool REG, bool PERROW>
hipError_t launch_w1(const SeqArgs& a, hipStream_t stream) {
  W1Geom geo;
  const int nchain = a.batch * a.heads;
  geo.nrbg = (a.dv + RW - 1) / RW;
  geo.remap = (nchain % 8 == 0) ? 1 : 0;
  geo.nchunks = (int)((a.seqlen + CS - 1) / CS);
  const unsigned nblocks = (unsigned)(nchain * geo.nrbg);
  hipLaunchKernelGGL((chunk_w1_kernel<DK, CS, REG, PERROW>), dim3(nblocks), dim3(NT), 0, stream,
                     a, geo);
  return hipGetLastError();
}

template <int DK, int CS>
hipError_t launch_w1_mode(const SeqArgs& a, hipStream_t stream) {
  const bool perrow = a.beta_kind == 2;
  if (perrow) {
    // per-channel scalars are per row: at most 32-step sub-chunks (LDS budget)
    constexpr int CSP = CS > 32 ? 32 : CS;
    return a.regression ? launch_w1<DK, CSP, true, true>(a, stream)
                        : launch_w1<DK, CSP, false, true>(a, stream);
  }
  return a.regression ? launch_w1<DK, CS, true, false>(a, stream)
                      : launch_w1<DK, CS, false, false>(a, stream);
}

}  // namespace

// Window-1 chunk form; cs is the sub-chunk length (16, 32 or 64; 32 at most for
// dk = 128).
hipError_t launch_chunk_w1(const SeqArgs& a, hipStream_t stream, int cs) {
  switch (a.dk) {
    case 16:
      if (cs == 16) return launch_w1_mode<16, 16>(a, stream);
      if (cs == 32) return launch_w1_mode<16, 32>(a, stream);
      return launch_w1_mode<16, 64>(a, stream);
    case 32:
      if (cs == 16) return launch_w1_mode<32, 16>(a, stream);
      if (cs == 32) return launch_w1_mode<32, 32>(a, stream);
      return launch_w1_mode<32, 64>(a, stream);
    case 64:
      if (cs == 16) return launch_w1_mode<64, 16>(a, stream);
      if (cs == 32) return launch_w1_mode<64, 32>(a, stream);
      return launch_w1_mode<64, 64>(a, stream);
    case 128:
      if (cs == 16) return launch_w1_mode<128, 16>(a, stream);
      return launch_w1_mode<128, 32>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace falcon
