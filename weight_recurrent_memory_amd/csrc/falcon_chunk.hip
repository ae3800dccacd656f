// falcon_chunk.hip - chunk-parallel form of the Falcon update and readout on
// gfx950 matrix cores.
//
// Method: explainer of arXiv 2608.27763, section 核心方法 §3 ("chunk-parallel":
// split L into chunks, parallel inside a chunk, recurrent across chunks) and the
// 163.com article, section 02 (2) (only the fixed-size state passes between
// chunks; the per-column variant is made GPU-computable with a Gram / WY
// representation and a batched triangular solve).  The algebra below is
// derived from the recurrence itself.
//
// Within a sub-chunk of c steps that starts from state S0 (per value row i;
// t, s are local steps, w = 0..B-1 a window slot, u = t*B + w an unknown whose
// key is j(u) = t - w):
//   g_t    = prod_{r<=t} a_r,  g_{-1} = 1,   zeta_t = eta_t / g_t
//   regression unknowns e_u = y_{j(u)} - S_{t-1} x_{j(u)} solve the
//   unit-lower-triangular system
//     e_u + g_{t-1} sum_{s(u')<t} G[j(u), j(u')] z_{u'} = y_{j(u)} - g_{t-1} (S0 x_{j(u)})
//     with z_u = zeta_t e_u and G the Gram matrix of the keys;
//   inner-product family: z_u = zeta_t y_{j(u)} (no solve);
//   o_t = g_t (S0 q_t + sum_{s(u)<=t} (q_t . x_{j(u)}) z_u)
//   S_c = g_{c-1} (S0 + sum_j F_j x_j^T),   F_j = sum_{u: j(u)=j} z_u
//
// Work decomposition.  One workgroup of 8 wave64 owns one (batch*head) chain
// and 32 value rows (two blocks of 16); rows of S evolve independently, so the
// d_v split needs no communication, and the fp32 state stays in LDS for the
// whole sequence.  The per-chain quantities (Gram, q.x, decay products,
// triangular factors) are computed once per workgroup and shared by both row
// blocks.  Per sub-chunk (phase = the work between two workgroup barriers):
//   P0  commit the prefetched q/k/v/beta registers to LDS (keys also
//       transposed, key norms by lane-group reductions), then issue the global
//       loads of the next sub-chunk so HBM latency hides behind this one
//   P1  MFMA: Gram X X^T and P = Q X^T (exact: bf16 inputs, fp32 accumulate),
//       S0 Q^T; wave 0: eta, a, g (prefix-product wave scan), zeta
//   P2  wave 0: 16x16 diagonal-block inverses T_bb = (I + A_bb)^-1 by forward
//       substitution; other waves: S0 X^T and the right-hand sides
//   P2' MFMA: M_bj = T_bb diag(g_{t-1}) G_bj for the off-diagonal blocks
//   P3  blocked solve, one wave per row block: each 16-unknown stage is one
//       MFMA group  E_b = [T_bb | -M_b0 | ... ] [R_b ; Z_0 ; ...]
//       (per-channel eta: off-diagonal coupling on MFMA, diagonal block by
//       per-row forward substitution)
//   P4  MFMA: readout O^T = S0 Q^T + Z^T P^T scaled by g_t, stored fp32;
//       carry S = g_{c-1} (S0 + F^T X)
// Operands that are not exact bf16 inputs are stored in LDS pre-split into
// bf16 hi + lo (split-bf16, Henry, Tang & Heinecke, ARITH 2019) so the MFMA
// loops issue no conversion work: hi*hi + hi*lo + lo*hi with fp32 accumulation.
// The sub-chunk length is the caller's chunk, halved until chunk * window <= 64
// (at most 64 unknowns per triangular system) and to at most 32 for dk = 128
// (LDS budget); the result does not depend on it beyond rounding.
#include "falcon_device.h"
#include "falcon_exact.h"
#include "falcon_launch.h"
#include "falcon_mma.h"

namespace falcon {
namespace {

constexpr int RB = 16;    // value rows per row block (one MFMA tile)
constexpr int NRB = 2;    // row blocks per workgroup
constexpr int RW = RB * NRB;
constexpr int NW = 8;     // waves per workgroup
constexpr int NT = 64 * NW;

template <int DK, int CS, int B>
struct Cfg {
  static constexpr int U = CS * B;                 // unknowns per sub-chunk
  static constexpr int NB = U / 16;                // 16-unknown blocks
  static constexpr int NX = CS + B - 1;            // keys per sub-chunk (window halo)
  static constexpr int NXP = (NX + 15) / 16 * 16;
  static constexpr int VPR = DK / 8;               // 16-byte vectors per key row
  static constexpr int KV = (NXP * VPR + NT - 1) / NT;
  static constexpr int QV = (CS * VPR + NT - 1) / NT;
  static constexpr int YV = (NXP * (RW / 8) + NT - 1) / NT;
  static_assert(U % 16 == 0 && U <= 64, "at most 64 unknowns, whole blocks");
};

template <int DK, int CS, int B, bool REG, bool PERROW>
struct Lds {
  using C = Cfg<DK, CS, B>;
  static constexpr int U = C::U, NXP = C::NXP, NB = C::NB;
  static constexpr int SR = PERROW ? RW : 1;       // rows of per-step scalars
  struct Split {
    uint16_t hi[RW][U + 8];
    uint16_t lo[RW][U + 8];
  };
  union {                    // keys (P0..P2), then z pre-split (P3..P4)
    uint16_t X[NXP][DK + 8];
    Split ZT;
  } ra;
  union {                    // queries (P0..P1), then right-hand sides (P2..P3)
    uint16_t Q[CS][DK + 8];
    Split RT;
  } rb;
  uint16_t XT[DK][NXP + 8];          // keys transposed (carry operand)
  float YT[RW][NXP + 4];             // values of this workgroup's rows, transposed
  float S[RW][DK + 4];               // state rows, fp32
  uint16_t Shi[RW][DK + 8];          // state rows, split
  uint16_t Slo[RW][DK + 8];
  float OT[RW][CS + 4];              // S0 q_t
  uint16_t Phi[CS][U + 8];           // masked q.x over unknowns, split
  uint16_t Plo[CS][U + 8];
  float GT[REG ? U : 1][U + 4];      // masked Gram over unknowns (see use)
  float G[B > 1 ? NXP : 1][NXP + 4]; // key Gram (window gather source)
  float P[B > 1 ? CS : 1][NXP + 4];  // key q.x (window gather source)
  float XS[(REG && B > 1) ? RW : 1][NXP + 4];
  uint16_t SAhi[(REG && !PERROW) ? NB : 1][16][U + 8];  // [T_bb | -M_b0 | ...]
  uint16_t SAlo[(REG && !PERROW) ? NB : 1][16][U + 8];
  uint16_t FThi[B > 1 ? RW : 1][NXP + 8];               // folded z (window)
  uint16_t FTlo[B > 1 ? RW : 1][NXP + 8];
  float RP[PERROW && REG ? RW : 1][U + 4];              // per-row right-hand sides
  float nrm[NXP];
  float beta[SR][CS];
  float gam[SR][CS];
  float gm1[SR][CS];
  float zeta[SR][CS];
  int bad;                           // some sub-chunk's decay products left the range
};

struct Geom {
  int nchain;
  int nrbg;    // row-block groups per chain (ceil(dv / RW))
  int remap;   // XCD-aware block mapping
};

template <int DK, int CS, int B, bool REG, bool PERROW>
__global__ __launch_bounds__(NT) void chunk_kernel(SeqArgs a, Geom geo) {
  using C = Cfg<DK, CS, B>;
  using SM = Lds<DK, CS, B, REG, PERROW>;
  constexpr int U = C::U, NB = C::NB, NX = C::NX, NXP = C::NXP, VPR = C::VPR;
  constexpr int KV = C::KV, QV = C::QV, YV = C::YV;
  constexpr int NTT = CS / 16;     // step tiles
  static_assert(!(PERROW && B > 1), "per-channel variants have window 1");
  __shared__ __align__(16) SM sm;

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(a.v);
  const uint16_t* __restrict__ kpg = static_cast<const uint16_t*>(a.k_prev);
  const uint16_t* __restrict__ xhg = static_cast<const uint16_t*>(a.x_hist);
  const uint16_t* __restrict__ yhg = static_cast<const uint16_t*>(a.y_hist);
  const uint16_t* __restrict__ bg = static_cast<const uint16_t*>(a.beta_t);

  // Block -> (chain, row-block group).  Workgroups are dealt to the 8 XCDs round
  // robin; with remap, the groups of one chain land on one XCD (same L2) and are
  // dispatched back to back, so they share the q/k tiles they all read.
  int chain, rbg;
  {
    const int b = blockIdx.x;
    if (geo.remap) {
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
  const int nrb = (dv - i0) >= RW ? NRB : 1;       // active row blocks (dv = 16: one)
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int lane = tid & 63;
  const int lr = lane & 15;          // tile column / fragment row
  const int lg = lane >> 4;          // lane group
  const long L = a.seqlen;
  const long qk_base = (long)chain * L * DK;
  const long v_base = (long)chain * L * dv;
  // z lives over the keys (dead after P2') for the regression family and over
  // the queries (dead after P1) for the inner-product family, whose z is written
  // in P2 while the keys are still needed for the transposed copy.
  typename SM::Split* const zt = REG ? &sm.ra.ZT : &sm.rb.RT;

  // ---------------- prefetch registers ----------------
  uint4 pk[KV], pq[QV], py[YV];
  float pb[(PERROW ? RW : 1) * CS / NT + 1];
  auto prefetch = [&](long t0) __attribute__((always_inline)) {
    const int c = (int)((L - t0) < CS ? (L - t0) : CS);
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int idx = tid + v * NT;
      const int jj = idx / VPR, kv = idx % VPR;
      const long g = t0 - (B - 1) + jj;            // global step of key x_g
      uint4 val = {0u, 0u, 0u, 0u};
      if (idx < NXP * VPR && jj < NX && g < t0 + c) {
        if (g >= a.key_shift) val = *reinterpret_cast<const uint4*>(kg + qk_base + (g - a.key_shift) * DK + kv * 8);
        else if (g == 0 && kpg) val = *reinterpret_cast<const uint4*>(kpg + (long)chain * DK + kv * 8);
        else if (g < 0 && xhg)   // carried window history, slot B-1+g
          val = *reinterpret_cast<const uint4*>(xhg + ((long)chain * (B - 1) + (B - 1) + g) * DK + kv * 8);
      }
      pk[v] = val;
    }
#pragma unroll
    for (int v = 0; v < QV; ++v) {
      const int idx = tid + v * NT;
      const int t = idx / VPR, kv = idx % VPR;
      uint4 val = {0u, 0u, 0u, 0u};
      if (idx < CS * VPR && t < c) val = *reinterpret_cast<const uint4*>(qg + qk_base + (t0 + t) * DK + kv * 8);
      pq[v] = val;
    }
#pragma unroll
    for (int v = 0; v < YV; ++v) {
      const int idx = tid + v * NT;
      const int jj = idx / (RW / 8), h = idx % (RW / 8);
      const long g = t0 - (B - 1) + jj;
      uint4 val = {0u, 0u, 0u, 0u};
      if (idx < NXP * (RW / 8) && jj < NX && g < t0 + c && i0 + h * 8 < dv) {
        if (g >= 0) val = *reinterpret_cast<const uint4*>(vg + v_base + g * dv + i0 + h * 8);
        else if (yhg) val = *reinterpret_cast<const uint4*>(yhg + ((long)chain * (B - 1) + (B - 1) + g) * dv + i0 + h * 8);
      }
      py[v] = val;
    }
    constexpr int NBT = (PERROW ? RW : 1) * CS;
#pragma unroll
    for (int v = 0; v < NBT / NT + 1; ++v) {
      const int idx = tid + v * NT;
      float bv = a.beta;
      if (idx < NBT) {
        const int i = idx / CS, t = idx % CS;
        if (t < c) {
          if (a.beta_kind == 1) bv = bf16_to_f32(bg[(long)chain * L + t0 + t]);
          else if (a.beta_kind == 2 && i0 + i < dv)
            bv = bf16_to_f32(bg[((long)chain * L + t0 + t) * dv + i0 + i]);
        }
      }
      pb[v] = bv;
    }
  };

  // ---------------- state ----------------
  if (tid == 0) sm.bad = 0;
  for (int idx = tid; idx < RW * DK; idx += NT) {
    const int i = idx / DK, kk = idx % DK;
    float s = 0.0f;
    if (a.S0 && i0 + i < dv) s = a.S0[((long)chain * dv + i0 + i) * DK + kk];
    sm.S[i][kk] = s;
    split1(s, sm.Shi[i][kk], sm.Slo[i][kk]);
  }
  prefetch(0);

  for (long t0 = 0; t0 < L; t0 += CS) {
    const int c = (int)((L - t0) < CS ? (L - t0) : CS);     // valid steps (ragged tail)
    __syncthreads();
    // ================= P0: commit prefetched tiles =================
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int idx = tid + v * NT;
      const int jj = idx / VPR, kv = idx % VPR;
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
      if (idx < NXP * VPR) {
        *reinterpret_cast<uint4*>(&sm.ra.X[jj][kv * 8]) = val;
        if (kv == 0) sm.nrm[jj] = part;
      }
    }
#pragma unroll
    for (int v = 0; v < QV; ++v) {
      const int idx = tid + v * NT;
      if (idx < CS * VPR) *reinterpret_cast<uint4*>(&sm.rb.Q[idx / VPR][(idx % VPR) * 8]) = pq[v];
    }
#pragma unroll
    for (int v = 0; v < YV; ++v) {
      const int idx = tid + v * NT;
      if (idx < NXP * (RW / 8)) {
        const int jj = idx / (RW / 8), h = idx % (RW / 8);
        const uint4 val = py[v];
        const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sm.YT[h * 8 + 2 * e][jj] = bf16_to_f32((uint16_t)(w4[e] & 0xFFFFu));
          sm.YT[h * 8 + 2 * e + 1][jj] = bf16_to_f32((uint16_t)(w4[e] >> 16));
        }
      }
    }
    {
      constexpr int NBT = (PERROW ? RW : 1) * CS;
#pragma unroll
      for (int v = 0; v < NBT / NT + 1; ++v) {
        const int idx = tid + v * NT;
        if (idx < NBT) sm.beta[idx / CS][idx % CS] = pb[v];
      }
    }
    if (t0 + CS < L) prefetch(t0 + CS);
    __syncthreads();

    // ================= P1: Gram, q.x, S0 q; scalars =================
    if (wave == 0 || (PERROW && wave < 4)) {
      // eta_t = beta_t / (eps + n_t), a_t = 1 - eta_t lambda; padded steps and the
      // fresh-sequence first step (x_1 = 0 on S_0 = 0) take eta = 0, a = 1.
      const int t = lane;
      float n = 0.0f;
      if (t < CS) {
#pragma unroll
        for (int w = 0; w < B; ++w) n += sm.nrm[t - w + B - 1];
      }
      const bool live = t < c && !(t0 + t == 0 && kpg == nullptr && a.key_shift);
      constexpr int NR = PERROW ? RW : 1;
      constexpr int WST = PERROW ? 4 : 1;
      for (int i = wave; i < NR; i += WST) {
        float eta = 0.0f, dec = 1.0f;
        if (live) {
          eta = sm.beta[i][t] / (a.eps + n);
          dec = 1.0f - eta * a.lambda;
        }
        float gsc = dec;   // inclusive prefix product over the wave's lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const float o = __shfl_up(gsc, d, 64);
          if (lane >= d) gsc *= o;
        }
        float gprev = __shfl_up(gsc, 1, 64);
        if (lane == 0) gprev = 1.0f;
        if (__builtin_amdgcn_ballot_w64(t < CS && gauge_out_of_range(gsc, dec)) != 0 && lane == 0) sm.bad = 1;
        if (t < CS) {
          sm.gam[i][t] = gsc;
          sm.gm1[i][t] = gprev;
          sm.zeta[i][t] = eta / gsc;
        }
      }
    }
    {
      // task list: [Gram tiles][q.x tiles][S0 q tiles]
      constexpr int GN = B == 1 ? NTT : NXP / 16;      // Gram tile grid
      constexpr int NG = REG ? (B == 1 ? NTT * (NTT + 1) / 2 : GN * GN) : 0;
      constexpr int NP = B == 1 ? NTT * (NTT + 1) / 2 : NTT * (NXP / 16);
      constexpr int NQ = NRB * NTT;
      const int first = PERROW ? 4 : 1;      // waves busy with scalars start later
      for (int task = (wave + NW - first) % NW; task < NG + NP + NQ; task += NW) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        if (task < NG + NP) {
          const bool isG = task < NG;
          int ti, tj, tt = isG ? task : task - NG;
          if (B == 1) {     // lower-triangular tile enumeration
            ti = 0;
            while ((ti + 1) * (ti + 2) / 2 <= tt) ++ti;
            tj = tt - ti * (ti + 1) / 2;
          } else {
            const int gn = isG ? GN : NXP / 16;
            ti = tt / gn;
            tj = tt % gn;
          }
          const uint16_t* Arow = isG ? &sm.ra.X[16 * ti][0] : &sm.rb.Q[16 * ti][0];
          acc = mma_nt<true, true>(acc, DK,
              [&](int r, int k) { return hl_bf16(Arow + r * (DK + 8) + k); },
              [&](int r, int k) { return hl_bf16(&sm.ra.X[16 * tj + r][k]); });
          const int col = 16 * tj + lr;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = 16 * ti + 4 * lg + e;
            if (B == 1) {
              if (isG) {
                const float gv = (col < row) ? acc[e] : 0.0f;
                if (PERROW) sm.GT[row][col] = gv;       // Gt[u][u']
                else sm.GT[col][row] = gv;              // Gt^T[u'][u]
              } else {
                split1((col <= row) ? acc[e] : 0.0f, sm.Phi[row][col], sm.Plo[row][col]);
              }
            } else {
              if (isG) sm.G[row][col] = acc[e];
              else sm.P[row][col] = acc[e];
            }
          }
        } else {
          const int qt = task - NG - NP;
          const int rbk = qt / NTT, tt = qt % NTT;
          if (rbk < nrb) {
            acc = mma_nt<false, true>(acc, DK,
                [&](int r, int k) { return hl_pair(&sm.Shi[16 * rbk + r][k], &sm.Slo[16 * rbk + r][k]); },
                [&](int r, int k) { return hl_bf16(&sm.rb.Q[16 * tt + r][k]); });
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.OT[16 * rbk + 4 * lg + e][16 * tt + lr] = acc[e];
          }
        }
      }
    }
    __syncthreads();

    if (B > 1) {
      // gather over unknowns u = t*B + w (key j(u) = t - w + B - 1)
      for (int idx = tid; idx < (REG ? U * U : 0) + CS * U; idx += NT) {
        if (REG && idx < U * U) {
          const int u = idx / U, u2 = idx % U;
          const int t = u / B, s = u2 / B;
          const float gv = (s < t) ? sm.G[t - u % B + B - 1][s - u2 % B + B - 1] : 0.0f;
          sm.GT[u2][u] = gv;                           // Gt^T (scalar eta only)
        } else {
          const int j = idx - (REG ? U * U : 0);
          const int t = j / U, u2 = j % U, s = u2 / B;
          const float pv = (s <= t) ? sm.P[t][s - u2 % B + B - 1] : 0.0f;
          split1(pv, sm.Phi[t][u2], sm.Plo[t][u2]);
        }
      }
      __syncthreads();
    }

    // ================= P2: diagonal inverses || S0 x and right-hand sides =================
    if (REG) {
      if (!PERROW && wave == NW - 1) {
        // T_bb = (I + Gamma_- Gs Z)^-1 = Gamma_- (I + Gs D)^-1 Gamma_-^{-1},
        // D = diag(zeta_m g_{t(m)-1}); lane = 16 b + column.
        const int bb = (lane >> 4) < NB ? (lane >> 4) : 0;   // lanes beyond NB blocks redo block 0
        const int cc = lane & 15;
        const int u0 = 16 * bb;
        float gmv[16], dm[16], acc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tr = (u0 + r) / B;
          gmv[r] = sm.gm1[0][tr];
          dm[r] = sm.zeta[0][tr] * gmv[r];
          acc[r] = (r == cc) ? 1.0f : 0.0f;
        }
        // rows of the block, two ahead of use (Gt^T[u_m][u_r] = Gs[r][m])
        float4 g0[4], g1[4], g2[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          g0[q4] = *reinterpret_cast<const float4*>(&sm.GT[u0][u0 + 4 * q4]);
          g1[q4] = *reinterpret_cast<const float4*>(&sm.GT[u0 + 1][u0 + 4 * q4]);
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          if (m + 2 < 16) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
              g2[q4] = *reinterpret_cast<const float4*>(&sm.GT[u0 + m + 2][u0 + 4 * q4]);
          }
          const float sv = dm[m] * acc[m];
          const float grow[16] = {g0[0].x, g0[0].y, g0[0].z, g0[0].w, g0[1].x, g0[1].y,
                                  g0[1].z, g0[1].w, g0[2].x, g0[2].y, g0[2].z, g0[2].w,
                                  g0[3].x, g0[3].y, g0[3].z, g0[3].w};
#pragma unroll
          for (int r = m + 1; r < 16; ++r) acc[r] -= grow[r] * sv;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            g0[q4] = g1[q4];
            g1[q4] = g2[q4];
          }
        }
        if ((lane >> 4) < NB) {
          const float inv_c = 1.0f / sm.gm1[0][(u0 + cc) / B];
#pragma unroll
          for (int r = 0; r < 16; ++r)
            split1(gmv[r] * acc[r] * inv_c, sm.SAhi[bb][r][cc], sm.SAlo[bb][r][cc]);
        }
      }
      // S0 x_j tiles (row block, key tile) -> right-hand sides; with scalar eta
      // the last wave is busy with the diagonal inverses
      constexpr int NXT = NXP / 16;
      constexpr int NWS = PERROW ? NW : NW - 1;
      for (int task = wave; wave < NWS && task < NRB * NXT; task += NWS) {
        const int rbk = task / NXT, tj = task % NXT;
        if (rbk >= nrb) continue;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_nt<false, true>(acc, DK,
            [&](int r, int k) { return hl_pair(&sm.Shi[16 * rbk + r][k], &sm.Slo[16 * rbk + r][k]); },
            [&](int r, int k) { return hl_bf16(&sm.ra.X[16 * tj + r][k]); });
        const int jj = 16 * tj + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * rbk + 4 * lg + e;
          if (B == 1) {
            const float rv = (jj < CS) ? sm.YT[i][jj] - sm.gm1[PERROW ? i : 0][jj] * acc[e] : 0.0f;
            if (PERROW) sm.RP[i][jj] = rv;
            else split1(rv, sm.rb.RT.hi[i][jj], sm.rb.RT.lo[i][jj]);
          } else {
            sm.XS[i][jj] = acc[e];
          }
        }
      }
    } else {
      // inner-product family: z_u = zeta_t y_{j(u)}
      for (int idx = tid; idx < RW * U; idx += NT) {
        const int i = idx / U, u = idx % U;
        const int t = u / B, jj = t - u % B + B - 1;
        const float zv = sm.zeta[PERROW ? i : 0][t] * sm.YT[i][jj];
        split1(zv, zt->hi[i][u], zt->lo[i][u]);
      }
    }
    __syncthreads();

    // ================= P2': off-diagonal solve blocks, window right-hand sides =================
    if (REG && !PERROW) {
      // M_bj = T_bb diag(g_{t-1})_b Gs_bj, stored negated next to T_bb
      constexpr int NM = NB * (NB - 1) / 2;
      for (int task = wave; task < NM; task += NW) {
        int bb = 1;
        while (bb * (bb + 1) / 2 <= task) ++bb;
        const int jb = task - bb * (bb - 1) / 2;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_nt<false, false>(acc, 16,
            [&](int r, int k) { return hl_pair(&sm.SAhi[bb][r][k], &sm.SAlo[bb][r][k]); },
            [&](int r, int k) {
              float v[8];
              const float* gp = &sm.GT[16 * jb + r][16 * bb + k];   // Gs[u_m][u'] = Gt^T[u'][u_m]
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] = gp[e] * sm.gm1[0][(16 * bb + k + e) / B];
              return hl_vals(v);
            });
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * lg + e;
          split1(-acc[e], sm.SAhi[bb][r][16 * (jb + 1) + lr], sm.SAlo[bb][r][16 * (jb + 1) + lr]);
        }
      }
    }
    // keys transposed for the carry: XT[k][j], one 16-byte write per (k, 8 keys)
    for (int idx = tid; idx < DK * (NXP / 8); idx += NT) {
      const int kk = idx % DK, j8 = idx / DK;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)sm.ra.X[8 * j8 + 2 * e][kk] | ((uint32_t)sm.ra.X[8 * j8 + 2 * e + 1][kk] << 16);
      *reinterpret_cast<uint4*>(&sm.XT[kk][8 * j8]) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    if (REG && B > 1) {
      for (int idx = tid; idx < RW * U; idx += NT) {
        const int i = idx / U, u = idx % U;
        const int t = u / B, jj = t - u % B + B - 1;
        const float rv = sm.YT[i][jj] - sm.gm1[0][t] * sm.XS[i][jj];
        split1(rv, sm.rb.RT.hi[i][u], sm.rb.RT.lo[i][u]);
      }
    }
    __syncthreads();

    // ================= P3: blocked solve, one wave per row block =================
    if (REG && wave < nrb) {
      const int rbk = wave;
      const int ib = 16 * rbk;
      if (!PERROW) {
        for (int bb = 0; bb < NB; ++bb) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          acc = mma_nt<false, false>(acc, 16 * (bb + 1),
              [&](int r, int k) { return hl_pair(&sm.SAhi[bb][r][k], &sm.SAlo[bb][r][k]); },
              [&](int r, int k) {
                if (k < 16) return hl_pair(&sm.rb.RT.hi[ib + r][16 * bb + k], &sm.rb.RT.lo[ib + r][16 * bb + k]);
                return hl_pair(&zt->hi[ib + r][k - 16], &zt->lo[ib + r][k - 16]);
              });
          // E_b[u][i]: lane holds u = 16 bb + 4 lg + e, i = lr
          float z[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] = sm.zeta[0][(16 * bb + 4 * lg + e) / B] * acc[e];
          store_split4(&zt->hi[ib + lr][16 * bb + 4 * lg], &zt->lo[ib + lr][16 * bb + 4 * lg], z);
          wave_sync();
        }
      } else {
        for (int bb = 0; bb < NB; ++bb) {
          const int u0 = 16 * bb;
          if (bb > 0) {
            floatx4 cacc = {0.f, 0.f, 0.f, 0.f};
            cacc = mma_nt<false, false>(cacc, u0,
                [&](int r, int k) { return hl_f32(&sm.GT[u0 + r][k]); },
                [&](int r, int k) { return hl_pair(&zt->hi[ib + r][k], &zt->lo[ib + r][k]); });
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int u = u0 + 4 * lg + e;
              sm.RP[ib + lr][u] -= sm.gm1[ib + lr][u] * cacc[e];
            }
            wave_sync();
          }
          if (lane < 16) {
            const int i = ib + lane;
            float acc[16], z[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
              const int u = u0 + m;
              const float e = sm.RP[i][u] - sm.gm1[i][u] * acc[m];
              z[m] = sm.zeta[i][u] * e;
#pragma unroll
              for (int r = m + 1; r < 16; ++r) acc[r] += sm.GT[u0 + r][u] * z[m];
            }
#pragma unroll
            for (int r = 0; r < 16; r += 4)
              store_split4(&zt->hi[i][u0 + r], &zt->lo[i][u0 + r], &z[r]);
          }
          wave_sync();
        }
      }
    }
    __syncthreads();

    // ================= P4: fold (window), readout, carry =================
    if (B > 1) {
      for (int idx = tid; idx < RW * NXP; idx += NT) {
        const int i = idx / NXP, jj = idx % NXP;
        float f = 0.0f;
#pragma unroll
        for (int w = 0; w < B; ++w) {
          const int t = jj + w - (B - 1);
          if (t >= 0 && t < CS) {
            const int u = t * B + w;
            f += bf16_to_f32(zt->hi[i][u]) + bf16_to_f32(zt->lo[i][u]);
          }
        }
        split1(f, sm.FThi[i][jj], sm.FTlo[i][jj]);
      }
      __syncthreads();
    }
    {
      constexpr int NR_T = NRB * NTT;          // readout tiles
      constexpr int NC_T = NRB * (DK / 16);    // carry tiles
      for (int task = wave; task < NR_T + NC_T; task += NW) {
        if (task < NR_T) {
          const int rbk = task / NTT, tt = task % NTT;
          if (rbk >= nrb) continue;
          const int ib = 16 * rbk;
          floatx4 acc;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = sm.OT[ib + 4 * lg + e][16 * tt + lr];
          const int K = (B == 1) ? 16 * (tt + 1) : (16 * (tt + 1) * B < U ? 16 * (tt + 1) * B : U);
          acc = mma_nt<false, false>(acc, K,
              [&](int r, int k) { return hl_pair(&zt->hi[ib + r][k], &zt->lo[ib + r][k]); },
              [&](int r, int k) { return hl_pair(&sm.Phi[16 * tt + r][k], &sm.Plo[16 * tt + r][k]); });
          const int t = 16 * tt + lr;
          if (t < c) {
            float ov[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) ov[e] = sm.gam[PERROW ? ib + 4 * lg + e : 0][t] * acc[e];
            *reinterpret_cast<float4*>(a.o + v_base + (t0 + t) * dv + i0 + ib + 4 * lg) =
                make_float4(ov[0], ov[1], ov[2], ov[3]);
          }
        } else {
          const int ct = task - NR_T;
          const int rbk = ct / (DK / 16), tk = ct % (DK / 16);
          if (rbk >= nrb) continue;
          const int ib = 16 * rbk;
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          if (B == 1) {
            acc = mma_nt<false, true>(acc, CS,
                [&](int r, int k) { return hl_pair(&zt->hi[ib + r][k], &zt->lo[ib + r][k]); },
                [&](int r, int k) { return hl_bf16(&sm.XT[16 * tk + r][k]); });
          } else {
            acc = mma_nt<false, true>(acc, NXP,
                [&](int r, int k) { return hl_pair(&sm.FThi[ib + r][k], &sm.FTlo[ib + r][k]); },
                [&](int r, int k) { return hl_bf16(&sm.XT[16 * tk + r][k]); });
          }
          const int kk = 16 * tk + lr;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = ib + 4 * lg + e;
            const float s = sm.gam[PERROW ? i : 0][CS - 1] * (sm.S[i][kk] + acc[e]);
            sm.S[i][kk] = s;
            split1(s, sm.Shi[i][kk], sm.Slo[i][kk]);
          }
        }
      }
    }
  }
  __syncthreads();
  if (a.S_out && !sm.bad) {
    for (int idx = tid; idx < RW * DK; idx += NT) {
      const int i = idx / DK, kk = idx % DK;
      if (i0 + i < dv) a.S_out[((long)chain * dv + i0 + i) * DK + kk] = sm.S[i][kk];
    }
  }
  // a chain whose decay products left the range of the chunk algebra: its rows
  // again, exactly, by the recurrence (S_out was left untouched above)
  __syncthreads();
  if (sm.bad) recurrence_rows<DK, NT, B>(chain, i0, dv - i0 < RW ? dv - i0 : RW);
}

template <int DK, int CS, int B, bool REG, bool PERROW>
hipError_t launch5(const SeqArgs& a, hipStream_t stream) {
  Geom geo;
  geo.nchain = a.batch * a.heads;
  geo.nrbg = (a.dv + RW - 1) / RW;
  geo.remap = (geo.nchain % 8 == 0) ? 1 : 0;
  const unsigned nblocks = (unsigned)(geo.nchain * geo.nrbg);
  hipLaunchKernelGGL((chunk_kernel<DK, CS, B, REG, PERROW>), dim3(nblocks), dim3(NT), 0, stream,
                     a, geo);
  return hipGetLastError();
}

template <int DK, int CS, int B>
hipError_t launch_mode(const SeqArgs& a, hipStream_t stream) {
  return a.regression ? launch5<DK, CS, B, true, false>(a, stream)
                      : launch5<DK, CS, B, false, false>(a, stream);
}

template <int DK>
hipError_t launch_shape(const SeqArgs& a, hipStream_t stream, int cs) {
  switch (a.window) {
    case 2:
      if (cs == 16) return launch_mode<DK, 16, 2>(a, stream);
      if (cs == 32) return launch_mode<DK, 32, 2>(a, stream);
      break;
    case 3: return launch_mode<DK, 16, 3>(a, stream);
    case 4: return launch_mode<DK, 16, 4>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Sub-chunk length: the caller's chunk, halved until chunk * window <= 64, and
// at most 32 steps when dk = 128.
int chunk_sub_length(int chunk, int window, int dk) {
  int c = chunk;
  while (c * window > 64) c >>= 1;
  if (dk == 128 && c > 32) c = 32;
  return c;
}

hipError_t launch_chunk(const SeqArgs& a, hipStream_t stream, void* ws, size_t ws_bytes) {
  (void)hipGetLastError();
  const int cs = chunk_sub_length(a.chunk, a.window, a.dk);
  // a call of at most 64 steps (window 1, gains shared by the value rows) is a
  // single chunk: the masked-parallel kernel solves that system once for every
  // value row, exactly (no decay product is divided by) and faster than the
  // 32-step kernel's pipeline, which needs several chunks to fill
  if (a.window == 1 && a.beta_kind != 2 && a.seqlen <= kMaskedMaxLen) return launch_masked(a, stream);
  if (chunk_wy_supported(a)) return launch_chunk_wy(a, stream);
  if (chunk_ip_supported(a)) return launch_chunk_ip(a, stream);
  if (ws != nullptr) {
    const size_t need = chunk_wyb2_workspace_bytes(a);
    if (need > 0 && ws_bytes >= need) return launch_chunk_wyb2(a, ws, stream);
  }
  if (chunk_wyb_supported(a)) return launch_chunk_wyb(a, stream);
  if (a.window == 1) return launch_chunk_w1(a, stream, cs);
  switch (a.dk) {
    case 16: return launch_shape<16>(a, stream, cs);
    case 32: return launch_shape<32>(a, stream, cs);
    case 64: return launch_shape<64>(a, stream, cs);
    case 128: return launch_shape<128>(a, stream, cs);
  }
  return hipErrorInvalidValue;
}

}  // namespace falcon
