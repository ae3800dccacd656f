// falcon_chunk.hip - chunk-parallel form of the Falcon update and readout on
// gfx950 matrix cores.
//
// Method: explainer of arXiv 2608.27763, section 核心方法 §3 ("chunk-parallel":
// split L into chunks, parallel inside a chunk, recurrent across chunks) and the
// 163.com article, section 02 (2) (only the fixed-size state passes between
// chunks; the per-column variant is made GPU-computable with a Gram / WY
// representation and a batched triangular solve).  The algebra below is
// derived from the recurrence itself:
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
// Kernel structure: one workgroup (4 wave64) per (batch*head, block of 16 value
// rows); rows of S evolve independently, so the d_v split needs no
// communication, and the state block stays on chip (LDS, fp32) for the whole
// sequence.  Per sub-chunk:
//   stage    keys (shifted by one, with a halo of B-1 keys for the window), q,
//            v (this block's columns), beta into LDS; keys also transposed
//   MFMA     Gram G = X X^T and P = Q X^T (exact: bf16 inputs, fp32 accumulate)
//   scalars  norms from diag(G), eta, a, prefix products g (wave scan)
//   T        16x16 diagonal-block inverses (I + A_bb)^-1, forward substitution
//   MFMA     S0 X^T, S0 Q^T (S0 split into bf16 hi + lo)
//   solve    blocked forward substitution over 16-unknown blocks: off-diagonal
//            coupling G Z on MFMA (both operands split), diagonal block by
//            T_bb (scalar eta) or per-row substitution (per-channel eta)
//   MFMA     readout O += Z^T P^T, scaled by g_t, stored as fp32
//   MFMA     carry S = g_{c-1} (S0 + F^T X)
// The sub-chunk size is the caller's chunk (window 1) or the largest power of
// two with c*B <= 64, so every triangular system has at most 64 unknowns.
#include "falcon_device.h"
#include "falcon_launch.h"

namespace falcon {
namespace {

constexpr int kChunkThreads = 256;
constexpr int RB = 16;      // value rows per workgroup
constexpr int UP = 64;      // max unknowns per sub-chunk

__device__ __forceinline__ int round_up(int x, int m) { return (x + m - 1) / m * m; }

// One 16x16 output tile: acc[m][n] += sum_k A[m][k] * Bt[n][k], operands stored
// K-contiguous (row stride lda / ldb elements).  K is a multiple of 8; lanes
// whose 8-wide k slot lies beyond K supply zeros.
//   ABF / BBF: operand is exact bf16 (uint16_t*), otherwise fp32 split hi/lo.
template <bool ABF, bool BBF>
__device__ __forceinline__ floatx4 tile_nt(floatx4 acc, const void* A, int lda, const void* Bt,
                                           int ldb, int K) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int kq = (lane >> 4) * 8;
  for (int k0 = 0; k0 < K; k0 += 32) {
    const bool in = (k0 + kq) < K;
    bf16x8 ah, al, bh, bl;
    if (ABF) {
      ah = in ? frag_bf16(static_cast<const uint16_t*>(A) + r * lda + k0 + kq) : zero_frag();
      al = zero_frag();
    } else if (in) {
      frag_split(static_cast<const float*>(A) + r * lda + k0 + kq, ah, al);
    } else {
      ah = al = zero_frag();
    }
    if (BBF) {
      bh = in ? frag_bf16(static_cast<const uint16_t*>(Bt) + r * ldb + k0 + kq) : zero_frag();
      bl = zero_frag();
    } else if (in) {
      frag_split(static_cast<const float*>(Bt) + r * ldb + k0 + kq, bh, bl);
    } else {
      bh = bl = zero_frag();
    }
    acc = mfma16(ah, bh, acc);
    if (!BBF) acc = mfma16(ah, bl, acc);
    if (!ABF) acc = mfma16(al, bh, acc);
  }
  return acc;
}

struct Geom {
  int nchain;     // batch * heads
  int nrb;        // dv / RB
  int remap;      // 1: XCD-aware block mapping
};

template <int DK, int CS>
struct Smem {
  static constexpr int NXP = (CS == 64) ? 64 : CS + 16;   // padded key rows (max over windows)
  static constexpr int GN = (CS == 64) ? 16 : NXP;        // gather-source Gram size
  uint16_t X[NXP][DK + 8];          // keys x_j, row-major
  uint16_t XT[DK][NXP + 8];         // keys transposed
  uint16_t Q[CS][DK + 8];
  float YT[RB][NXP + 4];            // values, this block's columns, transposed
  float S[RB][DK + 4];              // state rows (fp32, carried)
  float Gt[UP][UP + 4];             // masked Gram over unknowns (s(u') < t(u))
  float Pt[CS][UP + 4];             // masked readout weights (s(u') <= t)
  float G[GN][GN + 4];              // key Gram (window > 1)
  float P[CS][GN + 4];              // q . x (window > 1)
  float T[4][16][20];               // diagonal-block inverses
  float XS[RB][NXP + 4];            // S0 x_j
  float RT[RB][UP + 4];             // right-hand sides (transposed)
  float ZT[RB][UP + 4];             // z (transposed)
  float FT[RB][NXP + 4];            // per-key folded z (window > 1)
  float nrm[NXP];
  float beta[RB][CS];
  float gam[RB][CS];
  float gm1[RB][CS];
  float zeta[RB][CS];
};

template <int DK, int CS, bool REG, bool PERROW>
__global__ __launch_bounds__(kChunkThreads) void chunk_kernel(SeqArgs a, Geom geo) {
  using SM = Smem<DK, CS>;
  constexpr int NXP = SM::NXP;
  __shared__ __align__(16) SM sm;

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(a.v);
  const uint16_t* __restrict__ kpg = static_cast<const uint16_t*>(a.k_prev);
  const uint16_t* __restrict__ bg = static_cast<const uint16_t*>(a.beta_t);

  // Block -> (chain, row block).  Workgroups are dealt to the 8 XCDs round
  // robin; with remap, the row blocks of one chain land on one XCD (same L2)
  // and are dispatched back to back, so they share the q/k tiles they all read.
  int chain, rb;
  {
    const int b = blockIdx.x;
    if (geo.remap) {
      const int xcd = b & 7, slot = b >> 3;
      chain = xcd + 8 * (slot / geo.nrb);
      rb = slot % geo.nrb;
    } else {
      chain = b / geo.nrb;
      rb = b % geo.nrb;
    }
  }
  const int i0 = rb * RB;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int B = a.window;
  const long L = a.seqlen;
  const int dv = a.dv;
  const int cs = CS;                   // sub-chunk length (window fits: cs * B <= 64)
  const int U = cs * B;                // unknowns per sub-chunk
  const int NX = cs + B - 1;           // keys per sub-chunk (with halo)
  const int nxp = round_up(NX, 16);
  const int nb = U / 16;               // diagonal blocks
  const long qk_base = (long)chain * L * DK;
  const long v_base = (long)chain * L * dv;

  // state rows
  for (int idx = tid; idx < RB * DK; idx += kChunkThreads) {
    const int i = idx / DK, kk = idx % DK;
    sm.S[i][kk] = a.S0 ? a.S0[((long)chain * dv + i0 + i) * DK + kk] : 0.0f;
  }

  for (long t0 = 0; t0 < L; t0 += CS) {
    const int c = (int)((L - t0) < CS ? (L - t0) : CS);   // valid steps (ragged tail)
    __syncthreads();
    // ---------------- stage ----------------
    constexpr int VPR = DK / 8;   // 16-byte vectors per key row
    for (int idx = tid; idx < NXP * VPR; idx += kChunkThreads) {
      const int jj = idx / VPR, kv = idx % VPR;
      const long g = t0 - (B - 1) + jj;            // global step of key x_g
      uint4 val = {0u, 0u, 0u, 0u};
      if (jj < NX && g < t0 + c) {
        if (g >= 1) val = *reinterpret_cast<const uint4*>(kg + qk_base + (g - 1) * DK + kv * 8);
        else if (g == 0 && kpg) val = *reinterpret_cast<const uint4*>(kpg + (long)chain * DK + kv * 8);
      }
      *reinterpret_cast<uint4*>(&sm.X[jj][kv * 8]) = val;
      const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.XT[kv * 8 + 2 * e][jj] = (uint16_t)(w4[e] & 0xFFFFu);
        sm.XT[kv * 8 + 2 * e + 1][jj] = (uint16_t)(w4[e] >> 16);
      }
    }
    for (int idx = tid; idx < CS * VPR; idx += kChunkThreads) {
      const int t = idx / VPR, kv = idx % VPR;
      uint4 val = {0u, 0u, 0u, 0u};
      if (t < c) val = *reinterpret_cast<const uint4*>(qg + qk_base + (t0 + t) * DK + kv * 8);
      *reinterpret_cast<uint4*>(&sm.Q[t][kv * 8]) = val;
    }
    for (int idx = tid; idx < NXP * (RB / 8); idx += kChunkThreads) {
      const int jj = idx / (RB / 8), h = idx % (RB / 8);
      const long g = t0 - (B - 1) + jj;
      uint4 val = {0u, 0u, 0u, 0u};
      if (jj < NX && g >= 0 && g < t0 + c)
        val = *reinterpret_cast<const uint4*>(vg + v_base + g * dv + i0 + h * 8);
      const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.YT[h * 8 + 2 * e][jj] = bf16_to_f32((uint16_t)(w4[e] & 0xFFFFu));
        sm.YT[h * 8 + 2 * e + 1][jj] = bf16_to_f32((uint16_t)(w4[e] >> 16));
      }
    }
    for (int idx = tid; idx < (PERROW ? RB : 1) * CS; idx += kChunkThreads) {
      const int i = idx / CS, t = idx % CS;
      float bv = a.beta;
      if (t < c) {
        if (a.beta_kind == 1) bv = bf16_to_f32(bg[(long)chain * L + t0 + t]);
        else if (a.beta_kind == 2) bv = bf16_to_f32(bg[((long)chain * L + t0 + t) * dv + i0 + i]);
      }
      sm.beta[i][t] = bv;
    }
    __syncthreads();

    // ---------------- Gram and q.x products (exact, MFMA) ----------------
    if (B == 1) {
      // keys and unknowns coincide: write the masked forms directly
      constexpr int NT = CS / 16;
      for (int task = wave; task < 2 * NT * NT; task += 4) {
        const bool isG = task < NT * NT;
        const int tt = isG ? task : task - NT * NT;
        const int ti = tt / NT, tj = tt % NT;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        if (tj <= ti) {
          const uint16_t* Ap = isG ? &sm.X[16 * ti][0] : &sm.Q[16 * ti][0];
          acc = tile_nt<true, true>(acc, Ap, DK + 8, &sm.X[16 * tj][0], DK + 8, DK);
        }
        const int col = 16 * tj + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * ti + 4 * (lane >> 4) + r;
          if (isG) {
            sm.Gt[row][col] = (col < row) ? acc[r] : 0.0f;
            if (col == row) sm.nrm[row] = acc[r];
          } else {
            sm.Pt[row][col] = (col <= row) ? acc[r] : 0.0f;
          }
        }
      }
      // unknowns beyond CS (CS < 64): zero rows/cols so K-padding reads zeros
      for (int idx = tid; idx < UP * UP; idx += kChunkThreads) {
        const int r = idx / UP, cc = idx % UP;
        if (r >= CS || cc >= CS) {
          if (REG) sm.Gt[r][cc] = 0.0f;
          if (r < CS) sm.Pt[r][cc] = 0.0f;
        }
      }
    } else {
      const int nt = nxp / 16;
      constexpr int NQ = CS / 16;
      for (int task = wave; task < nt * nt + NQ * nt; task += 4) {
        const bool isG = task < nt * nt;
        const int tt = isG ? task : task - nt * nt;
        const int ti = tt / nt, tj = tt % nt;
        const uint16_t* Ap = isG ? &sm.X[16 * ti][0] : &sm.Q[16 * ti][0];
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = tile_nt<true, true>(acc, Ap, DK + 8, &sm.X[16 * tj][0], DK + 8, DK);
        const int col = 16 * tj + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * ti + 4 * (lane >> 4) + r;
          if (isG) sm.G[row][col] = acc[r];
          else sm.P[row][col] = acc[r];
        }
      }
      __syncthreads();
      for (int jj = tid; jj < nxp; jj += kChunkThreads) sm.nrm[jj] = sm.G[jj][jj];
      // gather over unknowns u = t*B + w with key j(u) = t - w + B - 1
      for (int idx = tid; idx < UP * UP; idx += kChunkThreads) {
        const int u = idx / UP, u2 = idx % UP;
        const int t = u / B, s = u2 / B;
        if (REG) {
          float gv = 0.0f;
          if (u < U && u2 < U && s < t) gv = sm.G[t - u % B + B - 1][s - u2 % B + B - 1];
          sm.Gt[u][u2] = gv;
        }
        if (u < CS) {
          float pv = 0.0f;
          if (u2 < U && s <= u) pv = sm.P[u][s - u2 % B + B - 1];
          sm.Pt[u][u2] = pv;
        }
      }
    }
    __syncthreads();

    // ---------------- per-step scalars ----------------
    // eta_t = beta_t / (eps + n_t), a_t = 1 - eta_t lambda; padded steps and
    // the fresh-sequence first step (x_1 = 0 on S_0 = 0) take eta = 0, a = 1.
    {
      const int t = lane;
      float n = 0.0f;
      for (int w = 0; w < B; ++w) {
        const int jj = t - w + B - 1;
        if (t < CS) n += sm.nrm[jj];
      }
      const bool live = t < c && !(t0 + t == 0 && kpg == nullptr);
      constexpr int NR = PERROW ? RB : 1;
      for (int i = wave; i < NR; i += 4) {
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
        if (t < CS) {
          sm.gam[i][t] = gsc;
          sm.gm1[i][t] = gprev;
          sm.zeta[i][t] = eta / gsc;
        }
      }
    }
    __syncthreads();

    // ---------------- diagonal-block inverses (scalar eta, regression) ----------------
    if (REG && !PERROW) {
      for (int bb = wave; bb < nb; bb += 4) {
        if (lane < 16) {
          const int cc = lane;
          float tc[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ur = 16 * bb + r;
            const float gr = sm.gm1[0][ur / B];
            float acc = (r == cc) ? 1.0f : 0.0f;
#pragma unroll
            for (int m = 0; m < r; ++m) {
              const int um = 16 * bb + m;
              acc -= gr * sm.Gt[ur][um] * sm.zeta[0][um / B] * tc[m];
            }
            tc[r] = acc;
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) sm.T[bb][r][cc] = tc[r];
        }
      }
    }

    // ---------------- S0 products ----------------
    floatx4 oacc = {0.f, 0.f, 0.f, 0.f};
    const int ntq = CS / 16;
    if (wave < ntq)
      oacc = tile_nt<false, true>(oacc, &sm.S[0][0], DK + 4, &sm.Q[16 * wave][0], DK + 8, DK);
    if (REG) {
      for (int tj = wave; tj < nxp / 16; tj += 4) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = tile_nt<false, true>(acc, &sm.S[0][0], DK + 4, &sm.X[16 * tj][0], DK + 8, DK);
        const int col = 16 * tj + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.XS[4 * (lane >> 4) + r][col] = acc[r];
      }
    }
    __syncthreads();

    // ---------------- right-hand sides / inner-product z ----------------
    for (int idx = tid; idx < RB * UP; idx += kChunkThreads) {
      const int i = idx / UP, u = idx % UP;
      const int ir = PERROW ? i : 0;
      float val = 0.0f;
      if (u < U) {
        const int t = u / B, jj = t - u % B + B - 1;
        if (REG) val = sm.YT[i][jj] - sm.gm1[ir][t] * sm.XS[i][jj];
        else val = sm.zeta[ir][t] * sm.YT[i][jj];
      }
      if (REG) sm.RT[i][u] = val;
      else sm.ZT[i][u] = val;
    }
    __syncthreads();

    // ---------------- blocked forward substitution (regression) ----------------
    if (REG) {
      for (int bb = 0; bb < nb; ++bb) {
        if (wave == 0) {
          const int u0 = 16 * bb;
          if (bb > 0) {
            floatx4 cacc = {0.f, 0.f, 0.f, 0.f};
            cacc = tile_nt<false, false>(cacc, &sm.Gt[u0][0], UP + 4, &sm.ZT[0][0], UP + 4, u0);
            const int i = lane & 15;
            const int ir = PERROW ? i : 0;
            float4 rv = *reinterpret_cast<float4*>(&sm.RT[i][u0 + 4 * (lane >> 4)]);
            float rr[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int u = u0 + 4 * (lane >> 4) + r;
              rr[r] -= sm.gm1[ir][u / B] * cacc[r];
            }
            *reinterpret_cast<float4*>(&sm.RT[i][u0 + 4 * (lane >> 4)]) =
                make_float4(rr[0], rr[1], rr[2], rr[3]);
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          if (!PERROW) {
            floatx4 eacc = {0.f, 0.f, 0.f, 0.f};
            eacc = tile_nt<false, false>(eacc, &sm.T[bb][0][0], 20, &sm.RT[0][u0], UP + 4, 16);
            const int i = lane & 15;
            float zz[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int u = u0 + 4 * (lane >> 4) + r;
              zz[r] = sm.zeta[0][u / B] * eacc[r];
            }
            *reinterpret_cast<float4*>(&sm.ZT[i][u0 + 4 * (lane >> 4)]) =
                make_float4(zz[0], zz[1], zz[2], zz[3]);
          } else if (lane < RB) {
            const int i = lane;
            float z[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int u = u0 + r;
              float acc = 0.0f;
#pragma unroll
              for (int m = 0; m < r; ++m) acc += sm.Gt[u][u0 + m] * z[m];
              const float e = sm.RT[i][u] - sm.gm1[i][u / B] * acc;
              z[r] = sm.zeta[i][u / B] * e;
            }
#pragma unroll
            for (int r = 0; r < 16; r += 4)
              *reinterpret_cast<float4*>(&sm.ZT[i][u0 + r]) = make_float4(z[r], z[r + 1], z[r + 2], z[r + 3]);
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
      }
      __syncthreads();
    }

    // ---------------- readout ----------------
    if (wave < ntq) {
      oacc = tile_nt<false, false>(oacc, &sm.ZT[0][0], UP + 4, &sm.Pt[16 * wave][0], UP + 4,
                                   round_up(U, 16));
      const int t = 16 * wave + (lane & 15);
      const int ib = 4 * (lane >> 4);
      if (t < c) {
        float ov[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ov[r] = sm.gam[PERROW ? ib + r : 0][t] * oacc[r];
        *reinterpret_cast<float4*>(a.o + v_base + (t0 + t) * dv + i0 + ib) =
            make_float4(ov[0], ov[1], ov[2], ov[3]);
      }
    }
    // fold z onto keys for the window (j(u) = t - w + B - 1)
    if (B > 1) {
      for (int idx = tid; idx < RB * NXP; idx += kChunkThreads) {
        const int i = idx / NXP, jj = idx % NXP;
        float f = 0.0f;
        for (int w = 0; w < B; ++w) {
          const int t = jj + w - (B - 1);
          if (t >= 0 && t < CS) f += sm.ZT[i][t * B + w];
        }
        sm.FT[i][jj] = f;
      }
      __syncthreads();
    }

    // ---------------- carry: S = g_{c-1} (S0 + F^T X) ----------------
    {
      const float* Fp = (B > 1) ? &sm.FT[0][0] : &sm.ZT[0][0];
      const int ldf = (B > 1) ? NXP + 4 : UP + 4;
      for (int tk = wave; tk < DK / 16; tk += 4) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = tile_nt<false, true>(acc, Fp, ldf, &sm.XT[16 * tk][0], NXP + 8, nxp);
        const int kk = 16 * tk + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * (lane >> 4) + r;
          sm.S[i][kk] = sm.gam[PERROW ? i : 0][CS - 1] * (sm.S[i][kk] + acc[r]);
        }
      }
    }
  }
  __syncthreads();
  if (a.S_out) {
    for (int idx = tid; idx < RB * DK; idx += kChunkThreads) {
      const int i = idx / DK, kk = idx % DK;
      a.S_out[((long)chain * dv + i0 + i) * DK + kk] = sm.S[i][kk];
    }
  }
}

template <int DK, int CS, bool REG, bool PERROW>
hipError_t launch4(const SeqArgs& a, hipStream_t stream) {
  Geom geo;
  geo.nchain = a.batch * a.heads;
  geo.nrb = a.dv / RB;
  geo.remap = (geo.nchain % 8 == 0) ? 1 : 0;
  const unsigned nblocks = (unsigned)(geo.nchain * geo.nrb);
  hipLaunchKernelGGL((chunk_kernel<DK, CS, REG, PERROW>), dim3(nblocks), dim3(kChunkThreads), 0,
                     stream, a, geo);
  return hipGetLastError();
}

template <int DK, int CS>
hipError_t launch_mode(const SeqArgs& a, hipStream_t stream) {
  const bool perrow = a.beta_kind == 2;
  if (a.regression) {
    return perrow ? launch4<DK, CS, true, true>(a, stream) : launch4<DK, CS, true, false>(a, stream);
  }
  return perrow ? launch4<DK, CS, false, true>(a, stream) : launch4<DK, CS, false, false>(a, stream);
}

template <int DK>
hipError_t launch_cs(const SeqArgs& a, hipStream_t stream, int cs) {
  switch (cs) {
    case 16: return launch_mode<DK, 16>(a, stream);
    case 32: return launch_mode<DK, 32>(a, stream);
    case 64: return launch_mode<DK, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Sub-chunk length: the caller's chunk, halved until chunk * window <= 64.
int chunk_sub_length(int chunk, int window) {
  int c = chunk;
  while (c * window > UP) c >>= 1;
  return c;
}

hipError_t launch_chunk(const SeqArgs& a, hipStream_t stream) {
  (void)hipGetLastError();
  const int cs = chunk_sub_length(a.chunk, a.window);
  switch (a.dk) {
    case 16: return launch_cs<16>(a, stream, cs);
    case 32: return launch_cs<32>(a, stream, cs);
    case 64: return launch_cs<64>(a, stream, cs);
    case 128: return launch_cs<128>(a, stream, cs);
  }
  return hipErrorInvalidValue;
}

}  // namespace falcon
