// falcon_masked.hip - masked-parallel form of the Falcon update for short
// sequences (explainer of arXiv 2608.27763, section 核心方法 §3: the recurrence
// unrolled under a causal mask into one parallel, attention-like system over
// the whole sequence; the summary's 计算形式与数值稳定 lists the same form).
//
// A call of L <= 64 steps is one masked system.  Samples j are the window
// history (B-1 rows) followed by x_1..x_L with their values y_j; queries are
// q_1..q_L.  The only dk-long work is two products on the fp32 matrix cores:
//   G = X X^T   (samples x samples),   P = X Q^T   (samples x queries).
// The state itself never appears in the sequential part: value row i of S is
// represented by its projections on every sample and query of the sequence,
// r_j = s_i . x_j and p_u = s_i . q_u (initially S0 x_j and S0 q_u).  Step t
// with window W_t (explainer §1, article 163.com 02 (1) for eta and the decay):
//   e_j = y_{j,i} - r_j                        (regression; y_{j,i} for the
//                                               inner-product family)
//   r_m <- a_t r_m + eta_t sum_{j in W_t} e_j G[j][m]   for every later sample m
//   p_u <- a_t p_u + eta_t sum_{j in W_t} e_j P[j][u]   for every query u >= t
//   o_t = p_t
// This is the unit-lower-triangular masked system (I + A) e = y - D S0 x with
// A[(t,j)][(s,j')] = eta_s D[t-1][s] G[j'][j] and D[t][s] = prod_{s<r<=t} a_r,
// solved column by column (forward substitution, right-looking): the causal
// mask is the order of the steps and the decay mask is applied as a running
// product, so nothing is divided by a decay product and strong forgetting
// needs no special case.  The final state is S_L = D[L][0] S0 + sum_j c_j x_j^T,
// c_j = sum over the steps s whose window holds sample j of eta_s D[L][s] e_{s,j},
// kept as a running sum and multiplied by X once at the end.
//
// Work decomposition: one workgroup per (batch*head, block of RB <= 64 value
// rows), RB / 4 waves; a value row is one 16-lane DPP row, lane l holding the
// samples and queries 16 m + l.  The step loop is unrolled, so the owner lane
// and slot of every window sample are compile-time constants: e is broadcast
// from its owner with one DPP row_newbcast.
#include <type_traits>

#include "falcon_device.h"
#include "falcon_launch.h"
#include "falcon_mma.h"

namespace falcon {
namespace {

constexpr int kMaskedMaxL = kMaskedMaxLen;
constexpr int kNSP = 80;            // sample rows: 64 + up to 7 history, padded to 16
constexpr int kMaskedMaxRows = 64;  // value rows per workgroup

template <int DKM>
struct MaskedLds {
  float X[kNSP][DKM + 4];           // samples, fp32 (row stride 16-byte aligned)
  float G[kNSP][kNSP];              // X X^T
  float P[kNSP][kMaskedMaxL];       // X Q^T
  union {
    float Y[kNSP][kMaskedMaxRows];  // values of the workgroup's rows [sample][row], read
                                    // into registers before the step loop
    float C[kMaskedMaxRows][kNSP];  // final-state coefficients [row][sample], written in it
  };
  float O[kMaskedMaxL][kMaskedMaxRows];
  float Bc[kMaskedMaxL][kMaskedMaxRows];  // per-channel gains [step][row]
  float eta[kMaskedMaxL], dec[kMaskedMaxL], nt[kMaskedMaxL];
  float BP[kMaskedMaxL / 16 + 1][kMaskedMaxRows];  // per-block decay products [block][row]
};

__device__ __forceinline__ float ld_elem(const void* p, long i, bool bf16) {
  return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

// four consecutive elements (16-byte aligned for fp32, 8-byte for bf16)
__device__ __forceinline__ float4 ld4(const void* p, long i, bool bf16) {
  if (bf16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    return make_float4(__builtin_bit_cast(float, u.x << 16), __builtin_bit_cast(float, u.x & 0xffff0000u),
                       __builtin_bit_cast(float, u.y << 16), __builtin_bit_cast(float, u.y & 0xffff0000u));
  }
  return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
}

__device__ __forceinline__ floatx4 mfma_f32x4(const float4 a, const float4 b, floatx4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
}

// v of lane N of the same 16-lane row, on every lane of the row (the nop gives
// the two wait states a DPP read of a just-written VGPR needs)
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
  float r;
  asm("s_nop 1\n\tv_mov_b32_dpp %0, %1 row_newbcast:%2 row_mask:0xf bank_mask:0xf"
      : "=v"(r) : "v"(v), "i"(N));
  return r;
}
// the same for a lane index that is a constant after unrolling (the switch folds)
__device__ __forceinline__ float row_bcast_dyn(float v, int n) {
  switch (n) {
    case 0: return row_bcast<0>(v);
    case 1: return row_bcast<1>(v);
    case 2: return row_bcast<2>(v);
    case 3: return row_bcast<3>(v);
    case 4: return row_bcast<4>(v);
    case 5: return row_bcast<5>(v);
    case 6: return row_bcast<6>(v);
    case 7: return row_bcast<7>(v);
    case 8: return row_bcast<8>(v);
    case 9: return row_bcast<9>(v);
    case 10: return row_bcast<10>(v);
    case 11: return row_bcast<11>(v);
    case 12: return row_bcast<12>(v);
    case 13: return row_bcast<13>(v);
    case 14: return row_bcast<14>(v);
    default: return row_bcast<15>(v);
  }
}

// f(std::integral_constant<int, t>) for t = T0, T0 + 1, ... while it returns true
// (at most N calls): every call sees t as a constant expression
template <int T0, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    if (f(std::integral_constant<int, T0>{})) static_for<T0 + 1, N - 1>(f);
  }
}

template <int DKM, int BW, bool RG>
__global__ __launch_bounds__(1024) void masked_kernel(SeqArgs a, int rb) {
  using SM = MaskedLds<DKM>;
  __shared__ __align__(16) SM sm;
  const bool bf = a.dtype == 0;
  const int DK = a.dk, dv = a.dv;
  const int L = a.seqlen;                    // <= 64
  const int NS = L + BW - 1;                 // samples
  const int NT = (NS + 15) / 16, QT = (L + 15) / 16;
  const int chain = blockIdx.x;
  const int row0 = blockIdx.y * rb;
  const int tid = threadIdx.x, nth = rb * 16;
  const int lane = tid & 63, wave = tid >> 6, nw = nth >> 6;
  const int ks = a.key_shift;
  const bool fresh = ks == 1 && a.k_prev == nullptr;
  const long qk_base = (long)chain * L * DK;
  const long v_base = (long)chain * L * dv;

  // ---- stage samples, values and per-channel gains in LDS
  const int DK4 = DK / 4;
  for (int idx = tid; idx < kNSP * DK4; idx += nth) {
    const int jj = idx / DK4, c = 4 * (idx % DK4);
    const int g = jj - (BW - 1);             // 0-based step of the sample
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (jj < NS) {
      if (g >= ks) x = ld4(a.k, qk_base + (long)(g - ks) * DK + c, bf);
      else if (g == 0) { if (a.k_prev) x = ld4(a.k_prev, (long)chain * DK + c, bf); }
      else if (g < 0 && a.x_hist) x = ld4(a.x_hist, ((long)chain * (BW - 1) + (BW - 1) + g) * DK + c, bf);
    }
    *reinterpret_cast<float4*>(&sm.X[jj][c]) = x;
  }
  for (int idx = tid; idx < kNSP * rb; idx += nth) {
    const int jj = idx / rb, i = idx % rb;
    const int g = jj - (BW - 1);
    float y = 0.0f;
    if (jj < NS) {
      if (g >= 0) y = ld_elem(a.v, v_base + (long)g * dv + row0 + i, bf);
      else if (a.y_hist) y = ld_elem(a.y_hist, ((long)chain * (BW - 1) + (BW - 1) + g) * dv + row0 + i, bf);
    }
    sm.Y[jj][i] = y;
  }
  if (a.beta_kind == 2) {
    for (int idx = tid; idx < L * rb; idx += nth) {
      const int t = idx / rb, i = idx % rb;
      sm.Bc[t][i] = ld_elem(a.beta_t, ((long)chain * L + t) * dv + row0 + i, bf);
    }
  }
  __syncthreads();

  // ---- G = X X^T and P = X Q^T, 16 x 16 tiles on the fp32 matrix cores (lane l
  // holds rows 4 (l / 16) + r, column l % 16; K step k of a 16-wide block is fed
  // by lane group k / 4, element k % 4)
  {
    const int mn = lane & 15, k4 = 4 * (lane >> 4);
    const int ntile = NT * NT + NT * QT;
    for (int tile = wave; tile < ntile; tile += nw) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      const bool isg = tile < NT * NT;
      const int ta = isg ? tile / NT : (tile - NT * NT) / QT;
      const int tb = isg ? tile % NT : (tile - NT * NT) % QT;
      const int arow = 16 * ta + mn, brow = 16 * tb + mn;
      if (isg) {
        for (int kb = 0; kb < DK; kb += 16)
          acc = mfma_f32x4(*reinterpret_cast<const float4*>(&sm.X[arow][kb + k4]),
                           *reinterpret_cast<const float4*>(&sm.X[brow][kb + k4]), acc);
      } else {
        const bool live = brow < L;
        for (int kb = 0; kb < DK; kb += 16) {
          const float4 qv = live ? ld4(a.q, qk_base + (long)brow * DK + kb + k4, bf)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
          acc = mfma_f32x4(*reinterpret_cast<const float4*>(&sm.X[arow][kb + k4]), qv, acc);
        }
      }
      const int orow = 16 * ta + 4 * (lane >> 4), ocol = 16 * tb + mn;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (isg) sm.G[orow + r][ocol] = acc[r];
        else sm.P[orow + r][ocol] = acc[r];
      }
    }
  }

  // ---- per-lane projections of the start state: r_j = S0_i . x_j, p_u = S0_i . q_u
  const int l16 = lane & 15;
  const int il = 4 * wave + (lane >> 4);     // value row of this 16-lane row
  const int row = row0 + il;
  float r[5], p[4], y[5], c[2] = {0.0f, 0.0f};
#pragma unroll
  for (int m = 0; m < 5; ++m) r[m] = 0.0f;
#pragma unroll
  for (int m = 0; m < 4; ++m) p[m] = 0.0f;
  if (a.S0) {
    const float* s0 = a.S0 + ((long)chain * dv + row) * DK;
    for (int kb = 0; kb < DK; kb += 4) {
      const float4 s = *reinterpret_cast<const float4*>(s0 + kb);
      if (RG) {
#pragma unroll
        for (int m = 0; m < 5; ++m) {
          const float4 x = *reinterpret_cast<const float4*>(&sm.X[16 * m + l16][kb]);
          r[m] = __builtin_fmaf(s.x, x.x, __builtin_fmaf(s.y, x.y, __builtin_fmaf(s.z, x.z, __builtin_fmaf(s.w, x.w, r[m]))));
        }
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int u = 16 * m + l16;
        const float4 qv = u < L ? ld4(a.q, qk_base + (long)u * DK + kb, bf) : make_float4(0.f, 0.f, 0.f, 0.f);
        p[m] = __builtin_fmaf(s.x, qv.x, __builtin_fmaf(s.y, qv.y, __builtin_fmaf(s.z, qv.z, __builtin_fmaf(s.w, qv.w, p[m]))));
      }
    }
  }
  __syncthreads();

  // ---- per-step scalars: n_t = sum of the window's squared norms (the diagonal
  // of G), eta_t = beta_t / (eps + n_t), a_t = 1 - eta_t lambda; a fresh sequence
  // (S_0 = 0, x_1 = 0) takes its first step with eta = 0, a = 1
  for (int t = tid; t < L; t += nth) {
    float n = 0.0f;
#pragma unroll
    for (int w = 0; w < BW; ++w) n += sm.G[t + BW - 1 - w][t + BW - 1 - w];
    float beta = a.beta;
    if (a.beta_kind == 1) beta = ld_elem(a.beta_t, (long)chain * L + t, bf);
    float eta = beta / (a.eps + n), dec = 1.0f - eta * a.lambda;
    if (t == 0 && fresh) { eta = 0.0f; dec = 1.0f; }
    sm.nt[t] = n;
    sm.eta[t] = eta;
    sm.dec[t] = dec;
  }
#pragma unroll
  for (int m = 0; m < 5; ++m) y[m] = sm.Y[16 * m + l16][il];
  __syncthreads();

  // ---- the masked system, step by step, in blocks of 16 steps.  Each block is
  // unrolled, so the step's lane and the slots of its window samples are
  // constants; between blocks every per-lane array moves down one slot, so slot
  // m of block M holds samples and queries 16 (M + m) + l.
  const bool chan = a.beta_kind == 2;
  const bool want_s = a.S_out != nullptr;
  int M = 0;
  for (; 16 * M < L; ++M) {
    const int t0 = 16 * M;
    float bp = 1.0f;                         // product of the block's decays
    static_for<0, 16>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      const int t = t0 + i;
      if (t >= L) return false;
      __builtin_amdgcn_sched_barrier(0);     // keep each step's loads in its step
      float eta, dec;
      if (chan) {
        eta = sm.Bc[t][il] / (a.eps + sm.nt[t]);
        dec = 1.0f - eta * a.lambda;
        if (t == 0 && fresh) { eta = 0.0f; dec = 1.0f; }
      } else {
        eta = sm.eta[t];
        dec = sm.dec[t];
      }
      float he[BW];
#pragma unroll
      for (int w = 0; w < BW; ++w) {
        const int jr = i + BW - 1 - w;       // sample t + BW-1-w, relative to the block
        const float ev = RG ? y[jr >> 4] - r[jr >> 4] : y[jr >> 4];
        he[w] = eta * row_bcast_dyn(ev, jr & 15);
      }
      if (RG) {
#pragma unroll
        for (int m = 0; m < 5; ++m) {
          // slot still holds samples of a later window, and samples at all
          if (16 * m + 15 >= i + 1 && t0 + 16 * m < NS) {
            float acc = dec * r[m];
#pragma unroll
            for (int w = 0; w < BW; ++w)
              acc = __builtin_fmaf(he[w], sm.G[t + BW - 1 - w][t0 + 16 * m + l16], acc);
            r[m] = acc;
          }
        }
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (16 * m + 15 >= i && t0 + 16 * m < L) {   // queries not yet read
          float acc = dec * p[m];
#pragma unroll
          for (int w = 0; w < BW; ++w)
            acc = __builtin_fmaf(he[w], sm.P[t + BW - 1 - w][t0 + 16 * m + l16], acc);
          p[m] = acc;
        }
      }
      if (l16 == i) sm.O[t][il] = p[0];
      if (want_s) {
        bp *= dec;
#pragma unroll
        for (int m = 0; m < 2; ++m)
          if (16 * m <= i + BW - 1) c[m] *= dec;
#pragma unroll
        for (int w = 0; w < BW; ++w) {
          const int jr = i + BW - 1 - w;
          if (l16 == (jr & 15)) c[jr >> 4] += he[w];
        }
      }
      return true;
    });
    if (want_s) {
      // samples t0 .. t0 + 15 are in no later window: later steps only decay them
      sm.C[il][t0 + l16] = c[0];
      if (l16 == 0) sm.BP[M][il] = bp;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      r[m] = r[m + 1];
      y[m] = y[m + 1];
    }
    r[4] = 0.0f;
    y[4] = 0.0f;
#pragma unroll
    for (int m = 0; m < 3; ++m) p[m] = p[m + 1];
    p[3] = 0.0f;
    c[0] = c[1];
    c[1] = 0.0f;
  }
  if (want_s) sm.C[il][16 * M + l16] = c[0];   // the window's samples past the last block
  __syncthreads();

  // ---- outputs: o (coalesced over value rows), then the final state
  for (int idx = tid; idx < L * rb; idx += nth) {
    const int t = idx / rb, i = idx % rb;
    a.o[v_base + (long)t * dv + row0 + i] = sm.O[t][i];
  }
  if (want_s) {
    // S_L = D[L][0] S0 + sum_j c_j x_j^T; the coefficients of block M still take
    // the decays of the blocks after it: walk the blocks from the last one with
    // the running product f of those decays (f ends as D[L][0])
    const int NB = M;
    for (int idx = tid; idx < rb * DK; idx += nth) {
      const int i = idx / DK, col = idx % DK;
      float acc = 0.0f, f = 1.0f;
      for (int b = NB; b >= 0; --b) {
        float part = 0.0f;
        const int j1 = 16 * b + 16 < NS ? 16 * b + 16 : NS;
        for (int jj = 16 * b; jj < j1; ++jj) part = __builtin_fmaf(sm.C[i][jj], sm.X[jj][col], part);
        acc = __builtin_fmaf(f, part, acc);
        if (b < NB) f *= sm.BP[b][i];
      }
      const long off = ((long)chain * dv + row0 + i) * DK + col;
      if (a.S0) acc = __builtin_fmaf(f, a.S0[off], acc);
      a.S_out[off] = acc;
    }
  }
}

// ---------------------------------------------------------------------------
// Window 1 with gains shared by the value rows (Falcon-1/1A, and Falcon-2/2A,
// Falcon-3/3A called with window 1 and a scalar or per-token beta): every value
// row sees the same masked system, so it is solved once for all of them on the
// matrix cores.  Steps t = 0..63 (steps past L: zero sample, eta = 0, a = 1),
// D[t][s] = prod_{s<r<=t} a_r, d_t = prod_{r<=t} a_r (d_{-1} = 1):
//   A[t][s] = eta_s D[t-1][s] (x_t . x_s)   (s < t)
//   (I + A) E = Y - diag(d_{t-1}) X S0^T     (regression; E = Y for the
//                                             inner-product family)
//   W[t][s] = eta_s D[t][s] (q_t . x_s)      (s <= t)
//   O = diag(d_t) Q S0^T + W E
//   S_L = d_63 S0 + E^T diag(eta_s D[63][s]) X
// (the same unrolling of the recurrence as above, written as matrices).  Every
// decay factor is a product of decays, never a quotient: inside a 16-step block
// D comes from a running product; across blocks it factors as
// D[t-1][s] = suf_s mid(k, b) pin_t, with suf_s the product over the rest of
// s's block k, mid the products of the whole blocks strictly between k and b,
// and pin_t the product over t's block b before t (up to t itself for W), so
// strong forgetting stays exact here too.  The solve is blocked:
// T_bb = (I + A_bb)^-1 by a DPP forward substitution, then
// E_b = T_bb (R_b - sum_{k<b} A_bk E_k) on the matrix cores.  Precision: the
// entry-wise factors (A, W, T, E) are split-bf16 (Henry, Tang & Heinecke, ARITH
// 2019: hi + lo, three products); every dot product that may cancel (x . x,
// q . x, X S0^T, Q S0^T) is exact up to fp32 accumulation: bf16 inputs on the
// bf16 matrix cores, the fp32 start state in three bf16 pieces (2^-24), fp32
// inputs on the fp32 matrix cores.
//
// Work decomposition: one workgroup (4 waves, about 37 KB of LDS at dk = 64, so
// four workgroups share a compute unit) per (chain, block of <= 64 value rows);
// phases separated by barriers: (0) every global read issued at once, as
// 16-byte loads (samples, queries, values and squared norms to LDS; the
// start-state row to registers), (1) per-step scalars and block products |
// the Gram and key-query tiles, kept in registers in the layout of the operand
// fragments they become | X S0^T and Q S0^T, (2) the diagonal blocks of T |
// the -A and W fragments, (3) each wave solves and reads out its 16 value rows,
// then forms its rows of the final state.
constexpr int kWyThreads = 256;

template <int DK, bool F32IN>
struct MaskedWyLds {
  // bf16 inputs: samples and queries as bf16 (exact; product depth padded to the
  // MFMA K of 32); fp32 inputs: as fp32, for exact products on the fp32 matrix cores
  using XE = std::conditional_t<F32IN, float, uint16_t>;
  static constexpr int KP = F32IN ? DK : (DK < 32 ? 32 : DK);
  static constexpr int XR = F32IN ? DK + 4 : KP + 8;   // row over the features
  static constexpr int FR = 32;                         // bf16 row of an operand fragment
  XE X[64][XR];                     // samples, K-contiguous
  static constexpr int YR = F32IN ? 64 + 4 : 64 + 8;   // row over the value columns
  union {
    struct {
      XE Q[64][XR];                 // queries (until phase 1 ends)
      XE Y[64][YR];                 // values of the workgroup's rows (read to registers
                                    // at the start of phase 1)
    } qy;
    struct {
      uint16_t Ah[4][16][FR], Al[4][16][FR];   // -A fragments by (block, pair of blocks)
      uint16_t Wh[6][16][FR], Wl[6][16][FR];   // W fragments
    } f;
  };
  union {
    float Gd[4][16][20];            // diagonal 16 x 16 tiles of X X^T, [b][t][s]
    float Acol[4][16][20];          // columns of the diagonal blocks of A, [b][s][t]
    float TS[4][16][20];            // diagonal blocks of (I + A)^-1, [b][r][n]
  };
  float nrm[64], bet[64];
  alignas(16) float eta[64];
  alignas(16) float dec[64];
  alignas(16) float pinx[64];       // product over the block before t
  alignas(16) float pini[64];       // the same up to t
  alignas(16) float suf[64];        // product over the block after t
  float bpre[5], bsuf[4], mid[4][4];
};

// Position of the 16-byte group lg (0..3) of fragment row lr in a 64-byte row of
// Ah/Al/Wh/Wl: the group index is XORed with bits 2-3 of the row, so the 16 rows
// that a quarter-wave reads or writes at one group fall on 16 different 4-bank
// slots instead of four rows per slot.
__device__ __forceinline__ int wy_frag_col(int lr, int lg) { return 8 * (lg ^ ((lr >> 2) & 3)); }

template <int N>
__device__ __forceinline__ float wy_shr(float v, float fill) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill), __builtin_bit_cast(int, v),
                                                             0x110 + N, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float wy_shl(float v, float fill) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill), __builtin_bit_cast(int, v),
                                                             0x100 + N, 0xF, 0xF, false));
}
// acc + g(lane N of this 16-lane row) * r (g is loaded from LDS, never written
// by the vector ALU, so the DPP read needs no wait states)
template <int N>
__device__ __forceinline__ float wy_fmac_bcast(float acc, float g, float r) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(g), "v"(r), "i"(N));
  return acc;
}
// column n (this lane) of (I + A_bb)^-1: x_p = [p == n] - sum_{q<p} A[p][q] x_q,
// with A[.][q] held by lane q of the 16-lane row in g[]
template <int P>
__device__ __forceinline__ void wy_sweep(float (&x)[16], float (&acc)[16], const float (&g)[16]) {
  x[P] -= acc[P];
#pragma unroll
  for (int r = P + 1; r < 16; ++r) acc[r] = wy_fmac_bcast<P>(acc[r], g[r], x[P]);
  if constexpr (P < 15) wy_sweep<P + 1>(x, acc, g);
}
__device__ __forceinline__ floatx4 wy_mma3(floatx4 acc, const HL& a, const HL& b) {
  acc = mfma16(a.hi, b.lo, acc);
  acc = mfma16(a.lo, b.hi, acc);
  return mfma16(a.hi, b.hi, acc);
}
__device__ __forceinline__ floatx4 wy_mma2(floatx4 acc, const bf16x8& a, const HL& b) {
  acc = mfma16(a, b.hi, acc);
  return mfma16(a, b.lo, acc);
}
// 4 values in slots 0-3 and 4 in slots 4-7 as one split fragment
__device__ __forceinline__ HL wy_hl(const float* a, const float* b) {
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return hl_vals(v);
}
// 8 consecutive input elements as fp32 (16-byte aligned for bf16, 32 for fp32)
template <bool F32IN>
__device__ __forceinline__ void wy_load8(const void* p, long i, float (&v)[8]) {
  if constexpr (F32IN) {
    const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    const float4 y = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i + 4);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
}
// 8 exact bf16 values to an LDS row
__device__ __forceinline__ void wy_put8(uint16_t* row, const float (&v)[8]) {
  uint32_t h[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
  *reinterpret_cast<uint4*>(row) = make_uint4(h[0], h[1], h[2], h[3]);
}
// 8 fp32 values as three bf16 fragments whose sum is the value to 2^-24
// (an exact bf16 operand times the three pieces: an fp32-exact product)
struct Split3 {
  bf16x8 p[3];
};
__device__ __forceinline__ Split3 wy_split3(const float (&v)[8]) {
  uint32_t w[3][4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float r0 = v[2 * e], r1 = v[2 * e + 1];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const uint32_t h = pack_bf16x2(r0, r1);
      w[k][e] = h;
      r0 -= __uint_as_float(h << 16);
      r1 -= __uint_as_float(h & 0xffff0000u);
    }
  }
  Split3 s;
#pragma unroll
  for (int k = 0; k < 3; ++k) s.p[k] = __builtin_bit_cast(bf16x8, make_uint4(w[k][0], w[k][1], w[k][2], w[k][3]));
  return s;
}

// HS0: the call carries a start state (its terms cost registers, so a fresh
// call, which has none, runs at a higher occupancy)
template <int DK, bool RG, bool F32IN, bool HS0>
__global__ __launch_bounds__(kWyThreads, HS0 ? 2 : 4) void masked_wy_kernel(SeqArgs a, int rb) {
  using SM = MaskedWyLds<DK, F32IN>;
  constexpr int KP = SM::KP, NKS = KP / 32, NCT = DK / 16, C8 = DK / 8;
  constexpr int IT = (64 * C8 + kWyThreads - 1) / kWyThreads;   // 8-element pieces per thread
  __shared__ __align__(16) SM sm;
  const int L = a.seqlen;                    // 1..64
  const int dv = a.dv;
  const int chain = blockIdx.x;
  const int row0 = blockIdx.y * rb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int ks = a.key_shift;
  const bool fresh = ks == 1 && a.k_prev == nullptr;
  constexpr bool has_s0 = HS0;
  const long qk_base = (long)chain * L * DK;
  const long v_base = (long)chain * L * dv;
  const bool solver = wave < rb / 16;        // wave w owns value rows 16 w .. 16 w + 15
  const int col = row0 + 16 * wave + lr;     // the lane's value row (solver waves)

  // ---- phase 0: every global read is issued before any is used, as 16-byte
  // loads: values, samples (x_t = k_{t-ks}, x_0 = k_prev or 0 under the prefix
  // pairing) and queries go to LDS, with the samples' squared norms; the
  // start-state row to registers
  constexpr int IV = (64 * 8 + kWyThreads - 1) / kWyThreads;   // 8-value pieces per thread
  const int npr = rb / 8;                    // pieces per row of values
  float yl[IV][8];
#pragma unroll
  for (int it = 0; it < IV; ++it) {
    const int idx = tid + kWyThreads * it;
    const int t = idx / npr, c0 = 8 * (idx % npr);
#pragma unroll
    for (int e = 0; e < 8; ++e) yl[it][e] = 0.0f;
    if (idx < 64 * npr && t < L) wy_load8<F32IN>(a.v, v_base + (long)t * dv + row0 + c0, yl[it]);
  }
  float xv[IT][8], qv[IT][8];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + kWyThreads * it;
    const int t = idx / C8, c0 = 8 * (idx % C8);
    const int g = t - ks;
#pragma unroll
    for (int e = 0; e < 8; ++e) xv[it][e] = qv[it][e] = 0.0f;
    if (idx < 64 * C8 && t < L) {
      if (g >= 0) wy_load8<F32IN>(a.k, qk_base + (long)g * DK + c0, xv[it]);
      else if (a.k_prev) wy_load8<F32IN>(a.k_prev, (long)chain * DK + c0, xv[it]);
      wy_load8<F32IN>(a.q, qk_base + (long)t * DK + c0, qv[it]);
    }
  }
  // start-state row of the lane (fp32 inputs: 4 features per 16-wide K block;
  // bf16 inputs: 8 per 32-wide K step, in three bf16 pieces)
  float4 s0v[F32IN ? DK / 16 : 1];
  float s08[F32IN ? 1 : NKS][8];
  if constexpr (F32IN) {
#pragma unroll
    for (int kq = 0; kq < DK / 16; ++kq)
      s0v[kq] = (solver && has_s0) ? *reinterpret_cast<const float4*>(a.S0 + ((long)chain * dv + col) * DK + 16 * kq + 4 * lg)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s08[kk][e] = 0.0f;
      if (solver && has_s0 && 32 * kk + 8 * lg < DK) {
        const float* sr = a.S0 + ((long)chain * dv + col) * DK + 32 * kk + 8 * lg;
        const float4 u = *reinterpret_cast<const float4*>(sr);
        const float4 w = *reinterpret_cast<const float4*>(sr + 4);
        s08[kk][0] = u.x; s08[kk][1] = u.y; s08[kk][2] = u.z; s08[kk][3] = u.w;
        s08[kk][4] = w.x; s08[kk][5] = w.y; s08[kk][6] = w.z; s08[kk][7] = w.w;
      }
    }
  }
  if (tid < 64) sm.bet[tid] = (a.beta_kind == 1 && tid < L) ? ld_elem(a.beta_t, (long)chain * L + tid, !F32IN) : a.beta;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + kWyThreads * it;
    if (idx < 64 * C8) {
      const int t = idx / C8, c0 = 8 * (idx % C8);
      if constexpr (F32IN) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          *reinterpret_cast<float4*>(&sm.X[t][c0 + 4 * h]) =
              make_float4(xv[it][4 * h], xv[it][4 * h + 1], xv[it][4 * h + 2], xv[it][4 * h + 3]);
          *reinterpret_cast<float4*>(&sm.qy.Q[t][c0 + 4 * h]) =
              make_float4(qv[it][4 * h], qv[it][4 * h + 1], qv[it][4 * h + 2], qv[it][4 * h + 3]);
        }
      } else {
        wy_put8(&sm.X[t][c0], xv[it]);
        wy_put8(&sm.qy.Q[t][c0], qv[it]);
      }
      float n = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) n = __builtin_fmaf(xv[it][e], xv[it][e], n);
      n = group_sum<C8>(n);
      if (idx % C8 == 0) sm.nrm[t] = n;
    }
  }
#pragma unroll
  for (int it = 0; it < IV; ++it) {
    const int idx = tid + kWyThreads * it;
    if (idx < 64 * npr) {
      const int t = idx / npr, c0 = 8 * (idx % npr);
      if constexpr (F32IN) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          *reinterpret_cast<float4*>(&sm.qy.Y[t][c0 + 4 * h]) =
              make_float4(yl[it][4 * h], yl[it][4 * h + 1], yl[it][4 * h + 2], yl[it][4 * h + 3]);
      } else {
        wy_put8(&sm.qy.Y[t][c0], yl[it]);
      }
    }
  }
  if constexpr (DK < KP) {                   // zero the padding of the product depth (bf16)
    for (int t = tid; t < 64; t += kWyThreads)
      for (int c = DK; c < KP; c += 8) {
        *reinterpret_cast<uint4*>(&sm.X[t][c]) = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(&sm.qy.Q[t][c]) = make_uint4(0u, 0u, 0u, 0u);
      }
  }
  __syncthreads();

  // ---- phase 1: every dot product, exact up to fp32 accumulation (these are
  // the sums that may cancel).  Wave 0: per-step scalars (lane = step) and the
  // diagonal Gram tiles; waves 1-3: the Gram and key-query tiles of their
  // operand fragments, kept in registers (tile (kb, b) in the layout of the
  // matrix-core result holds on lane (lg, lr) the values of steps 16 kb + 4 lg + e
  // for row 16 b + lr: the lane's own fragment slots); solver waves: X S0^T and
  // Q S0^T of their value rows
  float yv[4][4];                            // the lane's values, rows 16 b + 4 lg + e
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      yv[b][e] = 0.0f;
      if (solver) {
        if constexpr (F32IN) yv[b][e] = sm.qy.Y[16 * b + 4 * lg + e][16 * wave + lr];
        else yv[b][e] = bf16_to_f32(sm.qy.Y[16 * b + 4 * lg + e][16 * wave + lr]);
      }
    }
  // tile product: rows 16 kb + 4 lg + e of X against rows 16 b + lr of X (or Q)
  auto tile = [&](int kb, int b, bool withq) __attribute__((always_inline)) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    const auto* ar = &sm.X[16 * kb + lr][0];
    const auto* br = withq ? &sm.qy.Q[16 * b + lr][0] : &sm.X[16 * b + lr][0];
    if constexpr (F32IN) {
#pragma unroll
      for (int kq = 0; kq < DK; kq += 16)
        acc = mfma_f32x4(*reinterpret_cast<const float4*>(ar + kq + 4 * lg),
                         *reinterpret_cast<const float4*>(br + kq + 4 * lg), acc);
    } else {
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) acc = mfma16(frag_bf16(ar + 32 * kk + 8 * lg), frag_bf16(br + 32 * kk + 8 * lg), acc);
    }
    return acc;
  };
  // fragment jobs: wave 1 the -A fragments (b, p) = (1,0) (2,0) (3,0) (3,1);
  // wave 2 the W fragments (0,0) (1,0) (2,0), wave 3 (2,1) (3,0) (3,1)
  floatx4 tl[3][2];
#pragma unroll
  for (int fi = 0; fi < 3; ++fi)
#pragma unroll
    for (int h = 0; h < 2; ++h) tl[fi][h] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto frag_bp = [&](int w, int fi, int& f, int& b, int& p) __attribute__((always_inline)) {
    if (w == 1) {
      f = fi;
      b = f == 0 ? 1 : f == 1 ? 2 : 3;
      p = f == 3 ? 1 : 0;
    } else {
      f = 3 * (w - 2) + fi;
      b = f == 0 ? 0 : f == 1 ? 1 : f <= 3 ? 2 : 3;
      p = (f == 3 || f == 5) ? 1 : 0;
    }
  };
  if (wave == 0) {
    const int t = lane;
    float eta = 0.0f, dec = 1.0f;
    if (t < L && !(t == 0 && fresh)) {
      eta = sm.bet[t] / (a.eps + sm.nrm[t]);
      dec = 1.0f - eta * a.lambda;
    }
    float pi = dec;                          // inclusive products within the 16-step block
    pi *= wy_shr<1>(pi, 1.0f);
    pi *= wy_shr<2>(pi, 1.0f);
    pi *= wy_shr<4>(pi, 1.0f);
    pi *= wy_shr<8>(pi, 1.0f);
    float su = dec;                          // inclusive products to the end of the block
    su *= wy_shl<1>(su, 1.0f);
    su *= wy_shl<2>(su, 1.0f);
    su *= wy_shl<4>(su, 1.0f);
    su *= wy_shl<8>(su, 1.0f);
    sm.eta[t] = eta;
    sm.dec[t] = dec;
    sm.pinx[t] = wy_shr<1>(pi, 1.0f);
    sm.pini[t] = pi;
    sm.suf[t] = wy_shl<1>(su, 1.0f);
    float bp[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) bp[b] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pi), 16 * b + 15));
    if (lane == 0) {
      sm.bpre[0] = 1.0f;
#pragma unroll
      for (int b = 0; b < 4; ++b) sm.bpre[b + 1] = sm.bpre[b] * bp[b];
      float s = 1.0f;
#pragma unroll
      for (int b = 3; b >= 0; --b) {
        sm.bsuf[b] = s;
        s *= bp[b];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float m = 1.0f;
#pragma unroll
        for (int b = k + 1; b < 4; ++b) {
          sm.mid[k][b] = m;
          m *= bp[b];
        }
      }
    }
    if constexpr (RG) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const floatx4 g4 = tile(b, b, false);
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.Gd[b][4 * lg + e][lr] = g4[e];
      }
    }
  } else if (RG || wave >= 2) {
    // the -A fragments couple earlier blocks only (kb < b), the W fragments
    // include the diagonal block (kb <= b)
#pragma unroll
    for (int fi = 0; fi < 3; ++fi) {
      int f, b, p;
      frag_bp(wave, fi, f, b, p);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kb = 2 * p + h;
        if (wave == 1 ? kb < b : kb <= b) tl[fi][h] = tile(kb, b, wave != 1);
      }
    }
  }
  floatx4 tl3 = {0.f, 0.f, 0.f, 0.f};        // wave 1's fourth fragment (3,1): G tile (2, 3)
  if (RG && wave == 1) tl3 = tile(2, 3, false);
  floatx4 xs0[4], qs0[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    xs0[b] = floatx4{0.f, 0.f, 0.f, 0.f};
    qs0[b] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  if (solver && has_s0) {
    if constexpr (F32IN) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int kq = 0; kq < DK / 16; ++kq) {
          const int c = 16 * kq + 4 * lg;
          if constexpr (RG) xs0[b] = mfma_f32x4(*reinterpret_cast<const float4*>(&sm.X[16 * b + lr][c]), s0v[kq], xs0[b]);
          qs0[b] = mfma_f32x4(*reinterpret_cast<const float4*>(&sm.qy.Q[16 * b + lr][c]), s0v[kq], qs0[b]);
        }
    } else {
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) {
        const Split3 s3 = wy_split3(s08[kk]);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int c = 32 * kk + 8 * lg;
          const bf16x8 xf = frag_bf16(&sm.X[16 * b + lr][c]);
          const bf16x8 qf = frag_bf16(&sm.qy.Q[16 * b + lr][c]);
#pragma unroll
          for (int k = 2; k >= 0; --k) {     // smallest piece first
            if constexpr (RG) xs0[b] = mfma16(xf, s3.p[k], xs0[b]);
            qs0[b] = mfma16(qf, s3.p[k], qs0[b]);
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- phase 2: diagonal blocks of T (wave 0: 16-lane row b = block b, lane n
  // = column n); the -A and W operand fragments (waves 1-3) from the tiles in
  // registers.  Fragment (b, pair p): row t = 16 b + lr, slots 0-3 the steps
  // 32 p + 4 lg + 0..3, slots 4-7 the steps 32 p + 16 + 4 lg + 0..3 (zero where
  // the block is not coupled)
  if (wave == 0) {
    if constexpr (RG) {
      const int b = lg, n = lr, s = 16 * b + n;
      const float es = sm.eta[s];
      float gv[16], dq[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 g4 = *reinterpret_cast<const float4*>(&sm.Gd[b][n][4 * q4]);   // G[s][16 b + r] (G symmetric)
        const float4 d4 = *reinterpret_cast<const float4*>(&sm.dec[16 * b + 4 * q4]);
        gv[4 * q4] = g4.x; gv[4 * q4 + 1] = g4.y; gv[4 * q4 + 2] = g4.z; gv[4 * q4 + 3] = g4.w;
        dq[4 * q4] = d4.x; dq[4 * q4 + 1] = d4.y; dq[4 * q4 + 2] = d4.z; dq[4 * q4 + 3] = d4.w;
      }
      float colv[16], run = 1.0f;            // A[16 b + r][s] = eta_s D[16 b + r - 1][s]
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        colv[r] = 0.0f;
        if (r > n) {
          colv[r] = es * run * gv[r];
          run *= dq[r];
        }
      }
      wave_sync();                           // every lane has read Gd before Acol overwrites it
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4*>(&sm.Acol[b][n][4 * q4]) =
            make_float4(colv[4 * q4], colv[4 * q4 + 1], colv[4 * q4 + 2], colv[4 * q4 + 3]);
      wave_sync();
      float g[16], x[16], acc[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 g4 = *reinterpret_cast<const float4*>(&sm.Acol[b][n][4 * q4]);
        g[4 * q4] = g4.x; g[4 * q4 + 1] = g4.y; g[4 * q4 + 2] = g4.z; g[4 * q4 + 3] = g4.w;
      }
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        x[m] = m == n ? 1.0f : 0.0f;
        acc[m] = 0.0f;
      }
      wave_sync();                           // every lane has read Acol before TS overwrites it
      wy_sweep<0>(x, acc, g);
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.TS[b][r][n] = x[r];
    }
  } else if (RG || wave >= 2) {
    const int nf = wave == 1 ? 4 : 3;
#pragma unroll
    for (int fi = 0; fi < 4; ++fi) {
      if (fi >= nf) break;
      int f, b, p;
      frag_bp(wave, fi, f, b, p);
      const int t = 16 * b + lr;
      float v[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kb = 2 * p + h;
        const floatx4 tv = fi == 3 ? (h == 0 ? tl3 : floatx4{0.f, 0.f, 0.f, 0.f}) : tl[fi][h];
        if (wave == 1) {                     // -A[t][s] = -eta_s D[t-1][s] G[t][s], blocks kb < b
          if (kb < b) {
            const float sc = -sm.pinx[t] * sm.mid[kb][b];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int s = 16 * kb + 4 * lg + e;
              v[4 * h + e] = sc * sm.eta[s] * sm.suf[s] * tv[e];
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * h + e] = 0.0f;
          }
        } else {                             // W[t][s] = eta_s D[t][s] P[t][s], s <= t
          if (kb < b) {
            const float sc = sm.pini[t] * sm.mid[kb][b];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int s = 16 * kb + 4 * lg + e;
              v[4 * h + e] = sc * sm.eta[s] * sm.suf[s] * tv[e];
            }
          } else if (kb == b) {
            // D[t][s] = prod_{s<q<=t} a_q for the four steps s = 16 b + 4 lg + e <= t
            float dq[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const float4 d4 = *reinterpret_cast<const float4*>(&sm.dec[16 * b + 4 * q4]);
              dq[4 * q4] = d4.x; dq[4 * q4 + 1] = d4.y; dq[4 * q4 + 2] = d4.z; dq[4 * q4 + 3] = d4.w;
            }
            float dd = 1.0f;                 // D[t][16 b + 4 lg + 3]
#pragma unroll
            for (int q = 0; q < 16; ++q)
              if (q > 4 * lg + 3 && q <= lr) dd *= dq[q];
            // D[t][s] = D[t][s+1] a_{s+1} while s + 1 <= t; D[t][t] = 1
            float dcur[4];
            dcur[3] = dd;
#pragma unroll
            for (int e = 2; e >= 0; --e) dcur[e] = 4 * lg + e + 1 <= lr ? dcur[e + 1] * dq[4 * lg + e + 1] : 1.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int sl = 4 * lg + e;
              v[4 * h + e] = sl <= lr ? sm.eta[16 * b + sl] * dcur[e] * tv[e] : 0.0f;
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * h + e] = 0.0f;
          }
        }
      }
      const int fc = wy_frag_col(lr, lg);
      uint16_t* fh = wave == 1 ? &sm.f.Ah[f][lr][fc] : &sm.f.Wh[f][lr][fc];
      uint16_t* fl = wave == 1 ? &sm.f.Al[f][lr][fc] : &sm.f.Wl[f][lr][fc];
      const HL hv = hl_vals(v);             // one 16-byte store per piece
      *reinterpret_cast<bf16x8*>(fh) = hv.hi;
      *reinterpret_cast<bf16x8*>(fl) = hv.lo;
    }
  }
  __syncthreads();

  // ---- phase 3: solve, readout and final state of the wave's 16 value rows
  if (!solver) return;
  const floatx4 zacc = {0.f, 0.f, 0.f, 0.f};
  const float z4[4] = {0.f, 0.f, 0.f, 0.f};
  floatx4 E[4];
  HL Eop[2];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    floatx4 acc;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * b + 4 * lg + e;
      acc[e] = yv[b][e];
      if (RG && has_s0) acc[e] = __builtin_fmaf(-sm.bpre[b] * sm.pinx[t], xs0[b][e], acc[e]);
    }
    if constexpr (RG) {
#pragma unroll
      for (int p = 0; 2 * p < b; ++p) {
        const int f = b == 1 ? 0 : b == 2 ? 1 : (p == 0 ? 2 : 3);
        acc = wy_mma3(acc, hl_pair(&sm.f.Ah[f][lr][wy_frag_col(lr, lg)], &sm.f.Al[f][lr][wy_frag_col(lr, lg)]), Eop[p]);
      }
      const float4 t4 = *reinterpret_cast<const float4*>(&sm.TS[b][lr][4 * lg]);
      const float tv[4] = {t4.x, t4.y, t4.z, t4.w};
      const float av[4] = {acc[0], acc[1], acc[2], acc[3]};
      E[b] = wy_mma3(zacc, wy_hl(tv, z4), wy_hl(av, z4));
    } else {
      E[b] = acc;
    }
    if (b & 1) {
      const float lo4[4] = {E[b - 1][0], E[b - 1][1], E[b - 1][2], E[b - 1][3]};
      const float hi4[4] = {E[b][0], E[b][1], E[b][2], E[b][3]};
      Eop[b >> 1] = wy_hl(lo4, hi4);
    } else {
      const float lo4[4] = {E[b][0], E[b][1], E[b][2], E[b][3]};
      Eop[b >> 1] = wy_hl(lo4, z4);
    }
  }
  // o_t = d_t (Q S0^T)_t + (W E)_t
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    floatx4 o = zacc;
    if (has_s0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = sm.bpre[b] * sm.pini[16 * b + 4 * lg + e] * qs0[b][e];
    }
#pragma unroll
    for (int p = 0; 2 * p <= b; ++p) {
      const int f = b == 0 ? 0 : b == 1 ? 1 : b == 2 ? 2 + p : 4 + p;
      o = wy_mma3(o, hl_pair(&sm.f.Wh[f][lr][wy_frag_col(lr, lg)], &sm.f.Wl[f][lr][wy_frag_col(lr, lg)]), Eop[p]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * b + 4 * lg + e;
      if (t < L) a.o[v_base + (long)t * dv + col] = o[e];
    }
  }
  if (a.S_out == nullptr) return;
  // S_L^T tile (16 features x 16 value rows) = d_63 S0^T + X^T diag(c) E,
  // c_s = eta_s D[63][s] = eta_s suf_s (products of the later blocks); the
  // operand X^T is read column-wise from the row-major samples
  HL ec[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    float v[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int b = 2 * p + h;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = 16 * b + 4 * lg + e;
        v[4 * h + e] = E[b][e] * (sm.eta[s] * sm.suf[s] * sm.bsuf[b]);
      }
    }
    ec[p] = hl_vals(v);
  }
  const float dL = sm.bpre[4];
  float* srow = a.S_out + ((long)chain * dv + col) * DK;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    floatx4 acc = zacc;
    if (has_s0) {
      const float4 s4 = *reinterpret_cast<const float4*>(a.S0 + ((long)chain * dv + col) * DK + 16 * ct + 4 * lg);
      acc = floatx4{dL * s4.x, dL * s4.y, dL * s4.z, dL * s4.w};
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int c = 16 * ct + lr;
      if constexpr (F32IN) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = sm.X[32 * p + 16 * (j >> 2) + 4 * lg + (j & 3)][c];
        acc = wy_mma3(acc, hl_vals(v), ec[p]);
      } else {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int s0 = 32 * p + 16 * (j >> 1) + 4 * lg + 2 * (j & 1);
          w[j] = (uint32_t)sm.X[s0][c] | ((uint32_t)sm.X[s0 + 1][c] << 16);
        }
        acc = wy_mma2(acc, __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3])), ec[p]);
      }
    }
    *reinterpret_cast<float4*>(srow + 16 * ct + 4 * lg) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
}

template <int DK, bool F32IN, bool HS0>
hipError_t launch_wy_s0(const SeqArgs& a, hipStream_t stream) {
  const int rb = a.dv < kMaskedMaxRows ? a.dv : kMaskedMaxRows;
  const dim3 grid((unsigned)(a.batch * a.heads), (unsigned)(a.dv / rb));
  if (a.regression)
    hipLaunchKernelGGL((masked_wy_kernel<DK, true, F32IN, HS0>), grid, dim3(kWyThreads), 0, stream, a, rb);
  else
    hipLaunchKernelGGL((masked_wy_kernel<DK, false, F32IN, HS0>), grid, dim3(kWyThreads), 0, stream, a, rb);
  return hipGetLastError();
}

template <int DK, bool F32IN>
hipError_t launch_wy_dt(const SeqArgs& a, hipStream_t stream) {
  return a.S0 ? launch_wy_s0<DK, F32IN, true>(a, stream) : launch_wy_s0<DK, F32IN, false>(a, stream);
}

template <int DK>
hipError_t launch_wy(const SeqArgs& a, hipStream_t stream) {
  return a.dtype == 0 ? launch_wy_dt<DK, false>(a, stream) : launch_wy_dt<DK, true>(a, stream);
}

template <int DKM, int BW>
hipError_t launch_bw(const SeqArgs& a, hipStream_t stream) {
  const int rb = a.dv < kMaskedMaxRows ? a.dv : kMaskedMaxRows;
  const dim3 grid((unsigned)(a.batch * a.heads), (unsigned)(a.dv / rb));
  if (a.regression)
    hipLaunchKernelGGL((masked_kernel<DKM, BW, true>), grid, dim3(rb * 16), 0, stream, a, rb);
  else
    hipLaunchKernelGGL((masked_kernel<DKM, BW, false>), grid, dim3(rb * 16), 0, stream, a, rb);
  return hipGetLastError();
}

template <int DKM>
hipError_t launch_dkm(const SeqArgs& a, hipStream_t stream) {
  switch (a.window) {
    case 1: return launch_bw<DKM, 1>(a, stream);
    case 2: return launch_bw<DKM, 2>(a, stream);
    case 3: return launch_bw<DKM, 3>(a, stream);
    case 4: return launch_bw<DKM, 4>(a, stream);
    case 5: return launch_bw<DKM, 5>(a, stream);
    case 6: return launch_bw<DKM, 6>(a, stream);
    case 7: return launch_bw<DKM, 7>(a, stream);
    case 8: return launch_bw<DKM, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_masked(const SeqArgs& a, hipStream_t stream) {
  (void)hipGetLastError();
  if (a.seqlen < 1 || a.seqlen > kMaskedMaxL || a.window < 1 || a.window > 8) return hipErrorInvalidValue;
  if (a.window == 1 && a.beta_kind != 2) {   // one system shared by every value row
    switch (a.dk) {
      case 16: return launch_wy<16>(a, stream);
      case 32: return launch_wy<32>(a, stream);
      case 64: return launch_wy<64>(a, stream);
      case 128: return launch_wy<128>(a, stream);
    }
    return hipErrorInvalidValue;
  }
  if (a.dk <= 64) return launch_dkm<64>(a, stream);
  return launch_dkm<128>(a, stream);
}

}  // namespace falcon
