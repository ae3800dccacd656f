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
  if (a.dk <= 64) return launch_dkm<64>(a, stream);
  return launch_dkm<128>(a, stream);
}

}  // namespace falcon
