// falcon_chunk_wy.hip - chunk-parallel Falcon forward for window 1 with gains
// shared by the value rows (Falcon-1, Falcon-1A; scalar or per-token beta).
//
// Method: explainer of arXiv 2608.27763, section 核心方法 §3 (chunk-parallel
// form) and the 163.com article, section 02 (2) (only the fixed-size state
// crosses chunks; Gram / WY representation with a triangular solve).  With
// window 1 the unknowns z_t of a chunk (t = 0..C-1, per value row) satisfy
//   z_t / zeta_t + g_{t-1} sum_{s<t} (x_t . x_s) z_s = y_t - g_{t-1} S0 x_t
// (g_t = prod_{r<=t} a_r, zeta_t = eta_t / g_t).  Dividing by g_{t-1} and
// scaling by omega_t = zeta_t g_{t-1} (= eta_t / a_t):
//   (I + M) z = diag(omega) (y / g_{t-1} - S0 x),   M = diag(omega) L,
// L the strictly lower Gram matrix.  (I + M) is unit lower triangular and the
// same for every value row, so with W = (I + M)^-1 R, R_t = [omega_t x_t | zeta_t y_t],
//   z = Ut - S0 Wt,   Wt^T = W[:, keys],  Ut^T = W[:, values]
//   o_t = g_t (S0 q_t + sum_{s<=t} (q_t . x_s) z_s),   S_C = g_{C-1} (S0 + sum_s z_s x_s^T)
// W is formed by a blocked forward solve over 16-step blocks:
//   W_0 = T_00 R_0,   W_1 = [T_11 | -T_11 M_10] [R_1 ; W_0],   T_bb = (I + M_bb)^-1
// The inner-product family has z_t = zeta_t y_t (no solve).
//
// Structure.  One workgroup = 8 wave64 = one (batch*head) chain x 32 value
// rows; chunks of C = 32 steps.  Waves 0 and 1 ("state waves") each own 16 rows
// of the state: S (fp32) and z never leave their registers; per chunk they run
// S q, z = Ut - Wt S, the carry S <- g (S + Z X^T) and the readout, four small
// matrix-core products.  Waves 2..7 prepare later chunks, each stage reading
// only what an earlier iteration wrote, so one barrier per chunk suffices:
//   iteration c:  state chunk c | solve and q.x of c+1 | keys transposed,
//                 scalars and [T_00], [T_11 | -T_11 M_10] of c+2 | Gram of c+3 |
//                 keys of c+4, queries and values of c+2 to LDS (loaded one
//                 iteration earlier)
// LDS operands that meet a register operand of the state waves are stored in
// the order of that register fragment: within every 32-wide group, positions
// 8g..8g+3 hold indices 4g..4g+3 and 8g+4..8g+7 hold 16+4g..16+4g+3, so every
// fragment is one 16-byte read.  Row strides are 32 mod 64 bytes, which keeps
// the 16-byte reads of a fragment (16 rows) on distinct banks.
// Non-exact operands are split into bf16 hi + lo (split-bf16, Henry, Tang &
// Heinecke, ARITH 2019): hi*hi + hi*lo + lo*hi with fp32 accumulation.
#include <type_traits>

#include "falcon_device.h"
#include "falcon_launch.h"
#include "falcon_mma.h"

namespace falcon {
namespace {

constexpr int CS = 32;       // chunk length
constexpr int RW = 32;       // value rows per workgroup
constexpr int NW = 8;
constexpr int NT = 64 * NW;
constexpr int NPRE = NT - 128;   // threads of the preparation waves

// position of index k in the fragment order (groups of 32)
__device__ __forceinline__ int fpos(int k) {
  const int kk = k & 31;
  return (k & ~31) + 8 * ((kk & 15) >> 2) + ((kk >> 4) << 2) + (kk & 3);
}

template <int DK>
struct WyLds {
  static constexpr int XR = DK + 16;     // bf16 row: DK (fragment order) + pad
  static constexpr int TR = CS + 16;     // bf16 row over steps
  uint16_t X[4][CS][XR];                 // keys by chunk & 3, k in fragment order
  uint16_t Q[4][CS][XR];                 // queries by chunk & 3
  uint16_t XT[4][DK][TR];                // keys transposed, t in fragment order
  uint16_t YT[2][RW][TR];                // values transposed, t natural
  uint16_t Phi[2][CS][TR];               // q.x (s <= t), s in fragment order
  uint16_t Plo[2][CS][TR];
  uint16_t Whi[2][CS][XR];               // Wt^T[t][k], k in fragment order
  uint16_t Wlo[2][CS][XR];
  uint16_t SAhi[2][2][16][TR];           // [T_00 | 0], [T_11 | -T_11 M_10], fragment order
  uint16_t SAlo[2][2][16][TR];
  float G[2][CS][CS + 8];                // Gram (whole 32 x 32)
  float Ut[2][RW][CS + 8];               // Ut[i][t]
  float beta[4][CS];                     // gains by chunk & 3
  alignas(16) float gam[4][CS];
  alignas(16) float gm1[4][CS];
  alignas(16) float zeta[4][CS];
  alignas(16) float omega[4][CS];
};

struct WyGeom {
  int nrbg;
  int remap;
  int nchunks;
};

// the three passes accumulate independently (no MFMA waits on the previous one)
__device__ __forceinline__ floatx4 mma3(floatx4 acc, const HL& a, const HL& b) {
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  const floatx4 c1 = mfma16(a.hi, b.lo, z);
  const floatx4 c2 = mfma16(a.lo, b.hi, z);
  acc = mfma16(a.hi, b.hi, acc);
  return acc + (c1 + c2);
}
__device__ __forceinline__ floatx4 mma2(floatx4 acc, const bf16x8& a, const HL& b) {
  acc = mfma16(a, b.hi, acc);
  return mfma16(a, b.lo, acc);
}
__device__ __forceinline__ floatx4 mma2(floatx4 acc, const HL& a, const bf16x8& b) {
  acc = mfma16(a.hi, b, acc);
  return mfma16(a.lo, b, acc);
}
// v of lane - N within the same 16-lane row (DPP row_shr); lanes 0..N-1 of a
// row, whose source lies outside it, return `fill`
template <int N>
__device__ __forceinline__ float dpp_shr(float v, float fill) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill), __builtin_bit_cast(int, v),
                                                             0x110 + N, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_value(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}
// a split fragment from two groups of 4 fp32 (slots 0-3, 4-7)
__device__ __forceinline__ HL hl_two(const float* a, const float* b) {
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return hl_vals(v);
}

template <int DK, bool REG>
__global__ __launch_bounds__(NT) void chunk_wy_kernel(SeqArgs a, WyGeom geo) {
  using SM = WyLds<DK>;
  constexpr int NKT = DK / 16, NKS = DK / 32, VPR = DK / 8;
  constexpr int KV = (CS * VPR + NPRE - 1) / NPRE;    // uint4 of k (or q) per prep thread
  constexpr int YV = (CS * (RW / 8) + NPRE - 1) / NPRE;
  static_assert(DK % 32 == 0 && DK <= 64, "dk in {32, 64}");
  __shared__ __align__(16) SM sm;

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(a.v);
  const uint16_t* __restrict__ kpg = static_cast<const uint16_t*>(a.k_prev);
  const uint16_t* __restrict__ bg = static_cast<const uint16_t*>(a.beta_t);

  int chain, rbg;
  {
    const int b = blockIdx.x;
    if (geo.remap) {   // the row groups of one chain share an XCD (and its L2)
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
  const int nrb = (dv - i0) >= RW ? 2 : 1;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int ptid = tid - 128;             // preparation-thread index (waves 2..7)
  const long L = a.seqlen;
  const long qk_base = (long)chain * L * DK;
  const long v_base = (long)chain * L * dv;
  const int nchunks = geo.nchunks;
  auto steps = [&](int j) __attribute__((always_inline)) {
    const long t0 = (long)j * CS;
    return (int)((L - t0) < CS ? (L - t0) : CS);
  };

  // ---------------- zero the fragment slots no stage writes ----------------
  for (int idx = tid; idx < 2 * 2 * 16 * SM::TR; idx += NT) {
    (&sm.SAhi[0][0][0][0])[idx] = 0;
    (&sm.SAlo[0][0][0][0])[idx] = 0;
  }
  for (int idx = tid; idx < 2 * CS * SM::TR; idx += NT) {
    (&sm.Phi[0][0][0])[idx] = 0;
    (&sm.Plo[0][0][0])[idx] = 0;
  }

  // ---------------- global loads, issued one iteration before their commit ----------------
  uint4 pk[KV], pq[KV], py[YV];
  uint32_t pbt = 0;
  auto prefetch_k = [&](int j) __attribute__((always_inline)) {   // keys (and beta) of chunk j
    const long t0 = (long)j * CS;
    const int c = steps(j);
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int idx = ptid + v * NPRE;
      const int t = idx / VPR, kv = idx % VPR;
      uint4 kval = {0u, 0u, 0u, 0u};
      if (idx < CS * VPR && t < c) {
        const long g = t0 + t;   // key x_g = k_{g-1}; x_0 = k_prev or 0
        if (g >= 1) kval = *reinterpret_cast<const uint4*>(kg + qk_base + (g - 1) * DK + kv * 8);
        else if (kpg) kval = *reinterpret_cast<const uint4*>(kpg + (long)chain * DK + kv * 8);
      }
      pk[v] = kval;
    }
    pbt = 0;
    if (a.beta_kind == 1 && ptid < c) pbt = (uint32_t)bg[(long)chain * L + t0 + ptid];
  };
  auto prefetch_qv = [&](int j) __attribute__((always_inline)) {  // queries and values of chunk j
    const long t0 = (long)j * CS;
    const int c = steps(j);
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int idx = ptid + v * NPRE;
      const int t = idx / VPR, kv = idx % VPR;
      uint4 qval = {0u, 0u, 0u, 0u};
      if (idx < CS * VPR && t < c) qval = *reinterpret_cast<const uint4*>(qg + qk_base + (t0 + t) * DK + kv * 8);
      pq[v] = qval;
    }
#pragma unroll
    for (int v = 0; v < YV; ++v) {
      const int idx = ptid + v * NPRE;
      const int t = idx / (RW / 8), h = idx % (RW / 8);
      uint4 val = {0u, 0u, 0u, 0u};
      if (idx < CS * (RW / 8) && t < c && i0 + h * 8 < dv)
        val = *reinterpret_cast<const uint4*>(vg + v_base + (t0 + t) * dv + i0 + h * 8);
      py[v] = val;
    }
  };
  // 8 consecutive k (k0 % 8 == 0) -> two 4-groups at their fragment positions
  auto put8 = [&](uint16_t* row, int k0, uint4 val) __attribute__((always_inline)) {
    *reinterpret_cast<uint2*>(row + fpos(k0)) = make_uint2(val.x, val.y);
    *reinterpret_cast<uint2*>(row + fpos(k0 + 4)) = make_uint2(val.z, val.w);
  };
  auto commit_k = [&](int j) __attribute__((always_inline)) {
    const int xb = j & 3, nb = j & 3;
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int idx = ptid + v * NPRE;
      if (idx < CS * VPR) {
        const int t = idx / VPR, kv = idx % VPR;
        put8(&sm.X[xb][t][0], kv * 8, pk[v]);
      }
    }
    if (ptid < CS) sm.beta[nb][ptid] = a.beta_kind == 0 ? a.beta : bf16_to_f32((uint16_t)pbt);
  };
  auto commit_qv = [&](int j) __attribute__((always_inline)) {
    const int qb = j & 3, yb = j & 1;
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int idx = ptid + v * NPRE;
      if (idx < CS * VPR) {
        const int t = idx / VPR, kv = idx % VPR;
        put8(&sm.Q[qb][t][0], kv * 8, pq[v]);
      }
    }
#pragma unroll
    for (int v = 0; v < YV; ++v) {
      const int idx = ptid + v * NPRE;
      if (idx < CS * (RW / 8)) {
        const int t = idx / (RW / 8), h = idx % (RW / 8);
        const uint4 val = py[v];
        const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sm.YT[yb][h * 8 + 2 * e][t] = (uint16_t)(w4[e] & 0xFFFFu);
          sm.YT[yb][h * 8 + 2 * e + 1][t] = (uint16_t)(w4[e] >> 16);
        }
      }
    }
  };

  // eta_t = beta_t / (eps + ||x_t||^2), a_t = 1 - eta_t lambda; padded steps and
  // the fresh-sequence first step (x_1 = 0 on S_0 = 0) take eta = 0, a = 1.
  // One wave; lane = step; prefix product by a wave scan.
  // ||x_t||^2 is the Gram diagonal (regression) or summed from the key row.
  auto scalars = [&](int j) __attribute__((always_inline)) {
    const int sb = j & 3;
    const long t0 = (long)j * CS;
    const int c = steps(j);
    const int t = lane;
    const bool live = t < c && !(t0 + t == 0 && kpg == nullptr);
    const int tr = t < CS ? t : 0;
    float nrm;
    if constexpr (REG) {
      nrm = sm.G[j & 1][tr][tr];
    } else {
      nrm = 0.0f;
      uint4 xr[DK / 8];
#pragma unroll
      for (int k8 = 0; k8 < DK; k8 += 8) xr[k8 / 8] = *reinterpret_cast<const uint4*>(&sm.X[j & 3][tr][k8]);
#pragma unroll
      for (int k8 = 0; k8 < DK; k8 += 8) {
        const uint4 w = xr[k8 / 8];
        const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(w4[e] << 16);
          const float hi = __uint_as_float(w4[e] & 0xFFFF0000u);
          nrm += lo * lo + hi * hi;
        }
      }
    }
    float eta = 0.0f, dec = 1.0f;
    if (live) {
      eta = sm.beta[sb][t] / (a.eps + nrm);
      dec = 1.0f - eta * a.lambda;
    }
    // inclusive prefix product over the 32 steps: within rows of 16 lanes by
    // DPP row shifts (lanes shifted in from outside the row read 1), then the
    // second row times the first row's total
    float gsc = dec;
    gsc *= dpp_shr<1>(gsc, 1.0f);
    gsc *= dpp_shr<2>(gsc, 1.0f);
    gsc *= dpp_shr<4>(gsc, 1.0f);
    gsc *= dpp_shr<8>(gsc, 1.0f);
    const float row0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gsc), 15));
    if (lane >= 16) gsc *= row0;
    const float gprev = dpp_shr<1>(gsc, lane == 16 ? row0 : 1.0f);
    if (t < CS) {
      const float z = eta / gsc;
      sm.gam[sb][t] = gsc;
      sm.gm1[sb][t] = gprev;
      sm.zeta[sb][t] = z;
      sm.omega[sb][t] = z * gprev;
    }
  };

  // Gram tile (ti, tj) of chunk j: G[t][s] = x_t . x_s (lane: 4 consecutive s of one t)
  auto gram_tile = [&](int j, int ti, int tj) __attribute__((always_inline)) {
    const int xb = j & 3;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 fa = frag_bf16(&sm.X[xb][16 * tj + lr][32 * ks + 8 * lg]);
      const bf16x8 fb = frag_bf16(&sm.X[xb][16 * ti + lr][32 * ks + 8 * lg]);
      if (ks & 1) acc2 = mfma16(fa, fb, acc2);
      else acc = mfma16(fa, fb, acc);
    }
    acc += acc2;
    *reinterpret_cast<float4*>(&sm.G[j & 1][16 * ti + lr][16 * tj + 4 * lg]) =
        make_float4(acc[0], acc[1], acc[2], acc[3]);
  };
  // q.x tile (ti >= tj) of chunk j: P[t][s] = q_t . x_s for s <= t, split, s in fragment order
  auto qx_tile = [&](int j, int ti, int tj) __attribute__((always_inline)) {
    const int xb = j & 3;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 fa = frag_bf16(&sm.X[xb][16 * tj + lr][32 * ks + 8 * lg]);
      const bf16x8 fb = frag_bf16(&sm.Q[xb][16 * ti + lr][32 * ks + 8 * lg]);
      if (ks & 1) acc2 = mfma16(fa, fb, acc2);
      else acc = mfma16(fa, fb, acc);
    }
    acc += acc2;
    const int t = 16 * ti + lr;
    float pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] = (16 * tj + 4 * lg + e <= t) ? acc[e] : 0.0f;
    const int p = 8 * lg + 4 * tj;
    store_split4(&sm.Phi[j & 1][t][p], &sm.Plo[j & 1][t][p], pv);
  };
  // keys transposed: XT[k][t] from X[t][k]; a thread moves a 4 (t) x 4 (k) block
  auto transpose_keys = [&](int j) __attribute__((always_inline)) {
    const int xb = j & 3;
    for (int idx = ptid; idx < (CS / 4) * (DK / 4); idx += NPRE) {
      const int t4 = 4 * (idx % (CS / 4)), k4 = 4 * (idx / (CS / 4));
      const int pk4 = fpos(k4);
      uint2 rw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) rw[e] = *reinterpret_cast<const uint2*>(&sm.X[xb][t4 + e][pk4]);
      const int pt4 = fpos(t4);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = (kk < 2) ? rw[e].x : rw[e].y;
          h[e] = (kk & 1) ? (w >> 16) : (w & 0xFFFFu);
        }
        *reinterpret_cast<uint2*>(&sm.XT[xb][k4 + kk][pt4]) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      }
    }
  };
  // [T_00 | 0] and [T_11 | -T_11 M_10] of chunk j by forward substitution, one
  // wave: lanes 0..15 the columns of T_00, lanes 16..47 the 32 columns of block 1.
  // Every Gram entry the sweep uses is read before it starts (one wait).
  auto solve_factors = [&](int j) __attribute__((always_inline)) {
    const int gb = j & 1, sb = j & 3;
    const int blk = lane < 16 ? 0 : 1;
    const int col = lane < 16 ? lane : (lane < 48 ? lane - 16 : 0);   // 0..15 / 0..31
    const int u0 = 16 * blk;
    float rhs[16], acc[16];               // rhs becomes the solution in place
    float4 gr[16][4];
#pragma unroll
    for (int m = 0; m < 16; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (4 * q + 3 > m) gr[m][q] = *reinterpret_cast<const float4*>(&sm.G[gb][u0 + m][u0 + 4 * q]);
    float om[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 o4 = *reinterpret_cast<const float4*>(&sm.omega[sb][u0 + 4 * q]);
      om[4 * q] = o4.x; om[4 * q + 1] = o4.y; om[4 * q + 2] = o4.z; om[4 * q + 3] = o4.w;
    }
    if (blk == 1 && col >= 16) {
      // -M_10[:, c'] = -omega_{16+m} G[16+m][c'] = -omega_{16+m} G[c'][16+m]
      const int cp = col - 16;
#pragma unroll
      for (int m = 0; m < 16; m += 4) {
        const float4 gv = *reinterpret_cast<const float4*>(&sm.G[gb][cp][16 + m]);
        rhs[m] = -om[m] * gv.x;
        rhs[m + 1] = -om[m + 1] * gv.y;
        rhs[m + 2] = -om[m + 2] * gv.z;
        rhs[m + 3] = -om[m + 3] * gv.w;
      }
    } else {
#pragma unroll
      for (int m = 0; m < 16; ++m) rhs[m] = (m == col) ? 1.0f : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      rhs[m] -= om[m] * acc[m];
#pragma unroll
      for (int r = m + 1; r < 16; ++r) {   // column m below m: G[u0+r][u0+m] = G[u0+m][u0+r]
        const float4 g4 = gr[m][r >> 2];
        const float gv = (r & 3) == 0 ? g4.x : (r & 3) == 1 ? g4.y : (r & 3) == 2 ? g4.z : g4.w;
        acc[r] += gv * rhs[m];
      }
    }
    if (lane < 48) {
      const int cc = col & 15;
      const int p = 8 * (cc >> 2) + ((col >> 4) << 2) + (cc & 3);
#pragma unroll
      for (int m = 0; m < 16; ++m) split1(rhs[m], sm.SAhi[gb][blk][m][p], sm.SAlo[gb][blk][m][p]);
    }
  };
  // Blocked solve of chunk j for one 16-column tile of R = [omega x | zeta y]:
  // keys: columns 16 tile.. of the keys (-> Wt^T); else value rows 16 tile.. (-> Ut).
  // Results: lane holds t = 4 lg + e (block 0) and 16 + 4 lg + e (block 1), column lr.
  auto solve_tile = [&](int j, bool keys, int tile) __attribute__((always_inline)) {
    const int gb = j & 1, sb = j & 3, xb = j & 3;
    float r0[4], r1[4];
    {
      const float4 s0 = *reinterpret_cast<const float4*>(keys ? &sm.omega[sb][4 * lg] : &sm.zeta[sb][4 * lg]);
      const float4 s1 = *reinterpret_cast<const float4*>(keys ? &sm.omega[sb][16 + 4 * lg] : &sm.zeta[sb][16 + 4 * lg]);
      uint2 x0, x1;
      if (keys) {   // XT positions 8 lg.. hold t = 4 lg.., 8 lg + 4.. hold t = 16 + 4 lg..
        x0 = *reinterpret_cast<const uint2*>(&sm.XT[xb][16 * tile + lr][8 * lg]);
        x1 = *reinterpret_cast<const uint2*>(&sm.XT[xb][16 * tile + lr][8 * lg + 4]);
      } else {
        x0 = *reinterpret_cast<const uint2*>(&sm.YT[gb][16 * tile + lr][4 * lg]);
        x1 = *reinterpret_cast<const uint2*>(&sm.YT[gb][16 * tile + lr][16 + 4 * lg]);
      }
      r0[0] = s0.x * __uint_as_float(x0.x << 16);
      r0[1] = s0.y * __uint_as_float(x0.x & 0xFFFF0000u);
      r0[2] = s0.z * __uint_as_float(x0.y << 16);
      r0[3] = s0.w * __uint_as_float(x0.y & 0xFFFF0000u);
      r1[0] = s1.x * __uint_as_float(x1.x << 16);
      r1[1] = s1.y * __uint_as_float(x1.x & 0xFFFF0000u);
      r1[2] = s1.z * __uint_as_float(x1.y << 16);
      r1[3] = s1.w * __uint_as_float(x1.y & 0xFFFF0000u);
    }
    const float zero4[4] = {0.f, 0.f, 0.f, 0.f};
    const HL a0 = hl_pair(&sm.SAhi[gb][0][lr][8 * lg], &sm.SAlo[gb][0][lr][8 * lg]);
    const HL a1 = hl_pair(&sm.SAhi[gb][1][lr][8 * lg], &sm.SAlo[gb][1][lr][8 * lg]);
    const floatx4 zacc = {0.f, 0.f, 0.f, 0.f};
    const HL b0 = hl_two(r0, zero4);
    const floatx4 w0 = mma3(zacc, a0, b0);
    const float w0v[4] = {w0[0], w0[1], w0[2], w0[3]};
    const HL b1 = hl_two(r1, w0v);
    if (keys) {
      // Wt^T rows are written with 8-byte stores: the same products with the
      // operands swapped give the transposed tiles (lane: 4 consecutive k of one t)
      const floatx4 v0 = mma3(zacc, b0, a0);
      const floatx4 v1 = mma3(zacc, b1, a1);
      const int p = fpos(16 * tile + 4 * lg);
      const float f0[4] = {v0[0], v0[1], v0[2], v0[3]};
      const float f1[4] = {v1[0], v1[1], v1[2], v1[3]};
      store_split4(&sm.Whi[gb][lr][p], &sm.Wlo[gb][lr][p], f0);
      store_split4(&sm.Whi[gb][16 + lr][p], &sm.Wlo[gb][16 + lr][p], f1);
    } else {
      const floatx4 w1 = mma3(zacc, a1, b1);
      float* u = &sm.Ut[gb][16 * tile + lr][0];
      *reinterpret_cast<float4*>(u + 4 * lg) = make_float4(w0[0], w0[1], w0[2], w0[3]);
      *reinterpret_cast<float4*>(u + 16 + 4 * lg) = make_float4(w1[0], w1[1], w1[2], w1[3]);
    }
  };
  // inner-product family: z_t = zeta_t y_t, kept where the regression keeps Ut
  auto zeta_y = [&](int j) __attribute__((always_inline)) {
    const int gb = j & 1, sb = j & 3;
    for (int idx = ptid; idx < RW * (CS / 4); idx += NPRE) {
      const int i = idx / (CS / 4), t4 = 4 * (idx % (CS / 4));
      const uint2 yb = *reinterpret_cast<const uint2*>(&sm.YT[gb][i][t4]);
      const float4 z = *reinterpret_cast<const float4*>(&sm.zeta[sb][t4]);
      *reinterpret_cast<float4*>(&sm.Ut[gb][i][t4]) =
          make_float4(z.x * __uint_as_float(yb.x << 16), z.y * __uint_as_float(yb.x & 0xFFFF0000u),
                      z.z * __uint_as_float(yb.y << 16), z.w * __uint_as_float(yb.y & 0xFFFF0000u));
    }
  };

  // The state waves and the preparation waves run separate loops with the same
  // barrier count (one per iteration), so neither carries the other's registers.
  if (wave < 2) {
    // ---------------- state waves ----------------
    const int rt = wave;                       // row tile
    const bool state_wave = rt < nrb;
    float sv[NKT][4];                          // S[16 rt + lr][16 kt + 4 lg + e]
    HL sf[NKS];                                // S fragments (rows i, k in fragment order)
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[kt][e] = 0.0f;
    if (state_wave && a.S0) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const float4 s = *reinterpret_cast<const float4*>(
            a.S0 + ((long)chain * dv + i0 + 16 * rt + lr) * DK + 16 * kt + 4 * lg);
        sv[kt][0] = s.x; sv[kt][1] = s.y; sv[kt][2] = s.z; sv[kt][3] = s.w;
      }
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) sf[ks] = hl_two(sv[2 * ks], sv[2 * ks + 1]);
    __syncthreads();
    for (int c = -4; c < nchunks; ++c) {
      if (state_wave && c >= 0) {
        // ---- state chain of chunk c (registers) ----
        const int cb = c & 1, xb = c & 3;
        const long t0 = (long)c * CS;
        // every LDS operand of the chunk is read before the first product
        bf16x8 qf[2][NKS], xf[NKT];
        HL wf[2][NKS], pf[2];
        float4 ut4[2];
        float gt[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            if constexpr (REG)
              wf[tt][ks] = hl_pair(&sm.Whi[cb][16 * tt + lr][32 * ks + 8 * lg], &sm.Wlo[cb][16 * tt + lr][32 * ks + 8 * lg]);
            qf[tt][ks] = frag_bf16(&sm.Q[xb][16 * tt + lr][32 * ks + 8 * lg]);
          }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) ut4[tt] = *reinterpret_cast<const float4*>(&sm.Ut[cb][16 * rt + lr][16 * tt + 4 * lg]);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) xf[kt] = frag_bf16(&sm.XT[xb][16 * kt + lr][8 * lg]);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          pf[tt] = hl_pair(&sm.Phi[cb][16 * tt + lr][8 * lg], &sm.Plo[cb][16 * tt + lr][8 * lg]);
          gt[tt] = sm.gam[xb][16 * tt + lr];
        }
        const float gC = sm.gam[xb][CS - 1];

        floatx4 oacc[2], zacc[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          oacc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
          zacc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            if constexpr (REG) zacc[tt] = mma3(zacc[tt], wf[tt][ks], sf[ks]);   // (Wt^T S)[t][i]
            oacc[tt] = mma2(oacc[tt], sf[ks], qf[tt][ks]);                      // (S q)[i][t]
          }
        }
        // z[t][i] = Ut[i][t] - (Wt^T S)[t][i]; lane: t = 16 tt + 4 lg + e, i = lr
        float z[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          z[tt][0] = ut4[tt].x - zacc[tt][0];
          z[tt][1] = ut4[tt].y - zacc[tt][1];
          z[tt][2] = ut4[tt].z - zacc[tt][2];
          z[tt][3] = ut4[tt].w - zacc[tt][3];
        }
        const HL zf = hl_two(z[0], z[1]);                               // rows i, t in fragment order
        // carry: S[i][k] <- g_{C-1} (S[i][k] + sum_t z[i][t] x_t[k])
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          floatx4 cacc = {0.f, 0.f, 0.f, 0.f};
          cacc = mma2(cacc, xf[kt], zf);
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[kt][e] = gC * (sv[kt][e] + cacc[e]);
        }
        // readout: o[t][i] = g_t ((S q)[i][t] + sum_{s<=t} z[i][s] (q_t . x_s))
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          oacc[tt] = mma3(oacc[tt], zf, pf[tt]);
          const int t = 16 * tt + lr;
          if (t0 + t < L)
            *reinterpret_cast<float4*>(a.o + v_base + (t0 + t) * dv + i0 + 16 * rt + 4 * lg) =
                make_float4(gt[tt] * oacc[tt][0], gt[tt] * oacc[tt][1], gt[tt] * oacc[tt][2], gt[tt] * oacc[tt][3]);
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) sf[ks] = hl_two(sv[2 * ks], sv[2 * ks + 1]);
      }
      __syncthreads();
    }
    if (state_wave && a.S_out) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
        *reinterpret_cast<float4*>(a.S_out + ((long)chain * dv + i0 + 16 * rt + lr) * DK + 16 * kt + 4 * lg) =
            make_float4(sv[kt][0], sv[kt][1], sv[kt][2], sv[kt][3]);
    }
  } else {
    // ---------------- preparation waves ----------------
    prefetch_k(0);
    __syncthreads();
    for (int c = -4; c < nchunks; ++c) {
      // ---- preparation: every stage reads only what earlier iterations wrote ----
      if (c + 4 < nchunks) commit_k(c + 4);
      if (c + 2 >= 0 && c + 2 < nchunks) commit_qv(c + 2);
      if (c + 5 < nchunks) prefetch_k(c + 5);
      if (c + 3 >= 0 && c + 3 < nchunks) prefetch_qv(c + 3);
      const bool v1 = c + 1 >= 0 && c + 1 < nchunks;
      const bool v2 = c + 2 >= 0 && c + 2 < nchunks;
      const bool v3 = c + 3 >= 0 && c + 3 < nchunks;
      if (v2) transpose_keys(c + 2);
      if (v2 && wave == 7) {
        scalars(c + 2);
        wave_sync();
      }
      if constexpr (REG) {
        if (v3 && wave < 6) gram_tile(c + 3, (wave - 2) >> 1, (wave - 2) & 1);
        if (v2 && wave == 7) solve_factors(c + 2);
        if (v1) {
          if (wave - 2 < NKT) solve_tile(c + 1, true, wave - 2);
          if (wave == 6) {
            solve_tile(c + 1, false, 0);
            if (nrb > 1) solve_tile(c + 1, false, 1);
          }
        }
      } else {
        if (v1) zeta_y(c + 1);
      }
      // q.x tiles (0,0), (1,0), (1,1) of chunk c+1 on waves 2, 3, 4
      if (v1 && wave < 5) qx_tile(c + 1, (wave - 1) >> 1, (wave - 2) >> 1);
      __syncthreads();
    }
  }
}

template <int DK, bool REG>
hipError_t launch_wy(const SeqArgs& a, hipStream_t stream) {
  static_assert(sizeof(WyLds<DK>) <= 160 * 1024, "LDS budget");
  WyGeom geo;
  const int nchain = a.batch * a.heads;
  geo.nrbg = (a.dv + RW - 1) / RW;
  geo.remap = (nchain % 8 == 0) ? 1 : 0;
  geo.nchunks = (int)((a.seqlen + CS - 1) / CS);
  const unsigned nblocks = (unsigned)(nchain * geo.nrbg);
  hipLaunchKernelGGL((chunk_wy_kernel<DK, REG>), dim3(nblocks), dim3(NT), 0, stream, a, geo);
  return hipGetLastError();
}

}  // namespace

bool chunk_wy_supported(const SeqArgs& a) {
  return a.window == 1 && a.beta_kind != 2 && (a.dk == 32 || a.dk == 64);
}

// Window-1 chunk form with gains shared by the value rows, 32-step chunks.
hipError_t launch_chunk_wy(const SeqArgs& a, hipStream_t stream) {
  if (a.dk == 32) return a.regression ? launch_wy<32, true>(a, stream) : launch_wy<32, false>(a, stream);
  if (a.dk == 64) return a.regression ? launch_wy<64, true>(a, stream) : launch_wy<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace falcon
