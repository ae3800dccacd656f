// falcon_chunk_wyb.hip - chunk-parallel Falcon forward for a sliding window of
// B = 2 or 4 samples with gains shared by the value rows (Falcon-3, Falcon-3A;
// scalar or per-token beta), dk in {64, 128}.
//
// Method: explainer of arXiv 2608.27763, section 核心方法 §3 (chunk-parallel
// form) and the 163.com article, section 02 (2) (only the fixed-size state
// crosses chunks; Gram / WY representation with a triangular solve).  Key-folded
// form, derived from the recurrence:
//   sub-chunks of 16 steps; the key tile of sub-chunk c holds the 32 keys of
//   sub-chunks c-1 and c (tile index m).  The unknown u = (t, w) (step t, window
//   slot w) has key m(u) = 16 + t - w.  With g_t = prod_{r<=t} a_r,
//   zeta_t = eta_t / g_t, omega_t = zeta_t g_{t-1} and
//     M[u][u'] = omega_t(u) (x_m(u) . x_m(u'))  for t(u') < t(u),   V = (I + M)^-1
//     F_x = V diag(omega_t(u)) Gath,  F_y = V diag(zeta_t(u)) Gath   (Gath[u][m] = [m(u) = m])
//     H = Gath^T F,  Q = P' F,  P'[t][u] = (q_t . x_m(u)) [t(u) <= t]
//   the state enters only through XS = X S0^T (keys x value rows):
//     Fk = H_y Y - H_x XS,   o_t = g_t (S0 q_t + (Q_y Y)_t - (Q_x XS)_t),
//     S_c = g_15 (S0 + Fk^T X).
//   The inner-product family has F_x = 0 and F_y = diag(zeta) Gath, so
//   H_y = diag(c_m) with c_m the sum of zeta over the unknowns of key m.
//   V is formed over 16-unknown blocks: T_bb = (I + M_bb)^-1 by forward
//   substitution, then V_b = T_bb (R_b - sum_{b'<b} M_bb' V_b') for the folded
//   right-hand sides R = diag(s) Gath.
//
// Structure.  One workgroup = 8 wave64 = one (batch*head) chain x 32 value rows.
// Iteration c: waves 0, 1 run the state of sub-chunk c (16 rows each, S in
// registers); waves 2..7 prepare the sub-chunks after it, three deep, in two
// phases separated by workgroup barriers (regression family):
//   A  blocked substitution for F_x, F_y and the folds H, Q of c+1 (waves 2-5,
//      one per SIMD) | Gram and q.x of the key tile, keys transposed and
//      per-step scalars of c+2        (state: split S, XS = X S0^T, Fk, readout)
//   B  T_bb by a DPP forward substitution, -M and P' fragments of c+2 | H_y Y,
//      Q_y Y of c+1 | commit the loads of c+3 to LDS and issue those of c+4
//                                     (state: carry)
// The inner-product family: scalars, q.x and transposes of c+1 (state:
// readout, carry), then Fk and Q_y Y of c+1 and the commits.
// Operands are stored in the fragment order of the register operand they meet
// (within a 32-wide group, slots 8g..8g+3 hold indices 4g..4g+3 and
// 8g+4..8g+7 hold 16+4g..16+4g+3); non-exact operands are split-bf16 (Henry,
// Tang & Heinecke, ARITH 2019).
#include <type_traits>

#include "falcon_device.h"
#include "falcon_exact.h"
#include "falcon_launch.h"
#include "falcon_mma.h"

namespace falcon {
namespace {

constexpr int CS = 16;       // steps per sub-chunk
constexpr int NXT = 32;      // keys per tile
constexpr int RW = 32;       // value rows per workgroup
constexpr int NW = 8;
constexpr int NT = 64 * NW;

__device__ __forceinline__ int fpos(int k) {
  const int kk = k & 31;
  return (k & ~31) + 8 * ((kk & 15) >> 2) + ((kk >> 4) << 2) + (kk & 3);
}

template <int DK>
struct WybLds {
  static constexpr int XR = DK + 16;     // bf16 row: DK (fragment order) + pad
  static constexpr int TP = CS + 12;     // bf16 rows over the steps of a block
  static constexpr int HP = NXT + 16;    // bf16 rows over the key tile
  static constexpr int FP = NXT + 4;     // fp32 rows over the key tile
  static constexpr int OP = RW + 4;      // fp32 rows over the value rows
  static constexpr int SP = 16 + 8;      // fp32 rows of a 16 x 16 block
  // (pads chosen on the whole kernel by the LDS bank-conflict counter)
  uint16_t X[4][CS][XR];                 // key blocks by sub-chunk & 3
  uint16_t Q[4][CS][XR];                 // query blocks
  uint16_t XT[4][DK][TP];                // key blocks transposed, steps natural
  uint16_t YT[4][RW][TP];                // value blocks transposed, steps natural
  float knorm[4][CS];
  float beta[4][CS];
  float G[NXT][FP];                      // Gram of the key tile
  float P[CS][FP];                       // q . x over the tile
  alignas(16) float gam[4][CS];          // per-step scalars by sub-chunk & 3
  alignas(16) float zeta[4][CS];
  alignas(16) float omega[4][CS];
  alignas(16) float zcum[4][CS];         // prefix sums of zeta
  float TS[4][16][SP];                   // diagonal blocks of T, row-major
  uint16_t Hxhi[2][NXT][HP];             // -H_x rows, keys in fragment order
  uint16_t Hxlo[2][NXT][HP];
  uint16_t Qxhi[2][CS][HP];              // -Q_x rows
  uint16_t Qxlo[2][CS][HP];
  uint16_t Hyhi[2][NXT][HP];             // H_y rows
  uint16_t Hylo[2][NXT][HP];
  uint16_t Qyhi[2][CS][HP];              // Q_y rows
  uint16_t Qylo[2][CS][HP];
  float Ufk[2][RW][FP];                  // (H_y Y)[m][i] stored [i][m]
  float Oy[2][CS][OP];                   // (Q_y Y)[t][i]
  uint16_t Mhi[4][16][HP];               // -M fragments of the blocked solve, by (block, pair)
  uint16_t Mlo[4][16][HP];
  uint16_t Pfhi[2][CS][HP];              // P' fragments over the unknowns, by pair of blocks
  uint16_t Pflo[2][CS][HP];
  alignas(16) float cm[2][NXT];          // inner-product family: sum of zeta per key
  int bad;                               // some sub-chunk's decay products left the range
  int badj[4];                           // the same per sub-chunk (& 3), pre-pass form
};

struct WybGeom {
  int nrbg;
  int remap;
  int nchunks;
  int seg_len;          // pre-pass: sub-chunks per workgroup
  int nseg;             // pre-pass: workgroups per chain
  unsigned char* rec;   // pre-pass records, [chain][sub-chunk][kWybRecBytes]
};

// One pre-pass record per (chain, sub-chunk): the folds of the sub-chunk as
// split-bf16 rows in fragment order (-H_x, H_y: 32 x 32; -Q_x, Q_y: 16 x 32;
// hi then lo), the decay products g_t (16 fp32) and a flag set when they leave
// the range of the chunk algebra.
constexpr int kWybRecFrag = 12288;      // bytes of bf16 fragments
constexpr int kWybRecGam = 12288;       // offset of g_t
constexpr int kWybRecBad = 12352;       // offset of the flag
constexpr int kWybRecBytes = 12416;

// acc + g(lane N of this 16-lane row) * r as one DPP multiply-add (g is only
// loaded from LDS, never written by the vector ALU, so no wait states apply)
template <int N>
__device__ __forceinline__ float fmac_bcast(float acc, float g, float r) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(g), "v"(r), "i"(N));
  return acc;
}
// forward substitution of (I + M) x = rhs over a 16-unknown block from pivot
// P on, M = diag(om) L(g): lane m of each 16-lane row holds row m in g[].  The B
// unknowns of a step do not couple (g is zero between them), so a pivot updates
// only the unknowns of later steps and the pivots of one step are independent.
template <int B, int P>
__device__ __forceinline__ void sweep(float (&rhs)[16], float (&acc)[16], const float (&g)[16], const float (&om)[16]) {
  rhs[P] = __builtin_fmaf(-om[P], acc[P], rhs[P]);
#pragma unroll
  for (int r = B * (P / B + 1); r < 16; ++r) acc[r] = fmac_bcast<P>(acc[r], g[r], rhs[P]);
  if constexpr (P < 15) sweep<B, P + 1>(rhs, acc, g, om);
}
template <int N>
__device__ __forceinline__ float dpp_shr(float v, float fill) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill), __builtin_bit_cast(int, v),
                                                             0x110 + N, 0xF, 0xF, false));
}
__device__ __forceinline__ floatx4 mma3(floatx4 acc, const HL& a, const HL& b) {
  acc = mfma16(a.hi, b.lo, acc);
  acc = mfma16(a.lo, b.hi, acc);
  return mfma16(a.hi, b.hi, acc);
}
__device__ __forceinline__ floatx4 mma2(floatx4 acc, const bf16x8& a, const HL& b) {
  acc = mfma16(a, b.hi, acc);
  return mfma16(a, b.lo, acc);
}
__device__ __forceinline__ floatx4 mma2(floatx4 acc, const HL& a, const bf16x8& b) {
  acc = mfma16(a.hi, b, acc);
  return mfma16(a.lo, b, acc);
}
__device__ __forceinline__ HL hl_two(const float* a, const float* b) {
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return hl_vals(v);
}
__device__ __forceinline__ HL hl_x4(const floatx4& a, const floatx4& b) {
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return hl_vals(v);
}
__device__ __forceinline__ floatx4 f4x(const float4& v) { return floatx4{v.x, v.y, v.z, v.w}; }
// two groups of 4 bf16 (8-byte reads) as one fragment
__device__ __forceinline__ bf16x8 frag_two(const uint16_t* a, const uint16_t* b) {
  const uint2 x = *reinterpret_cast<const uint2*>(a);
  const uint2 y = *reinterpret_cast<const uint2*>(b);
  return __builtin_bit_cast(bf16x8, make_uint4(x.x, x.y, y.x, y.y));
}

// PREP: the pre-pass form.  A workgroup prepares sub-chunks [s0, s1) of one
// chain (no state, no outputs) and writes one record per sub-chunk; waves 0 and
// 1, the state waves of the fused form, store the records.
template <int DK, bool REG, int B, bool PREP>
__global__ __launch_bounds__(NT) void chunk_wyb_kernel(SeqArgs a, WybGeom geo) {
  using SM = WybLds<DK>;
  constexpr int NKT = DK / 16, NKS = DK / 32, VPR = DK / 8;
  constexpr int U = 16 * B, NB = B, NKU = (NB + 1) / 2;
  static_assert(B == 2 || B == 4, "window 2 or 4");
  static_assert(DK == 64 || DK == 128, "dk in {64, 128}");
  __shared__ __align__(16) SM sm;

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(a.v);
  const uint16_t* __restrict__ kpg = static_cast<const uint16_t*>(a.k_prev);
  const uint16_t* __restrict__ bg = static_cast<const uint16_t*>(a.beta_t);

  int chain, rbg, s0, s1;
  if constexpr (PREP) {
    const int b = blockIdx.x;
    chain = b / geo.nseg;
    rbg = 0;
    s0 = (b % geo.nseg) * geo.seg_len;
    s1 = s0 + geo.seg_len < geo.nchunks ? s0 + geo.seg_len : geo.nchunks;
  } else {
    s0 = 0;
    s1 = geo.nchunks;
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
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const long L = a.seqlen;
  const long qk_base = (long)chain * L * DK;
  const long v_base = (long)chain * L * dv;
  const int nchunks = geo.nchunks;
  auto live_chunk = [&](int j) __attribute__((always_inline)) { return j >= s0 && j < s1; };
  auto steps = [&](int j) __attribute__((always_inline)) {
    const long t0 = (long)j * CS;
    return (int)((L - t0) < CS ? (L - t0) : CS);
  };
  // key tile index of unknown u and its step
  auto mof = [](int u) __attribute__((always_inline)) { return 16 + u / B - u % B; };

  // ---------------- block -1 (before the sequence) is zero ----------------
  if (tid == 0) sm.bad = 0;
  if (PREP && s0 > 0) {
    // a later segment: block s0 - 1 of the sequence, whose keys the first
    // sub-chunk's tile and windows reach, is loaded here (below)
  } else {
  for (int idx = tid; idx < CS * SM::XR; idx += NT) (&sm.X[3][0][0])[idx] = 0;
  for (int idx = tid; idx < DK * SM::TP; idx += NT) (&sm.XT[3][0][0])[idx] = 0;
  for (int idx = tid; idx < RW * SM::TP; idx += NT) (&sm.YT[3][0][0])[idx] = 0;
  if (tid < CS) sm.knorm[3][tid] = 0.0f;
  if (a.x_hist) {
    // a resumed sequence: its last B-1 rows are the carried window samples
    // (oldest first), which the first steps' windows reach
    const uint16_t* __restrict__ xhg = static_cast<const uint16_t*>(a.x_hist);
    const uint16_t* __restrict__ yhg = static_cast<const uint16_t*>(a.y_hist);
    constexpr int NH = B - 1;
    __syncthreads();
    for (int idx = tid; idx < NH * DK; idx += NT) {
      const int h = idx / DK, kk = idx % DK, t = CS - NH + h;
      const uint16_t xv = xhg[((long)chain * NH + h) * DK + kk];
      sm.X[3][t][fpos(kk)] = xv;
      sm.XT[3][kk][t] = xv;
    }
    for (int idx = tid; idx < NH * RW; idx += NT) {
      const int h = idx / RW, i = idx % RW, t = CS - NH + h;
      sm.YT[3][i][t] = (i0 + i < dv) ? yhg[((long)chain * NH + h) * dv + i0 + i] : (uint16_t)0;
    }
    if (tid < NH) {
      float n = 0.0f;
      for (int kk = 0; kk < DK; ++kk) {
        const float xv = bf16_to_f32(xhg[((long)chain * NH + tid) * DK + kk]);
        n += xv * xv;
      }
      sm.knorm[3][CS - NH + tid] = n;
    }
  }
  }

  // ---------------- global loads (buffer resources, range checked) ----------------
  // wave 6 moves the keys of a sub-chunk, wave 7 its queries, values and gains;
  // loads are issued one iteration before their commit.  Pieces past the end of
  // the sequence (or before its start) read 0.
  constexpr int BUF_WORD3 = 0x00020000;
  constexpr uint32_t PARKED = 0xC0000000u;
  auto rsrc = [](const void* base, long bytes) __attribute__((always_inline)) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, BUF_WORD3);
  };
  auto ld128 = [](__amdgpu_buffer_rsrc_t r, uint32_t off) __attribute__((always_inline)) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  constexpr int KP = CS * VPR / 64;        // 16-byte pieces per lane of a key or query block
  struct KSet { uint4 p[KP]; };
  struct QSet { uint4 p[KP]; uint4 v, v2; uint32_t b; };
  const auto rk = rsrc(kg + qk_base, L * DK * 2);
  const auto rq = rsrc(qg + qk_base, L * DK * 2);
  const auto rv = rsrc(vg + v_base, L * dv * 2);
  const auto rb = a.beta_kind == 1 ? rsrc(bg + (long)chain * L, L * 2) : rsrc(vg, 0);
  constexpr uint32_t KQ_CHUNK = CS * DK * 2;
  // key x_g = k_{g-s}: piece p of the block is row p / VPR - s, k = 8 (p % VPR)
  auto koff = [&](int u) __attribute__((always_inline)) {
    const int p = lane + 64 * u;
    return (uint32_t)(((p / VPR - a.key_shift) * DK + (p % VPR) * 8) * 2);
  };
  auto qoff = [&](int u) __attribute__((always_inline)) {
    const int p = lane + 64 * u;
    return (uint32_t)(((p / VPR) * DK + (p % VPR) * 8) * 2);
  };
  // values: lanes 0..31 move a 4 (steps) x 4 (rows) block, t4 = 4 (lane / 8), i4 = 4 (lane % 8)
  const int vb_t4 = 4 * ((lane & 31) >> 3), vb_i4 = 4 * (lane & 7);
  const uint32_t voff = (lane < 32 && i0 + vb_i4 < dv) ? (uint32_t)((vb_t4 * dv + i0 + vb_i4) * 2) : PARKED;
  const uint32_t V_CHUNK = (uint32_t)(CS * dv * 2);
  uint4 kprev[KP];
#pragma unroll
  for (int u = 0; u < KP; ++u) {
    kprev[u] = make_uint4(0u, 0u, 0u, 0u);
    const int p = lane + 64 * u;
    if (wave == 6 && kpg != nullptr && p / VPR == 0)
      kprev[u] = *reinterpret_cast<const uint4*>(kpg + (long)chain * DK + (p % VPR) * 8);
  }
  auto prefetch_k = [&](KSet& s, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < KP; ++u) s.p[u] = ld128(rk, koff(u) + (uint32_t)j * KQ_CHUNK);
  };
  auto prefetch_q = [&](QSet& s, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < KP; ++u) s.p[u] = ld128(rq, qoff(u) + (uint32_t)j * KQ_CHUNK);
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto val = __builtin_amdgcn_raw_buffer_load_b64(rv, (int)(voff + (uint32_t)j * V_CHUNK + (uint32_t)(e * dv * 2)), 0, 0);
      w[2 * e] = val[0];
      w[2 * e + 1] = val[1];
    }
    s.v = make_uint4(w[0], w[1], w[2], w[3]);
    s.v2 = make_uint4(w[4], w[5], w[6], w[7]);
    s.b = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)((uint32_t)(lane & 15) * 2 + (uint32_t)j * (CS * 2)), 0, 0);
  };
  auto put8 = [&](uint16_t* row, int k0, uint4 val) __attribute__((always_inline)) {
    *reinterpret_cast<uint2*>(row + fpos(k0)) = make_uint2(val.x, val.y);
    *reinterpret_cast<uint2*>(row + fpos(k0 + 4)) = make_uint2(val.z, val.w);
  };
  // keys of sub-chunk j to LDS, with their squared norms (packed bf16 dot
  // products, then a DPP sum over the VPR threads of a row)
  auto commit_k = [&](const KSet& s, int j) __attribute__((always_inline)) {
    const int jb = j & 3;
#pragma unroll
    for (int u = 0; u < KP; ++u) {
      const int p = lane + 64 * u;
      const int t = p / VPR, kv = p % VPR;
      const uint4 val = (j == 0 && t == 0 && a.key_shift) ? kprev[u] : s.p[u];
      put8(&sm.X[jb][t][0], kv * 8, val);
      float part = 0.0f;
      const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 v = __builtin_bit_cast(bf16x2, w4[e]);
        part = __builtin_amdgcn_fdot2_f32_bf16(v, v, part, false);
      }
      part += dpp_shr<1>(part, 0.0f);
      part += dpp_shr<2>(part, 0.0f);
      part += dpp_shr<4>(part, 0.0f);
      if constexpr (VPR == 16) part += dpp_shr<8>(part, 0.0f);
      if (kv == VPR - 1) sm.knorm[jb][t] = part;
    }
  };
  auto commit_q = [&](const QSet& s, int j) __attribute__((always_inline)) {
    const int jb = j & 3;
#pragma unroll
    for (int u = 0; u < KP; ++u) {
      const int p = lane + 64 * u;
      put8(&sm.Q[jb][p / VPR][0], (p % VPR) * 8, s.p[u]);
    }
    if (lane < 32) {
      if constexpr (PREP) return;   // the pre-pass does not use the values
      const uint32_t w[8] = {s.v.x, s.v.y, s.v.z, s.v.w, s.v2.x, s.v2.y, s.v2.z, s.v2.w};
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const uint32_t sel = (ii & 1) ? 0x07060302u : 0x05040100u;
        const int h = ii >> 1;
        *reinterpret_cast<uint2*>(&sm.YT[jb][vb_i4 + ii][vb_t4]) =
            make_uint2(__builtin_amdgcn_perm(w[2 + h], w[h], sel), __builtin_amdgcn_perm(w[6 + h], w[4 + h], sel));
      }
    } else if (lane < 48) {
      sm.beta[jb][lane & 15] = a.beta_kind == 0 ? a.beta : bf16_to_f32((uint16_t)s.b);
    }
  };

  // ---------------- Gram, q.x, transposes, scalars (phase A of j - 2) ----------------
  // Gram tile (mi, mj) of the key tile (blocks j-1, j): stored transposed, G symmetric
  auto gram_tile = [&](int j, int mi, int mj) __attribute__((always_inline)) {
    const int bi = (j - 1 + mi) & 3, bj = (j - 1 + mj) & 3;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      acc = mfma16(frag_bf16(&sm.X[bi][lr][32 * ks + 8 * lg]), frag_bf16(&sm.X[bj][lr][32 * ks + 8 * lg]), acc);
    *reinterpret_cast<float4*>(&sm.G[16 * mj + lr][16 * mi + 4 * lg]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  };
  // q.x: P^T tile mj -> P[t][16 mj + 4 lg ..]
  auto qx_tile = [&](int j, int mj) __attribute__((always_inline)) {
    const int bj = (j - 1 + mj) & 3;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      acc = mfma16(frag_bf16(&sm.X[bj][lr][32 * ks + 8 * lg]), frag_bf16(&sm.Q[j & 3][lr][32 * ks + 8 * lg]), acc);
    *reinterpret_cast<float4*>(&sm.P[lr][16 * mj + 4 * lg]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  };
  // keys transposed: XT[k][t] from X[t][k]; item idx moves a 4 (t) x 4 (k) block
  auto transpose_keys = [&](int j, int idx) __attribute__((always_inline)) {
    const int jb = j & 3;
    if (idx < (CS / 4) * (DK / 4)) {
      const int t4 = 4 * (idx % (CS / 4)), k4 = 4 * (idx / (CS / 4));
      const int pk4 = fpos(k4);
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint2 r = *reinterpret_cast<const uint2*>(&sm.X[jb][t4 + e][pk4]);
        w[2 * e] = r.x;
        w[2 * e + 1] = r.y;
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint32_t sel = (kk & 1) ? 0x07060302u : 0x05040100u;
        const int h = kk >> 1;
        *reinterpret_cast<uint2*>(&sm.XT[jb][k4 + kk][t4]) =
            make_uint2(__builtin_amdgcn_perm(w[2 + h], w[h], sel), __builtin_amdgcn_perm(w[6 + h], w[4 + h], sel));
      }
    }
  };
  // c_{m,t} = sum of zeta_s over the unknowns (s, w) of key m with s <= t
  auto ckey = [&](int ss, int m, int t) __attribute__((always_inline)) {
    const int lo = m - 16 < 0 ? 0 : m - 16;
    const int hi0 = m - 16 + B - 1;
    const int hi = hi0 < t ? hi0 : t;
    const int hic = hi < 0 ? 0 : hi;
    const float top = sm.zcum[ss][hic];
    const float bot = sm.zcum[ss][lo > 0 ? lo - 1 : 0];
    const float v = top - (lo > 0 ? bot : 0.0f);
    return hi < lo ? 0.0f : v;
  };
  // eta_t = beta_t / (eps + n_t), n_t = sum of the window's squared key norms;
  // a_t = 1 - eta_t lambda; padded steps and the fresh-sequence first step take
  // eta = 0, a = 1.  Lanes 0..15 = steps (one DPP row).
  auto scalars = [&](int j) __attribute__((always_inline)) {
    const int t = lr;
    const int ss = j & 3;
    float n = 0.0f;
#pragma unroll
    for (int w = 0; w < B; ++w) {
      const int m = 16 + t - w;
      n += m >= 16 ? sm.knorm[j & 3][m - 16] : sm.knorm[(j - 1) & 3][m];
    }
    const bool live = t < steps(j) && !((long)j * CS + t == 0 && kpg == nullptr && a.key_shift);
    float eta = 0.0f, dec = 1.0f;
    if (live) {
      eta = sm.beta[j & 3][t] * __builtin_amdgcn_rcpf(a.eps + n);
      dec = 1.0f - eta * a.lambda;
    }
    float gsc = dec;
    gsc *= dpp_shr<1>(gsc, 1.0f);
    gsc *= dpp_shr<2>(gsc, 1.0f);
    gsc *= dpp_shr<4>(gsc, 1.0f);
    gsc *= dpp_shr<8>(gsc, 1.0f);
    const float gprev = dpp_shr<1>(gsc, 1.0f);
    const bool out_of_range = __builtin_amdgcn_ballot_w64(lane < 16 && gauge_out_of_range(gsc, dec)) != 0;
    if constexpr (PREP) {
      if (lane == 0) sm.badj[ss] = out_of_range ? 1 : 0;
    } else {
      if (out_of_range && lane == 0) sm.bad = 1;
    }
    const float z = eta * __builtin_amdgcn_rcpf(gsc);
    float zc = z;
    zc += dpp_shr<1>(zc, 0.0f);
    zc += dpp_shr<2>(zc, 0.0f);
    zc += dpp_shr<4>(zc, 0.0f);
    zc += dpp_shr<8>(zc, 0.0f);
    if (lane < 16) {
      sm.gam[ss][t] = gsc;
      sm.zeta[ss][t] = z;
      sm.omega[ss][t] = z * gprev;
      sm.zcum[ss][t] = zc;
    }
    if constexpr (!REG) {   // c_m: zeta summed over the unknowns of key m (this wave wrote zcum)
      if (lane < NXT) sm.cm[j & 1][lane] = ckey(ss, lane, CS - 1);
    }
  };

  // ---------------- phase B (regression): diagonal blocks of T ----------------
  // One wave; 16-lane row b = block b (rows beyond B repeat the last block).
  // Lane n solves column n of (I + M_bb).  Row n of the block's coupling,
  // G[m(u_n)][m(u_r)] for the unknowns u_r of other steps, is read around the
  // block's key range; the same-step entries are zero.
  auto diag_blocks = [&](int j) __attribute__((always_inline)) {
    const int ss = j & 3;
    const int b = lg < B ? lg : B - 1;
    const int n = lr;
    const int un = 16 * b + n;
    const int mn = mof(un);
    const int base = 16 + 16 * b / B;          // key of (first step of the block, w = 0)
    constexpr int NG = (B == 4) ? 2 : 3;       // float4 groups from base - 4
    float gr[4 * NG];
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const float4 g4 = *reinterpret_cast<const float4*>(&sm.G[mn][base - 4 + 4 * q]);
      gr[4 * q] = g4.x; gr[4 * q + 1] = g4.y; gr[4 * q + 2] = g4.z; gr[4 * q + 3] = g4.w;
    }
    float g[16], om[16];
    float os[16 / B];
#pragma unroll
    for (int q = 0; q < 16 / B; q += 4) {
      const float4 o4 = *reinterpret_cast<const float4*>(&sm.omega[ss][16 * b / B + q]);
      os[q] = o4.x; os[q + 1] = o4.y; os[q + 2] = o4.z; os[q + 3] = o4.w;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = r / B - r % B;           // key of u_r relative to base
      g[r] = (r / B == n / B) ? 0.0f : gr[off + 4];
      om[r] = os[r / B];
    }
    float rhs[16], acc[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      rhs[m] = (m == n) ? 1.0f : 0.0f;
      acc[m] = 0.0f;
    }
    asm volatile("s_nop 4");
    sweep<B, 0>(rhs, acc, g, om);
    if (lg < B) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.TS[b][r][n] = rhs[r];
    }
  };

  // ---------------- phase B (regression): operand fragments of the blocked solve ----------------
  // fragment f = (block b, pair k): -M[u][u'] for u = 16 b + lr and the unknowns
  // u' of blocks 2k (slots 0-3) and 2k+1 (slots 4-7, zero unless 2k+1 < b)
  constexpr int NMF = NB == 4 ? 4 : 1;
  auto mf_bk = [](int f, int& b, int& k) __attribute__((always_inline)) {
    b = f == 0 ? 1 : f == 1 ? 2 : 3;
    k = f == 3 ? 1 : 0;
  };
  auto mfrag_store = [&](int j, int f) __attribute__((always_inline)) {
    int b, k;
    mf_bk(f, b, k);
    const int b2 = 2 * k + 1 < b ? 2 * k + 1 : -1;
    const int u = 16 * b + lr;
    const float nom = -sm.omega[j & 3][u / B];
    const float* grow = &sm.G[mof(u)][0];
    float v[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = nom * grow[mof(32 * k + 4 * lg + q)];
      v[4 + q] = b2 >= 0 ? nom * grow[mof(16 * (b2 < 0 ? 0 : b2) + 4 * lg + q)] : 0.0f;
    }
    store_split4(&sm.Mhi[f][lr][8 * lg], &sm.Mlo[f][lr][8 * lg], v);
    store_split4(&sm.Mhi[f][lr][8 * lg + 4], &sm.Mlo[f][lr][8 * lg + 4], v + 4);
  };
  // P'[t][u] = P[t][m(u)] [t(u) <= t] over the unknowns of blocks 2k, 2k+1
  auto pfrag_store = [&](int k) __attribute__((always_inline)) {
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int u = 32 * k + 4 * lg + (e & 3) + 16 * (e >> 2);
      pv[e] = (u < U && u / B <= lr) ? sm.P[lr][mof(u < U ? u : 0)] : 0.0f;
    }
    store_split4(&sm.Pfhi[k][lr][8 * lg], &sm.Pflo[k][lr][8 * lg], pv);
    store_split4(&sm.Pfhi[k][lr][8 * lg + 4], &sm.Pflo[k][lr][8 * lg + 4], pv + 4);
  };

  // ---------------- phase A (regression): blocked substitution and folds ----------------
  // One wave per (F_x | F_y) x key-column tile mc.  V[b] (C layout) holds
  // V[16 b + 4 lg + e][16 mc + lr]; Vop[k] the split fragment over blocks 2k, 2k+1.
  // Gath fragments (B operand over the unknowns of blocks 2k, 2k+1; column m = 16 mj + lr)
  bf16x8 gath[2][NKU];
#pragma unroll
  for (int mj = 0; mj < 2; ++mj)
#pragma unroll
    for (int k = 0; k < NKU; ++k) {
      uint32_t gw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ua = 32 * k + 4 * lg + 2 * (e & 1) + 16 * (e >> 1);   // slots 2e, 2e+1
        const int m = 16 * mj + lr;
        const uint32_t lo = (ua < U && mof(ua) == m) ? 0x3F80u : 0u;
        const uint32_t hi = (ua + 1 < U && mof(ua + 1) == m) ? 0x3F80u : 0u;
        gw[e] = lo | (hi << 16);
      }
      gath[mj][k] = __builtin_bit_cast(bf16x8, make_uint4(gw[0], gw[1], gw[2], gw[3]));
    }
  auto combine = [&](int j, bool fx, int mc) __attribute__((always_inline)) {
    const int sb = j & 1;
    const float* sc = fx ? sm.omega[j & 3] : sm.zeta[j & 3];
    const float z4[4] = {0.f, 0.f, 0.f, 0.f};
    const floatx4 zacc = {0.f, 0.f, 0.f, 0.f};
    floatx4 V[NB];
    HL Vop[NKU];
    uint4 vh[NKU], vl[NKU];
    // every operand fragment is read before the substitution starts
    HL mf[NMF], tf[NB], pf[NKU];
#pragma unroll
    for (int f = 0; f < NMF; ++f) mf[f] = hl_pair(&sm.Mhi[f][lr][8 * lg], &sm.Mlo[f][lr][8 * lg]);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float4 t4 = *reinterpret_cast<const float4*>(&sm.TS[b][lr][4 * lg]);
      const float tv[4] = {t4.x, t4.y, t4.z, t4.w};
      tf[b] = hl_two(tv, z4);
    }
#pragma unroll
    for (int k = 0; k < NKU; ++k) pf[k] = hl_pair(&sm.Pfhi[k][lr][8 * lg], &sm.Pflo[k][lr][8 * lg]);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      floatx4 acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) {     // R_b = diag(s) Gath, column 16 mc + lr
        const int u = 16 * b + 4 * lg + e;
        acc[e] = mof(u) == 16 * mc + lr ? sc[u / B] : 0.0f;
      }
#pragma unroll
      for (int k = 0; 2 * k < b; ++k)    // - sum over earlier blocks 2k, 2k+1
        acc = mma3(acc, mf[b == 1 ? 0 : b == 2 ? 1 : (k == 0 ? 2 : 3)], Vop[k]);
      const float av[4] = {acc[0], acc[1], acc[2], acc[3]};
      V[b] = mma3(zacc, tf[b], hl_two(av, z4));
      // split V[b] once; its halves fill slots 0-3 (b even) or 4-7 (b odd) of Vop
      uint32_t hh[2], ll[2];
      split_pair(V[b][0], V[b][1], hh[0], ll[0]);
      split_pair(V[b][2], V[b][3], hh[1], ll[1]);
      if ((b & 1) == 0) {
        vh[b / 2] = make_uint4(hh[0], hh[1], 0u, 0u);
        vl[b / 2] = make_uint4(ll[0], ll[1], 0u, 0u);
      } else {
        vh[b / 2].z = hh[0]; vh[b / 2].w = hh[1];
        vl[b / 2].z = ll[0]; vl[b / 2].w = ll[1];
      }
      Vop[b / 2].hi = __builtin_bit_cast(bf16x8, vh[b / 2]);
      Vop[b / 2].lo = __builtin_bit_cast(bf16x8, vl[b / 2]);
    }
    // folds: (Gath^T V)^T tiles and (P' V)^T
    const float sign = fx ? -1.0f : 1.0f;          // -H_x, -Q_x; +H_y, +Q_y
    uint16_t* Hhi = fx ? &sm.Hxhi[sb][0][0] : &sm.Hyhi[sb][0][0];
    uint16_t* Hlo = fx ? &sm.Hxlo[sb][0][0] : &sm.Hylo[sb][0][0];
    uint16_t* Qhi = fx ? &sm.Qxhi[sb][0][0] : &sm.Qyhi[sb][0][0];
    uint16_t* Qlo = fx ? &sm.Qxlo[sb][0][0] : &sm.Qylo[sb][0][0];
    constexpr int HS = SM::HP;
#pragma unroll
    for (int mj = 0; mj < 2; ++mj) {
      floatx4 h = zacc;
#pragma unroll
      for (int k = 0; k < NKU; ++k) h = mma2(h, Vop[k], gath[mj][k]);
      const float hv[4] = {sign * h[0], sign * h[1], sign * h[2], sign * h[3]};
      store_split4(Hhi + (16 * mj + lr) * HS + 8 * lg + 4 * mc, Hlo + (16 * mj + lr) * HS + 8 * lg + 4 * mc, hv);
    }
    {
      floatx4 qa = zacc;
#pragma unroll
      for (int k = 0; k < NKU; ++k) qa = mma3(qa, Vop[k], pf[k]);
      const float qv[4] = {sign * qa[0], sign * qa[1], sign * qa[2], sign * qa[3]};
      store_split4(Qhi + lr * HS + 8 * lg + 4 * mc, Qlo + lr * HS + 8 * lg + 4 * mc, qv);
    }
  };

  // values of the key tile as a fragment over keys (slots 0-3: block j-1, 4-7: block j)
  auto yfrag = [&](int j, int i) __attribute__((always_inline)) {
    return frag_two(&sm.YT[(j - 1) & 3][i][4 * lg], &sm.YT[j & 3][i][4 * lg]);
  };
  // ---------------- phase B (regression): H_y Y and Q_y Y ----------------
  auto ufk_tile = [&](int j, int mt, int it) __attribute__((always_inline)) {
    const HL hy = hl_pair(&sm.Hyhi[j & 1][16 * mt + lr][8 * lg], &sm.Hylo[j & 1][16 * mt + lr][8 * lg]);
    const floatx4 acc = mma2(floatx4{0.f, 0.f, 0.f, 0.f}, hy, yfrag(j, 16 * it + lr));
    *reinterpret_cast<float4*>(&sm.Ufk[j & 1][16 * it + lr][16 * mt + 4 * lg]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  };
  auto oy_tile = [&](int j, int it, const HL& qy) __attribute__((always_inline)) {
    const floatx4 acc = mma2(floatx4{0.f, 0.f, 0.f, 0.f}, yfrag(j, 16 * it + lr), qy);
    *reinterpret_cast<float4*>(&sm.Oy[j & 1][lr][16 * it + 4 * lg]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  };
  // ---------------- phase 2 (inner-product family) ----------------
  auto ip_ufk = [&](int j) __attribute__((always_inline)) {   // Ufk[i][m] = c_m y_m[i]
    const int i = lane & 31, half = lane >> 5;
    const int jb = (j - 1 + half) & 3;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint2 y = *reinterpret_cast<const uint2*>(&sm.YT[jb][i][4 * q4]);
      const float yv[4] = {bf16_to_f32((uint16_t)(y.x & 0xFFFFu)), bf16_to_f32((uint16_t)(y.x >> 16)),
                           bf16_to_f32((uint16_t)(y.y & 0xFFFFu)), bf16_to_f32((uint16_t)(y.y >> 16))};
      float o[4];
      const float4 c4 = *reinterpret_cast<const float4*>(&sm.cm[j & 1][16 * half + 4 * q4]);
      o[0] = c4.x * yv[0]; o[1] = c4.y * yv[1]; o[2] = c4.z * yv[2]; o[3] = c4.w * yv[3];
      *reinterpret_cast<float4*>(&sm.Ufk[j & 1][i][16 * half + 4 * q4]) = make_float4(o[0], o[1], o[2], o[3]);
    }
  };
  auto ip_oy = [&](int j) __attribute__((always_inline)) {     // Q_y[t][m] = P[t][m] c_{m,t}
    const int t = lr;
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int m = 4 * lg + (e & 3) + 16 * (e >> 2);
      pv[e] = sm.P[t][m] * ckey(j & 3, m, t);
    }
    const HL qy = hl_vals(pv);
    oy_tile(j, 0, qy);
    oy_tile(j, 1, qy);
  };

  // Regression, iterations c = -3 .. nchunks-1, two phases each:
  //   A  state of sub-chunk c up to its readout | blocked substitution and folds
  //      of c+1 | Gram, q.x, scalars and transposed keys of c+2
  //   B  carry of c, H_y Y and Q_y Y of c+1 | diagonal blocks of T, -M and P'
  //      fragments of c+2 | commit of c+3, loads of c+4
  // Inner product, iterations c = -2 .. nchunks-1: state of c, preparation of
  // c+1, commit of c+2, loads of c+3, also in two phases.
  const int c_begin = REG ? s0 - 3 : -2;
  if (PREP && wave < 2) {
    // ---------------- pre-pass: record stores ----------------
    // iteration c prepares sub-chunk c + 1 in phase A (its folds) and stores its
    // record in phase B; g_t and the range flag were formed two iterations before
    for (int c = c_begin; c < s1 - 1; ++c) {
      __syncthreads();
      __syncthreads();
      const int j = c + 1;
      if (!live_chunk(j)) continue;
      unsigned char* rp = geo.rec + ((long)chain * nchunks + j) * kWybRecBytes;
      const int sb = j & 1;
      // piece pc = tid + 128 i (16 bytes): i < 4 the 32-row arrays -H_x hi, lo,
      // H_y hi, lo; i = 4, 5 the 16-row arrays -Q_x hi, lo, Q_y hi, lo (two per
      // i).  All six reads are issued before the stores, so the copy waits for
      // one LDS round trip instead of six.
      static_assert(kWybRecFrag == 16 * 128 * 6, "six 16-byte pieces per record thread");
      uint4 piece[6];
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        const int pc = tid + 128 * i;
        const uint16_t* src;
        if (i < 4) {
          const int r = (pc & 127) >> 2, g = pc & 3;
          const uint16_t* base = i == 0 ? &sm.Hxhi[sb][0][0] : i == 1 ? &sm.Hxlo[sb][0][0]
                               : i == 2 ? &sm.Hyhi[sb][0][0] : &sm.Hylo[sb][0][0];
          src = base + r * SM::HP + 8 * g;
        } else {
          const int q = pc - 512, ar = q >> 6, r = (q & 63) >> 2, g = q & 3;
          const uint16_t* base = ar == 0 ? &sm.Qxhi[sb][0][0] : ar == 1 ? &sm.Qxlo[sb][0][0]
                               : ar == 2 ? &sm.Qyhi[sb][0][0] : &sm.Qylo[sb][0][0];
          src = base + r * SM::HP + 8 * g;
        }
        piece[i] = *reinterpret_cast<const uint4*>(src);
      }
#pragma unroll
      for (int i = 0; i < 6; ++i) *reinterpret_cast<uint4*>(rp + 16 * (tid + 128 * i)) = piece[i];
      if (tid < CS) reinterpret_cast<float*>(rp + kWybRecGam)[tid] = sm.gam[j & 3][tid];
      if (tid == CS) *reinterpret_cast<int*>(rp + kWybRecBad) = sm.badj[j & 3];
    }
    return;
  }
  if (wave < 2) {
    // ---------------- state waves ----------------
    const int rt = wave;
    float sv[NKT][4];                          // S[16 rt + lr][16 kt + 4 lg + e]
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 16 * rt + lr, kk = 16 * kt + 4 * lg + e;
        sv[kt][e] = (a.S0 && i < dv) ? a.S0[((long)chain * dv + i) * DK + kk] : 0.0f;
      }
    HL sf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) sf[ks] = hl_two(sv[2 * ks], sv[2 * ks + 1]);
    float* orow = a.o + v_base + (long)lr * dv + i0 + 16 * rt + 4 * lg;
    const bool rows_in = i0 + 16 * rt < dv;
    for (int c = c_begin; c < nchunks; ++c) {
      const bool run = c >= 0 && rows_in;
      const int cb = c & 1;
      HL xsf;
      floatx4 fk[2];
      auto readout = [&]() __attribute__((always_inline)) {   // o_t = g_t (S0 q_t + O_y - Q_x XS)
        floatx4 oacc = f4x(*reinterpret_cast<const float4*>(&sm.Oy[cb][lr][16 * rt + 4 * lg]));
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) oacc = mma2(oacc, sf[ks], frag_bf16(&sm.Q[c & 3][lr][32 * ks + 8 * lg]));
        if constexpr (REG) oacc = mma3(oacc, xsf, hl_pair(&sm.Qxhi[cb][lr][8 * lg], &sm.Qxlo[cb][lr][8 * lg]));
        const float gt = sm.gam[c & 3][lr];
        if ((long)c * CS + lr < L)
          *reinterpret_cast<float4*>(orow) = make_float4(gt * oacc[0], gt * oacc[1], gt * oacc[2], gt * oacc[3]);
        orow += CS * dv;
      };
      auto carry = [&]() __attribute__((always_inline)) {     // S <- g_15 (S + Fk^T X)
        const HL fkf = hl_x4(fk[0], fk[1]);
        const float gC = sm.gam[c & 3][CS - 1];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          const bf16x8 xt = frag_two(&sm.XT[(c - 1) & 3][16 * kt + lr][4 * lg], &sm.XT[c & 3][16 * kt + lr][4 * lg]);
          const floatx4 cacc = mma2(floatx4{sv[kt][0], sv[kt][1], sv[kt][2], sv[kt][3]}, xt, fkf);
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[kt][e] = gC * cacc[e];
        }
      };
      auto resplit = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) sf[ks] = hl_two(sv[2 * ks], sv[2 * ks + 1]);
      };
      auto load_fk = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) fk[mi] = f4x(*reinterpret_cast<const float4*>(&sm.Ufk[cb][16 * rt + lr][16 * mi + 4 * lg]));
      };
      __syncthreads();
      if constexpr (REG) {
        // phase A: split the state, XS = X S0^T, Fk = Ufk - H_x XS, readout
        if (run) {
          resplit();
          floatx4 xs[2];
#pragma unroll
          for (int mi = 0; mi < 2; ++mi) {
            xs[mi] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
              xs[mi] = mma2(xs[mi], frag_bf16(&sm.X[(c - 1 + mi) & 3][lr][32 * ks + 8 * lg]), sf[ks]);
          }
          xsf = hl_x4(xs[0], xs[1]);
          load_fk();
#pragma unroll
          for (int mi = 0; mi < 2; ++mi)
            fk[mi] = mma3(fk[mi], hl_pair(&sm.Hxhi[cb][16 * mi + lr][8 * lg], &sm.Hxlo[cb][16 * mi + lr][8 * lg]), xsf);
          readout();
        }
        __syncthreads();
        // phase B: carry; one tile of H_y Y of the next sub-chunk
        if (run) carry();
        if (live_chunk(c + 1)) ufk_tile(c + 1, 0, rt);
      } else {
        if (run) load_fk();
        if (run) {                    // phase 1
          readout();
          carry();
        }
        __syncthreads();
        if (run) resplit();           // phase 2
      }
    }
    __syncthreads();
    if (rows_in && a.S_out && !sm.bad && i0 + 16 * rt + lr < dv) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
        *reinterpret_cast<float4*>(a.S_out + ((long)chain * dv + i0 + 16 * rt + lr) * DK + 16 * kt + 4 * lg) =
            make_float4(sv[kt][0], sv[kt][1], sv[kt][2], sv[kt][3]);
    }
  } else {
    // ---------------- preparation waves ----------------
    KSet ks0;
    QSet qs0;
    if (PREP && s0 > 0 && wave == 6) {   // block s0 - 1 of a later segment
      prefetch_k(ks0, s0 - 1);
      commit_k(ks0, s0 - 1);
    }
    if (wave == 6) prefetch_k(ks0, s0);
    if (wave == 7) prefetch_q(qs0, s0);
    // commit of sub-chunk c+2 (its ring slot is free during the whole iteration)
    // and the loads of c+3
    auto move = [&](int c) __attribute__((always_inline)) {
      if (wave == 6) {
        if (live_chunk(c + 2)) commit_k(ks0, c + 2);
        prefetch_k(ks0, c + 3);
      }
      if (wave == 7) {
        if (live_chunk(c + 2)) commit_q(qs0, c + 2);
        prefetch_q(qs0, c + 3);
      }
    };
    const int c_end = PREP ? s1 - 1 : nchunks;
    for (int c = c_begin; c < c_end; ++c) {
      const int j = c + 1;
      const bool pj = live_chunk(j);
      __syncthreads();
      if constexpr (REG) {
        const int j2 = c + 2;
        const bool pj2 = live_chunk(j2);
        // phase A: blocked substitution and folds of c+1 (one wave per SIMD:
        // waves 2, 3 F_x, waves 4, 5 F_y); Gram, q.x, scalars, transposed keys of c+2
        if (wave <= 5) {
          // window 4: the substitution (four blocks) is the longest chain of the
          // phase, so its waves issue first on the SIMDs they share with the state
          // and Gram waves (measured: 3-5% faster; with window 2 it is not, and
          // the priority costs time)
          if constexpr (B == 4) __builtin_amdgcn_s_setprio(2);
          if (pj) combine(j, wave < 4, wave & 1);
          if constexpr (B == 4) __builtin_amdgcn_s_setprio(0);
        } else if (wave == 6) {
          if (pj2) { gram_tile(j2, 0, 0); gram_tile(j2, 1, 0); gram_tile(j2, 0, 1); scalars(j2); }
        } else {
          if (pj2) {
            gram_tile(j2, 1, 1);
            qx_tile(j2, 0);
            qx_tile(j2, 1);
            if constexpr (!PREP) {     // the pre-pass has no carry to feed
              transpose_keys(j2, lane);
              transpose_keys(j2, 64 + lane);
            }
          }
        }
        __syncthreads();
        // phase B: diagonal blocks of T, -M and P' fragments of c+2; H_y Y and
        // Q_y Y of c+1; commit of c+3, loads of c+4
        if (pj2) {
          if (wave == 4) diag_blocks(j2);
          if (wave == 2) { mfrag_store(j2, 0); if (NMF > 1) mfrag_store(j2, 1); }
          if (wave == 3 && NMF > 2) { mfrag_store(j2, 2); mfrag_store(j2, 3); }
          if (wave == 5) pfrag_store(0);
          if (wave == 7 && NKU > 1) pfrag_store(NKU - 1);
        }
        if (pj && !PREP) {
          if (wave == 5) ufk_tile(j, 1, 0);
          if (wave == 6) {
            ufk_tile(j, 1, 1);
            oy_tile(j, 0, hl_pair(&sm.Qyhi[j & 1][lr][8 * lg], &sm.Qylo[j & 1][lr][8 * lg]));
          }
          if (wave == 7) oy_tile(j, 1, hl_pair(&sm.Qyhi[j & 1][lr][8 * lg], &sm.Qylo[j & 1][lr][8 * lg]));
        }
        move(c + 1);
      } else {
        // phase 1: Gram-free stages of c+1
        if (pj) {
          if (wave == 4) { qx_tile(j, 0); qx_tile(j, 1); }
          else if (wave == 5) scalars(j);
          else if (wave >= 6) transpose_keys(j, 64 * (wave - 6) + lane);
        }
        __syncthreads();
        // phase 2: Fk and readout terms; commits
        if (pj) {
          if (wave == 2) ip_ufk(j);
          if (wave == 3) ip_oy(j);
        }
        move(c);
      }
    }
    if constexpr (PREP) return;     // as many barriers as the record-store waves
    __syncthreads();
  }
  // a chain whose decay products left the range of the chunk algebra: its rows
  // again, exactly, by the recurrence (S_out was left untouched above)
  __syncthreads();
  if (sm.bad) recurrence_rows<DK, NT, B>(chain, i0, dv - i0 < RW ? dv - i0 : RW);
}

// ---------------------------------------------------------------------------
// State kernel of the two-kernel form: the sequential part only.  The pre-pass
// has written every sub-chunk's folds (-H_x, H_y, -Q_x, Q_y, split-bf16 rows in
// fragment order), its decay products and its range flag; per sub-chunk c this
// kernel forms XS = X S0^T, Fk = H_y Y - H_x XS, o_t = g_t (S0 q_t + (Q_y Y)_t -
// (Q_x XS)_t) and S_c = g_15 (S0 + Fk^T X) (the same equations as above).
// One workgroup = 8 wave64 = one chain x 32 value rows.  Waves 0-3 hold the
// state: wave w owns the 16-row tile w & 1 and the column half w >> 1 of S in
// registers (one wave per SIMD); XS and S0 q, sums over all columns, are formed
// as two column-half partials and added in LDS (one barrier per sub-chunk).
// Waves 4-7 move the data, each one part of every sub-chunk: its global reads
// four sub-chunks ahead, its commit to LDS two sub-chunks ahead (keys in
// fragment order and transposed, queries, values transposed, the -H_x and -Q_x
// fragments and g_t), and H_y Y and Q_y Y one ahead; waves 5 and 6 also form
// the outputs of the current sub-chunk from the state waves' partials, into
// LDS; state waves 0 and 1 store them to global memory two sub-chunks later
// (the data-movement waves then issue global loads only; measured no slower).
constexpr int ST_NW = 8;
constexpr int ST_NT = 64 * ST_NW;

template <int DK>
struct WybStLds {
  static constexpr int XR = DK + 16;
  static constexpr int TP = CS + 12;
  static constexpr int FP = NXT + 4;
  static constexpr int OP = RW + 4;
  static constexpr int FR = NXT + 8;     // bf16 row of a fold fragment array
  uint16_t X[4][CS][XR];                 // key blocks by sub-chunk & 3 (fragment order)
  uint16_t Q[4][CS][XR];                 // query blocks
  uint16_t XT[4][DK][TP];                // key blocks transposed
  uint16_t YT[4][RW][TP];                // value blocks transposed
  uint16_t Hx[4][2][NXT][FR];            // -H_x rows, hi / lo
  uint16_t Qx[4][2][CS][FR];             // -Q_x rows, hi / lo
  float gam[4][CS];                      // g_t
  float Ufk[4][RW][FP];                  // (H_y Y)[m][i] stored [i][m]
  float Oy[4][CS][OP];                   // (Q_y Y)[t][i]
  floatx4 PX[2][2][2][2][64];            // XS partials [c & 1][row tile][column half][key tile][lane]
  floatx4 PO[2][2][2][64];               // S0 q partials [c & 1][row tile][column half][lane]
  float4 OT[2][2][64];                   // outputs o_t [c & 1][row tile][lane]
  int bad;
};

template <int DK, int B>
__global__ __launch_bounds__(ST_NT) void wyb_state_kernel(SeqArgs a, WybGeom geo) {
  using SM = WybStLds<DK>;
  constexpr int NKT = DK / 16, NKS = DK / 32, VPR = DK / 8;
  constexpr int NKH = NKT / 2, NKSH = NKS / 2;     // 16-column tiles and 32-column steps per half
  static_assert(B == 2 || B == 4, "window 2 or 4");
  static_assert(DK == 64 || DK == 128, "dk in {64, 128}");
  __shared__ __align__(16) SM sm;

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(a.v);
  const uint16_t* __restrict__ kpg = static_cast<const uint16_t*>(a.k_prev);
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
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const long L = a.seqlen;
  const long qk_base = (long)chain * L * DK;
  const long v_base = (long)chain * L * dv;
  const int nchunks = geo.nchunks;

  // ---------------- block -1: zero, or the carried window samples ----------------
  if (tid == 0) sm.bad = 0;
  for (int idx = tid; idx < CS * SM::XR; idx += ST_NT) (&sm.X[3][0][0])[idx] = 0;
  for (int idx = tid; idx < DK * SM::TP; idx += ST_NT) (&sm.XT[3][0][0])[idx] = 0;
  for (int idx = tid; idx < RW * SM::TP; idx += ST_NT) (&sm.YT[3][0][0])[idx] = 0;
  if (a.x_hist) {
    const uint16_t* __restrict__ xhg = static_cast<const uint16_t*>(a.x_hist);
    const uint16_t* __restrict__ yhg = static_cast<const uint16_t*>(a.y_hist);
    constexpr int NH = B - 1;
    __syncthreads();
    for (int idx = tid; idx < NH * DK; idx += ST_NT) {
      const int h = idx / DK, kk = idx % DK, t = CS - NH + h;
      const uint16_t xv = xhg[((long)chain * NH + h) * DK + kk];
      sm.X[3][t][fpos(kk)] = xv;
      sm.XT[3][kk][t] = xv;
    }
    for (int idx = tid; idx < NH * RW; idx += ST_NT) {
      const int h = idx / RW, i = idx % RW, t = CS - NH + h;
      sm.YT[3][i][t] = (i0 + i < dv) ? yhg[((long)chain * NH + h) * dv + i0 + i] : (uint16_t)0;
    }
  }

  if (wave < 4) {
    // ---------------- state waves ----------------
    const int rt = wave & 1, ch = wave >> 1;
    float sv[NKH][4];                          // S[16 rt + lr][16 (NKH ch + kt) + 4 lg + e]
#pragma unroll
    for (int kt = 0; kt < NKH; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 16 * rt + lr, kk = 16 * (NKH * ch + kt) + 4 * lg + e;
        sv[kt][e] = (a.S0 && i < dv) ? a.S0[((long)chain * dv + i) * DK + kk] : 0.0f;
      }
    HL sf[NKSH];
    auto resplit = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < NKSH; ++ks) sf[ks] = hl_two(sv[2 * ks], sv[2 * ks + 1]);
    };
    resplit();
    const bool rows_in = i0 + 16 * rt < dv;
    // outputs of sub-chunk c (in LDS from waves 5, 6) to global memory: the
    // waves of column half 0, one row tile each
    auto store_o = [&](int c) __attribute__((always_inline)) {
      if (ch == 0 && (long)c * CS + lr < L)
        *reinterpret_cast<float4*>(a.o + v_base + ((long)c * CS + lr) * dv + i0 + 16 * rt + 4 * lg) =
            sm.OT[c & 1][rt][lane];
    };
    // Every operand but the partials and H_y Y was committed to LDS at least one
    // barrier before its use, so its read is issued off the chain: after barrier
    // c, the keys and queries of sub-chunk c + 1 and, once the carry of c has
    // used those of c, its -H_x rows, transposed keys and g_t.
    bf16x8 xf[2][NKSH], qf[NKSH];
    auto load_p1 = [&](int c) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < NKSH; ++ks) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) xf[mi][ks] = frag_bf16(&sm.X[(c - 1 + mi) & 3][lr][32 * (NKSH * ch + ks) + 8 * lg]);
        qf[ks] = frag_bf16(&sm.Q[c & 3][lr][32 * (NKSH * ch + ks) + 8 * lg]);
      }
    };
    HL hxf[2];
    bf16x8 xtf[NKH];
    float gC = 0.0f;
    auto load_p2 = [&](int c) __attribute__((always_inline)) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        hxf[mi] = hl_pair(&sm.Hx[c & 3][0][16 * mi + lr][8 * lg], &sm.Hx[c & 3][1][16 * mi + lr][8 * lg]);
#pragma unroll
      for (int kt = 0; kt < NKH; ++kt) {
        const int col = 16 * (NKH * ch + kt) + lr;
        xtf[kt] = frag_two(&sm.XT[(c - 1) & 3][col][4 * lg], &sm.XT[c & 3][col][4 * lg]);
      }
      gC = sm.gam[c & 3][CS - 1];
    };
    // this column half's partials of XS = X S_c^T and of S_c q for sub-chunk c,
    // from the state of its start
    auto products = [&](int c) __attribute__((always_inline)) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        floatx4 xs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKSH; ++ks) xs = mma2(xs, xf[mi][ks], sf[ks]);
        sm.PX[c & 1][rt][ch][mi][lane] = xs;
      }
      floatx4 oq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKSH; ++ks) oq = mma2(oq, sf[ks], qf[ks]);
      sm.PO[c & 1][rt][ch][lane] = oq;
    };
    for (int c = -2; c < nchunks; ++c) {
      const bool run = c >= 0 && rows_in;
      const int cb = c & 1, cs = c & 3;
      if (run) {
        if (c == 0) {
          load_p2(0);
          products(0);
        }
        if (c >= 2) store_o(c - 2);
      }
      __syncthreads();
      if (!run) {
        if (c == -1 && rows_in && nchunks > 0) load_p1(0);
        continue;
      }
      // XS, Fk = Ufk - H_x XS, the carry (the readout is on waves 5, 6), then
      // the products of sub-chunk c + 1 in the same block as the carry (after
      // the last sub-chunk they fill a partial buffer that nothing reads)
      floatx4 xs[2], fk[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const floatx4 p0 = sm.PX[cb][rt][0][mi][lane], p1 = sm.PX[cb][rt][1][mi][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) xs[mi][e] = p0[e] + p1[e];
        fk[mi] = f4x(*reinterpret_cast<const float4*>(&sm.Ufk[cs][16 * rt + lr][16 * mi + 4 * lg]));
      }
      load_p1(c + 1);
      const HL xsf = hl_x4(xs[0], xs[1]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) fk[mi] = mma3(fk[mi], hxf[mi], xsf);
      const HL fkf = hl_x4(fk[0], fk[1]);
#pragma unroll
      for (int kt = 0; kt < NKH; ++kt) {
        const floatx4 cacc = mma2(floatx4{sv[kt][0], sv[kt][1], sv[kt][2], sv[kt][3]}, xtf[kt], fkf);
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[kt][e] = gC * cacc[e];
      }
      resplit();
      load_p2(c + 1);
      products(c + 1);
    }
    __syncthreads();
    if (rows_in && !sm.bad) {
      if (nchunks >= 2) store_o(nchunks - 2);
      if (nchunks >= 1) store_o(nchunks - 1);
    }
    // the exact pass below rewrites this chain's outputs: the stores issued in
    // the loop complete first
    if (sm.bad) __threadfence();
    if (rows_in && a.S_out && !sm.bad && i0 + 16 * rt + lr < dv) {
#pragma unroll
      for (int kt = 0; kt < NKH; ++kt)
        *reinterpret_cast<float4*>(a.S_out + ((long)chain * dv + i0 + 16 * rt + lr) * DK + 16 * (NKH * ch + kt) + 4 * lg) =
            make_float4(sv[kt][0], sv[kt][1], sv[kt][2], sv[kt][3]);
    }
  } else {
    // ---------------- data-movement waves ----------------
    // Iteration c commits sub-chunk c + 2 and issues the reads of c + 6 (four
    // sub-chunks ahead, into a ring of four register sets indexed by c & 3):
    // wave 4 the keys (fragment order and transposed), wave 5 the queries and
    // values, wave 6 the -H_x / -Q_x fragments, g_t and the range flag; wave 7
    // forms H_y Y and Q_y Y of c + 1 from its own ring of H_y / Q_y fragments.
    const int role = wave - 4;
    constexpr int KP = CS * VPR / 64;          // 16-byte pieces per lane of a key or query block
    constexpr uint32_t KQ_CHUNK = CS * DK * 2;
    constexpr int BUF_WORD3 = 0x00020000;
    constexpr uint32_t PARKED = 0xC0000000u;
    auto rsrc = [](const void* base, long bytes) __attribute__((always_inline)) {
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, BUF_WORD3);
    };
    auto ld128 = [](__amdgpu_buffer_rsrc_t r, uint32_t off) __attribute__((always_inline)) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
      return make_uint4(v[0], v[1], v[2], v[3]);
    };
    const auto rk = rsrc(kg + qk_base, L * DK * 2);
    const auto rq = rsrc(qg + qk_base, L * DK * 2);
    const auto rv = rsrc(vg + v_base, L * dv * 2);
    const auto rrec = rsrc(geo.rec + (long)chain * nchunks * kWybRecBytes, (long)nchunks * kWybRecBytes);
    auto koff = [&](int u) __attribute__((always_inline)) {
      const int p = lane + 64 * u;
      return (uint32_t)(((p / VPR - a.key_shift) * DK + (p % VPR) * 8) * 2);
    };
    auto qoff = [&](int u) __attribute__((always_inline)) {
      const int p = lane + 64 * u;
      return (uint32_t)(((p / VPR) * DK + (p % VPR) * 8) * 2);
    };
    // record j: array ar (0 -H_x hi, 1 lo, 2 H_y hi, 3 lo; 4 -Q_x hi, 5 lo, 6 Q_y hi,
    // 7 lo), row r, this lane's 8 columns
    auto rec_frag = [&](int j, int ar, int r) __attribute__((always_inline)) {
      const uint32_t base = ar < 4 ? 2048u * ar : 8192u + 1024u * (ar - 4);
      return ld128(rrec, (uint32_t)j * kWybRecBytes + base + (uint32_t)((r * 4 + lg) * 16));
    };
    const int vb_t4 = 4 * ((lane & 31) >> 3), vb_i4 = 4 * (lane & 7);
    const uint32_t voff = (lane < 32 && i0 + vb_i4 < dv) ? (uint32_t)((vb_t4 * dv + i0 + vb_i4) * 2) : PARKED;
    const uint32_t V_CHUNK = (uint32_t)(CS * dv * 2);
    uint4 kprev[KP];
#pragma unroll
    for (int u = 0; u < KP; ++u) {
      kprev[u] = make_uint4(0u, 0u, 0u, 0u);
      const int p = lane + 64 * u;
      if (role == 0 && kpg != nullptr && p / VPR == 0)
        kprev[u] = *reinterpret_cast<const uint4*>(kpg + (long)chain * DK + (p % VPR) * 8);
    }
    auto put8 = [&](uint16_t* row, int k0, uint4 val) __attribute__((always_inline)) {
      *reinterpret_cast<uint2*>(row + fpos(k0)) = make_uint2(val.x, val.y);
      *reinterpret_cast<uint2*>(row + fpos(k0 + 4)) = make_uint2(val.z, val.w);
    };
    auto hl_u = [](uint4 h, uint4 l) __attribute__((always_inline)) {
      HL f;
      f.hi = __builtin_bit_cast(bf16x8, h);
      f.lo = __builtin_bit_cast(bf16x8, l);
      return f;
    };
    auto mover = [&](auto rc) __attribute__((always_inline)) {
      constexpr int R = decltype(rc)::value;
      // one register set per ring slot, read by role: w[0..KP) key pieces (role 0);
      // query pieces and values in w[4], w[5] (role 1); -H_x or H_y [2 tile + hi/lo]
      // in w[0..3] and -Q_x or Q_y [hi/lo] in w[4], w[5] (roles 2, 3); g_t of this
      // lane's step and the range flag (role 2)
      static_assert(KP <= 4, "key pieces fit the set");
      struct Set {
        uint4 w[6];
        float g;
        uint32_t flag;
      };
      Set ring0, ring1, ring2, ring3;             // the ring, one variable per slot
      auto slot = [&](auto ic) -> Set& {
        constexpr int i = decltype(ic)::value & 3;
        if constexpr (i == 0) return ring0;
        else if constexpr (i == 1) return ring1;
        else if constexpr (i == 2) return ring2;
        else return ring3;
      };
      auto load = [&](Set& st, int j) __attribute__((always_inline)) {
        if constexpr (R == 0) {
  #pragma unroll
          for (int u = 0; u < KP; ++u) st.w[u] = ld128(rk, koff(u) + (uint32_t)j * KQ_CHUNK);
        } else if constexpr (R == 1) {
  #pragma unroll
          for (int u = 0; u < KP; ++u) st.w[u] = ld128(rq, qoff(u) + (uint32_t)j * KQ_CHUNK);
          uint32_t w[8];
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            const auto val = __builtin_amdgcn_raw_buffer_load_b64(rv, (int)(voff + (uint32_t)j * V_CHUNK + (uint32_t)(e * dv * 2)), 0, 0);
            w[2 * e] = val[0];
            w[2 * e + 1] = val[1];
          }
          st.w[4] = make_uint4(w[0], w[1], w[2], w[3]);
          st.w[5] = make_uint4(w[4], w[5], w[6], w[7]);
        } else {
          constexpr int a0 = R == 2 ? 0 : 2;     // -H_x or H_y
  #pragma unroll
          for (int m = 0; m < 2; ++m)
  #pragma unroll
            for (int h = 0; h < 2; ++h) st.w[2 * m + h] = rec_frag(j, a0 + h, 16 * m + lr);
  #pragma unroll
          for (int h = 0; h < 2; ++h) st.w[4 + h] = rec_frag(j, 4 + a0 + h, lr);
          if constexpr (R == 2) {
            st.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                       rrec, (int)((uint32_t)j * kWybRecBytes + kWybRecGam + 4u * lr), 0, 0));
            st.flag = __builtin_amdgcn_raw_buffer_load_b32(rrec, (int)((uint32_t)j * kWybRecBytes + kWybRecBad), 0, 0);
          }
        }
      };
      auto commit = [&](const Set& st, int j) __attribute__((always_inline)) {
        const int jb = j & 3;
        if constexpr (R == 0) {
  #pragma unroll
          for (int u = 0; u < KP; ++u) {
            const int p = lane + 64 * u;
            const int t = p / VPR, kv = p % VPR;
            put8(&sm.X[jb][t][0], kv * 8, (j == 0 && t == 0 && a.key_shift) ? kprev[u] : st.w[u]);
          }
          // keys transposed: XT[k][t] from X[t][k]; item idx moves a 4 (t) x 4 (k) block
  #pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int idx = lane + 64 * h;
            if (idx < (CS / 4) * (DK / 4)) {
              const int t4 = 4 * (idx % (CS / 4)), k4 = 4 * (idx / (CS / 4));
              const int pk4 = fpos(k4);
              uint32_t w[8];
  #pragma unroll
              for (int e = 0; e < 4; ++e) {
                const uint2 r = *reinterpret_cast<const uint2*>(&sm.X[jb][t4 + e][pk4]);
                w[2 * e] = r.x;
                w[2 * e + 1] = r.y;
              }
  #pragma unroll
              for (int kk = 0; kk < 4; ++kk) {
                const uint32_t sel = (kk & 1) ? 0x07060302u : 0x05040100u;
                const int hh = kk >> 1;
                *reinterpret_cast<uint2*>(&sm.XT[jb][k4 + kk][t4]) =
                    make_uint2(__builtin_amdgcn_perm(w[2 + hh], w[hh], sel), __builtin_amdgcn_perm(w[6 + hh], w[4 + hh], sel));
              }
            }
          }
        } else if constexpr (R == 1) {
  #pragma unroll
          for (int u = 0; u < KP; ++u) {
            const int p = lane + 64 * u;
            put8(&sm.Q[jb][p / VPR][0], (p % VPR) * 8, st.w[u]);
          }
          if (lane < 32) {
            const uint32_t w[8] = {st.w[4].x, st.w[4].y, st.w[4].z, st.w[4].w, st.w[5].x, st.w[5].y, st.w[5].z, st.w[5].w};
  #pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
              const uint32_t sel = (ii & 1) ? 0x07060302u : 0x05040100u;
              const int h = ii >> 1;
              *reinterpret_cast<uint2*>(&sm.YT[jb][vb_i4 + ii][vb_t4]) =
                  make_uint2(__builtin_amdgcn_perm(w[2 + h], w[h], sel), __builtin_amdgcn_perm(w[6 + h], w[4 + h], sel));
            }
          }
        } else if constexpr (R == 2) {
  #pragma unroll
          for (int h = 0; h < 2; ++h) {
  #pragma unroll
            for (int m = 0; m < 2; ++m) *reinterpret_cast<uint4*>(&sm.Hx[jb][h][16 * m + lr][8 * lg]) = st.w[2 * m + h];
            *reinterpret_cast<uint4*>(&sm.Qx[jb][h][lr][8 * lg]) = st.w[4 + h];
          }
          if (lg == 0) sm.gam[jb][lr] = st.g;
          if (lane == 0 && st.flag != 0) sm.bad = 1;
        }
      };
      // role 3: H_y Y and Q_y Y of sub-chunk j (values of blocks j - 1 and j)
      auto fold_y = [&](const Set& st, int j) __attribute__((always_inline)) {
        const int jb = j & 3;
        const HL hy0 = hl_u(st.w[0], st.w[1]), hy1 = hl_u(st.w[2], st.w[3]);
        const HL qy = hl_u(st.w[4], st.w[5]);
  #pragma unroll
        for (int it = 0; it < 2; ++it) {
          const bf16x8 yf = frag_two(&sm.YT[(j - 1) & 3][16 * it + lr][4 * lg], &sm.YT[jb][16 * it + lr][4 * lg]);
  #pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const floatx4 acc = mma2(floatx4{0.f, 0.f, 0.f, 0.f}, mt == 0 ? hy0 : hy1, yf);
            *reinterpret_cast<float4*>(&sm.Ufk[jb][16 * it + lr][16 * mt + 4 * lg]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
          }
          const floatx4 oacc = mma2(floatx4{0.f, 0.f, 0.f, 0.f}, yf, qy);
          *reinterpret_cast<float4*>(&sm.Oy[jb][lr][16 * it + 4 * lg]) = make_float4(oacc[0], oacc[1], oacc[2], oacc[3]);
        }
      };
      // roles 1 and 2: the readout of sub-chunk c for row tile R - 1, from the
      // state waves' partials: o_t = g_t (S_c q_t + (Q_y Y)_t - (Q_x XS_c)_t)
      auto readout = [&](int c) __attribute__((always_inline)) {
        constexpr int rt = R - 1;
        if (i0 + 16 * rt >= dv) return;
        const int cb = c & 1, cs = c & 3;
        floatx4 xs[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          const floatx4 p0 = sm.PX[cb][rt][0][mi][lane], p1 = sm.PX[cb][rt][1][mi][lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) xs[mi][e] = p0[e] + p1[e];
        }
        const HL xsf = hl_x4(xs[0], xs[1]);
        floatx4 oacc = f4x(*reinterpret_cast<const float4*>(&sm.Oy[cs][lr][16 * rt + 4 * lg]));
        const floatx4 p0 = sm.PO[cb][rt][0][lane], p1 = sm.PO[cb][rt][1][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[e] += p0[e] + p1[e];
        oacc = mma3(oacc, xsf, hl_pair(&sm.Qx[cs][0][lr][8 * lg], &sm.Qx[cs][1][lr][8 * lg]));
        const float gt = sm.gam[cs][lr];
        sm.OT[cb][rt][lane] = make_float4(gt * oacc[0], gt * oacc[1], gt * oacc[2], gt * oacc[3]);
      };
      // the first reads: sub-chunks 0..3 (role 3: 0..2, its iteration -2 reads 3)
      load(ring0, 0);
      load(ring1, 1);
      load(ring2, 2);
      if constexpr (R != 3) load(ring3, 3);
      // iteration c = c4 + U; c4 + 2 is a multiple of 4, so the ring slots are constants
      auto iteration = [&](auto uc, int c4) __attribute__((always_inline)) {
        constexpr int U = decltype(uc)::value;
        const int c = c4 + U;
        if (c >= nchunks) return;
        __syncthreads();
        // let the state waves' reads of the partials, the first step of their
        // chain after the barrier, reach LDS before the commits (about 256
        // cycles; measured 1-2% faster at dk = 128, neutral at dk = 64)
        __builtin_amdgcn_s_sleep(4);
        if constexpr (R == 3) {
          Set& st = slot(std::integral_constant<int, U + 3>{});
          if (c + 1 >= 0 && c + 1 < nchunks) fold_y(st, c + 1);
          load(st, c + 5);
        } else {
          Set& st = slot(std::integral_constant<int, U>{});
          if (c + 2 < nchunks) commit(st, c + 2);
          load(st, c + 6);      // the reads go out as soon as their slot is free, before the readout
          if constexpr (R == 1 || R == 2) {
            if (c >= 0) readout(c);
          }
        }
      };
      for (int c4 = -2; c4 < nchunks; c4 += 4) {
        iteration(std::integral_constant<int, 0>{}, c4);
        iteration(std::integral_constant<int, 1>{}, c4);
        iteration(std::integral_constant<int, 2>{}, c4);
        iteration(std::integral_constant<int, 3>{}, c4);
      }
    };
    if (role == 0) mover(std::integral_constant<int, 0>{});
    else if (role == 1) mover(std::integral_constant<int, 1>{});
    else if (role == 2) mover(std::integral_constant<int, 2>{});
    else mover(std::integral_constant<int, 3>{});
    __syncthreads();
  }
  // a chain whose decay products left the range of the chunk algebra: its rows
  // again, exactly, by the recurrence (S_out was left untouched above)
  __syncthreads();
  if (sm.bad) recurrence_rows<DK, ST_NT, B>(chain, i0, dv - i0 < RW ? dv - i0 : RW);
}

template <int DK, bool REG, int B>
hipError_t launch_wyb(const SeqArgs& a, hipStream_t stream) {
  static_assert(sizeof(WybLds<DK>) <= 160 * 1024, "LDS budget");
  WybGeom geo;
  const int nchain = a.batch * a.heads;
  geo.nrbg = (a.dv + RW - 1) / RW;
  geo.remap = (nchain % 8 == 0) ? 1 : 0;
  geo.nchunks = (int)((a.seqlen + CS - 1) / CS);
  const unsigned nblocks = (unsigned)(nchain * geo.nrbg);
  geo.seg_len = 0;
  geo.nseg = 0;
  geo.rec = nullptr;
  hipLaunchKernelGGL((chunk_wyb_kernel<DK, REG, B, false>), dim3(nblocks), dim3(NT), 0, stream, a, geo);
  return hipGetLastError();
}

template <int DK>
hipError_t launch_wyb_dk(const SeqArgs& a, hipStream_t stream) {
  if (a.window == 2) return a.regression ? launch_wyb<DK, true, 2>(a, stream) : launch_wyb<DK, false, 2>(a, stream);
  return a.regression ? launch_wyb<DK, true, 4>(a, stream) : launch_wyb<DK, false, 4>(a, stream);
}

template <int DK, int B>
hipError_t launch_wyb2(const SeqArgs& a, void* ws, hipStream_t stream) {
  static_assert(sizeof(WybStLds<DK>) <= 160 * 1024, "LDS budget");
  WybGeom geo;
  const int nchain = a.batch * a.heads;
  geo.nrbg = (a.dv + RW - 1) / RW;
  geo.remap = (nchain % 8 == 0) ? 1 : 0;
  geo.nchunks = (int)((a.seqlen + CS - 1) / CS);
  geo.rec = static_cast<unsigned char*>(ws);
  // pre-pass: each workgroup prepares a run of sub-chunks of one chain (about one
  // workgroup per compute unit; every run restarts the preparation pipeline)
  const long total = (long)nchain * geo.nchunks;
  int seg = (int)((total + 255) / 256);
  if (seg < 16) seg = 16;
  if (seg > geo.nchunks) seg = geo.nchunks;
  geo.seg_len = seg;
  geo.nseg = (geo.nchunks + seg - 1) / seg;
  hipLaunchKernelGGL((chunk_wyb_kernel<DK, true, B, true>), dim3((unsigned)(nchain * geo.nseg)), dim3(NT), 0,
                     stream, a, geo);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((wyb_state_kernel<DK, B>), dim3((unsigned)(nchain * geo.nrbg)), dim3(ST_NT), 0, stream, a,
                     geo);
  return hipGetLastError();
}

}  // namespace

size_t chunk_wyb2_workspace_bytes(const SeqArgs& a) {
  if (!a.regression || !chunk_wyb_supported(a)) return 0;
  const long nchunks = ((long)a.seqlen + CS - 1) / CS;
  if (nchunks * kWybRecBytes >= (1L << 30)) return 0;   // per-chain buffer range
  return (size_t)a.batch * a.heads * nchunks * kWybRecBytes;
}

hipError_t launch_chunk_wyb2(const SeqArgs& a, void* workspace, hipStream_t stream) {
  if (a.dk == 64) return a.window == 2 ? launch_wyb2<64, 2>(a, workspace, stream) : launch_wyb2<64, 4>(a, workspace, stream);
  if (a.dk == 128) return a.window == 2 ? launch_wyb2<128, 2>(a, workspace, stream) : launch_wyb2<128, 4>(a, workspace, stream);
  return hipErrorInvalidValue;
}

bool chunk_wyb_supported(const SeqArgs& a) {
  const long bytes = (long)a.seqlen * (a.dk > a.dv ? a.dk : a.dv) * 2;
  return (a.window == 2 || a.window == 4) && a.beta_kind != 2 && (a.dk == 64 || a.dk == 128) &&
         a.dv % 4 == 0 && bytes < (1L << 30);
}

// Sliding-window chunk form (window 2 or 4), gains shared by the value rows,
// 16-step sub-chunks whatever the requested chunk.
hipError_t launch_chunk_wyb(const SeqArgs& a, hipStream_t stream) {
  if (a.dk == 64) return launch_wyb_dk<64>(a, stream);
  if (a.dk == 128) return launch_wyb_dk<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace falcon
