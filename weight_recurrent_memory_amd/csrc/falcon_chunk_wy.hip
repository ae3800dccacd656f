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
// W is formed from 16-step blocks: T_bb = (I + M_bb)^-1 by forward substitution,
// N = -T_11 M_10, and with the row scales s folded in (omega for x, zeta for y)
//   W = F [x | y],   F = T diag(s) = [[T_00 S_0, 0], [N T_00 S_0, T_11 S_1]].
// The inner-product family has z_t = zeta_t y_t (no solve).
//
// Structure.  One workgroup = 8 wave64 = one (batch*head) chain x 32 value
// rows; chunks of C = 32 steps.  Waves 0 and 1 ("state waves") each own 16 rows
// of the state: S (fp32) and z never leave their registers; per chunk they run
// S q, z = Ut - Wt S, the carry S <- g (S + Z X^T) and the readout, four small
// matrix-core products, then read the next chunk's operands.  Waves 2..7 prepare
// later chunks, each stage reading only what an earlier iteration wrote, so one
// barrier per chunk suffices:
//   iteration c:  state chunk c | Wt, Ut and q.x of c+2 | keys transposed and
//                 factors T_00, [T_11 | N] of c+3 | Gram and scalars of c+4 |
//                 keys of c+5, queries and values of c+3 to LDS (loaded two
//                 iterations earlier)
// LDS operands that meet a register operand of the state waves are stored in
// the order of that register fragment: within every 32-wide group, positions
// 8g..8g+3 hold indices 4g..4g+3 and 8g+4..8g+7 hold 16+4g..16+4g+3, so every
// fragment is one 16-byte read.  Row strides are 16 mod 64 bytes (measured on the
// whole kernel: 40% fewer LDS bank-conflict cycles than strides of 32 mod 64).
// Non-exact operands are split into bf16 hi + lo (split-bf16, Henry, Tang &
// Heinecke, ARITH 2019): hi*hi + hi*lo + lo*hi with fp32 accumulation.
#include <type_traits>

#include "falcon_device.h"
#include "falcon_exact.h"
#include "falcon_launch.h"
#include "falcon_mma.h"

namespace falcon {
namespace {

constexpr int CS = 32;       // chunk length
constexpr int RW = 32;       // value rows per workgroup
constexpr int NW = 8;
constexpr int NT = 64 * NW;

// position of index k in the fragment order (groups of 32)
__device__ __forceinline__ int fpos(int k) {
  const int kk = k & 31;
  return (k & ~31) + 8 * ((kk & 15) >> 2) + ((kk >> 4) << 2) + (kk & 3);
}

template <int DK>
struct WyLds {
  static constexpr int XR = DK + 8;      // bf16 row: DK (fragment order) + pad
  static constexpr int TR = CS + 8;      // bf16 row over steps
  uint16_t X[4][CS][XR];                 // keys by chunk & 3, k in fragment order
  uint16_t Q[4][CS][XR];                 // queries by chunk & 3
  uint16_t XT[4][DK][TR];                // keys transposed, t in fragment order
  uint16_t YT[2][RW][TR];                // values transposed, t in fragment order
  uint16_t Phi[2][CS][TR];               // q.x (s <= t), s in fragment order
  uint16_t Plo[2][CS][TR];
  uint16_t Whi[2][CS][XR];               // Wt^T[t][k], k in fragment order
  uint16_t Wlo[2][CS][XR];
  float SA[2][2][16][CS + 4];            // [T_00 | 0], [T_11 | -T_11 M_10], fragment order
  float TT[2][16][16 + 4];               // T_00^T (row = column of T_00)
  float G[2][CS][CS + 4];                // Gram (whole 32 x 32)
  float Ut[2][RW][CS + 4];               // Ut[i][t]
  float beta[4][CS];                     // gains by chunk & 3
  float knorm[4][CS];                    // squared key norms by chunk & 3
  alignas(16) float gam[8][CS];          // per-step scalars by chunk & 7
  alignas(16) float gm1[8][CS];
  alignas(16) float zeta[8][CS];
  alignas(16) float omega[8][CS];
  int bad;                               // some chunk's decay products left the range
};

struct WyGeom {
  int nrbg;
  int remap;
  int nchunks;
};

// split-bf16 product: the three passes chain through the accumulator (the matrix
// core forwards it between back-to-back products), small terms first
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
// acc + g(lane N of this 16-lane row) * r, the row broadcast folded into the
// multiply-add as a DPP operand.  g is only ever loaded from LDS (never written by
// the vector ALU), so the DPP read needs no wait states.
template <int N>
__device__ __forceinline__ float fmac_row_bcast(float acc, float g, float r) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(g), "v"(r), "i"(N));
  return acc;
}
// forward substitution of (I + M) x = rhs over one 16-step block from step M on,
// M = diag(om) L(G): lane m of each 16-lane row holds row m of the block's Gram
// matrix in g[], so entry G[m][r] (= G[r][m]) is a row broadcast from lane m
template <int M>
__device__ __forceinline__ void sweep_from(float (&rhs)[16], float (&acc)[16], const float (&g)[16], const float (&om)[16]) {
  rhs[M] = __builtin_fmaf(-om[M], acc[M], rhs[M]);
#pragma unroll
  for (int r = M + 1; r < 16; ++r) acc[r] = fmac_row_bcast<M>(acc[r], g[r], rhs[M]);
  if constexpr (M < 15) sweep_from<M + 1>(rhs, acc, g, om);
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
  static_assert(DK % 32 == 0 && DK <= 64, "dk in {32, 64}");
  static_assert((CS / 4) * (RW / 4) == 64 && CS <= 64, "values and gains: one wave");
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
  const long L = a.seqlen;
  const long qk_base = (long)chain * L * DK;
  const long v_base = (long)chain * L * dv;
  const int nchunks = geo.nchunks;
  auto steps = [&](int j) __attribute__((always_inline)) {
    const long t0 = (long)j * CS;
    return (int)((L - t0) < CS ? (L - t0) : CS);
  };

  // ---------------- zero the fragment slots no stage writes ----------------
  if (tid == 0) sm.bad = 0;
  for (int idx = tid; idx < 2 * 2 * 16 * (CS + 4); idx += NT) (&sm.SA[0][0][0][0])[idx] = 0.0f;
  for (int idx = tid; idx < 2 * CS * SM::TR; idx += NT) {
    (&sm.Phi[0][0][0])[idx] = 0;
    (&sm.Plo[0][0][0])[idx] = 0;
  }

  // ---------------- global loads and their commits to LDS ----------------
  // Waves 2, 3, 6, 7 move keys and queries (one 16-byte piece of a row per
  // thread), wave 4 values and gains.  A load is issued two iterations before its
  // commit, into one of two register sets used alternately.  The loads go through
  // per-chain buffer resources: a piece past the end of the sequence (or before
  // its start, or a padding lane's, whose offset is parked above 2^31) reads 0,
  // so every prefetch issues the same loads in the same order and the wait before
  // a commit counts only the loads of its own set.  The per-lane offsets are fixed;
  // a chunk adds a uniform stride.
  static_assert(CS * VPR <= 256, "one key piece and one query piece per thread");
  struct KQSet {            // one 16-byte piece of a key row and of a query row
    uint4 k, q;
  };
  struct VBSet {            // a 4 (steps) x 4 (value rows) block and one gain
    uint4 v, v2;
    uint32_t b;
  };
  constexpr int BUF_WORD3 = 0x00020000;     // raw 32-bit buffer, range checked
  constexpr uint32_t PARKED = 0xC0000000u;  // offset that is always out of range
  auto rsrc = [](const void* base, long bytes) __attribute__((always_inline)) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, BUF_WORD3);
  };
  // waves w and w + 4 share a SIMD (and its matrix core): the state waves 0, 1 are
  // paired with the VALU/LDS roles on waves 4, 5; the matrix-core roles take 2, 3, 6, 7
  const int kq_slot = wave == 2 ? 0 : wave == 3 ? 1 : wave == 6 ? 2 : 3;
  const int kt_id = 64 * kq_slot + lane;   // 0..255 on waves 2, 3, 6, 7
  const int vt_id = lane;                  // 0..63 on wave 4
  auto live_chunk = [&](int j) __attribute__((always_inline)) { return j >= 0 && j < nchunks; };
  // key and query piece of this thread: step kq_t of the chunk, k = 8 kq_kv ..
  const bool kq_in = kt_id < CS * VPR;     // uniform per wave
  const int kq_t = kt_id / VPR, kq_kv = kt_id % VPR;
  const auto rk = rsrc(kg + qk_base, L * DK * 2);
  const auto rq = rsrc(qg + qk_base, L * DK * 2);
  // key x_g = k_{g-s}: row g - s (with s = 1 the first step of the sequence reads 0
  // there and takes k_prev at commit)
  const uint32_t koff = kq_in ? (uint32_t)(((kq_t - a.key_shift) * DK + kq_kv * 8) * 2) : PARKED;
  const uint32_t qoff = kq_in ? (uint32_t)((kq_t * DK + kq_kv * 8) * 2) : PARKED;
  constexpr uint32_t KQ_CHUNK = CS * DK * 2;
  auto ld128 = [](__amdgpu_buffer_rsrc_t r, uint32_t off) __attribute__((always_inline)) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  // keys of chunk jk, queries of chunk jq
  auto prefetch_kq = [&](KQSet& p, int jk, int jq) __attribute__((always_inline)) {
    p.k = ld128(rk, koff + (uint32_t)jk * KQ_CHUNK);
    p.q = ld128(rq, qoff + (uint32_t)jq * KQ_CHUNK);
  };
  uint4 kprev = {0u, 0u, 0u, 0u};          // x_0 of the chain (0 on a fresh sequence)
  if (kpg != nullptr && kq_in && kq_t == 0 && wave >= 2 && wave != 4 && wave != 5)
    kprev = *reinterpret_cast<const uint4*>(kpg + (long)chain * DK + kq_kv * 8);
  // 8 consecutive k (k0 % 8 == 0) -> two 4-groups at their fragment positions
  auto put8 = [&](uint16_t* row, int k0, uint4 val) __attribute__((always_inline)) {
    *reinterpret_cast<uint2*>(row + fpos(k0)) = make_uint2(val.x, val.y);
    *reinterpret_cast<uint2*>(row + fpos(k0 + 4)) = make_uint2(val.z, val.w);
  };
  // The keys' squared norms are formed here, from the registers: packed bf16 dot
  // products, then a sum over the VPR threads of a row by DPP row shifts (the
  // row's last thread ends with the total).
  auto commit_kq = [&](const KQSet& p, int jk, int jq) __attribute__((always_inline)) {
    if (kq_in) {
      if (live_chunk(jk)) {
        const uint4 kv = (jk == 0 && kq_t == 0 && a.key_shift) ? kprev : p.k;
        put8(&sm.X[jk & 3][kq_t][0], kq_kv * 8, kv);
        float part = 0.0f;
        const uint32_t w4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 v = __builtin_bit_cast(bf16x2, w4[e]);
          part = __builtin_amdgcn_fdot2_f32_bf16(v, v, part, false);
        }
        part += dpp_shr<1>(part, 0.0f);
        part += dpp_shr<2>(part, 0.0f);
        if constexpr (VPR == 8) part += dpp_shr<4>(part, 0.0f);
        if (kq_kv == VPR - 1) sm.knorm[jk & 3][kq_t] = part;
      }
      if (live_chunk(jq)) put8(&sm.Q[jq & 3][kq_t][0], kq_kv * 8, p.q);
    }
  };
  // a 4 (steps) x 4 (value rows) block of wave 4's lane: steps t4.., value rows i4..
  const int vb_i4 = 4 * (vt_id % (RW / 4)), vb_t4 = 4 * (vt_id / (RW / 4));
  const auto rv = rsrc(vg + v_base, L * dv * 2);
  const auto rb = a.beta_kind == 1 ? rsrc(bg + (long)chain * L, L * 2) : rsrc(vg, 0);
  const uint32_t voff = i0 + vb_i4 < dv ? (uint32_t)((vb_t4 * dv + i0 + vb_i4) * 2) : PARKED;
  const uint32_t V_CHUNK = (uint32_t)(CS * dv * 2);
  // gains of chunk jb, values of chunk jv
  auto prefetch_vb = [&](VBSet& p, int jb, int jv) __attribute__((always_inline)) {
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto val = __builtin_amdgcn_raw_buffer_load_b64(rv, (int)(voff + (uint32_t)jv * V_CHUNK + (uint32_t)(e * dv * 2)), 0, 0);
      w[2 * e] = val[0];
      w[2 * e + 1] = val[1];
    }
    p.v = make_uint4(w[0], w[1], w[2], w[3]);
    p.v2 = make_uint4(w[4], w[5], w[6], w[7]);
    p.b = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)((uint32_t)vt_id * 2 + (uint32_t)jb * (CS * 2)), 0, 0);
  };
  auto commit_vb = [&](const VBSet& p, int jb, int jv) __attribute__((always_inline)) {
    if (live_chunk(jv)) {
      // step t4+e holds values i4..i4+3 in (w[2e], w[2e+1]); value row i4+ii takes
      // the low (ii even) or high (ii odd) halves of w[2e + ii/2], e = 0..3
      const uint32_t w[8] = {p.v.x, p.v.y, p.v.z, p.v.w, p.v2.x, p.v2.y, p.v2.z, p.v2.w};
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const uint32_t sel = (ii & 1) ? 0x07060302u : 0x05040100u;
        const int h = ii >> 1;
        *reinterpret_cast<uint2*>(&sm.YT[jv & 1][vb_i4 + ii][fpos(vb_t4)]) =
            make_uint2(__builtin_amdgcn_perm(w[2 + h], w[h], sel), __builtin_amdgcn_perm(w[6 + h], w[4 + h], sel));
      }
    }
    if (live_chunk(jb) && vt_id < CS)
      sm.beta[jb & 3][vt_id] = a.beta_kind == 0 ? a.beta : bf16_to_f32((uint16_t)p.b);
  };

  // eta_t = beta_t / (eps + ||x_t||^2), a_t = 1 - eta_t lambda; padded steps and
  // the fresh-sequence first step (x_1 = 0 on S_0 = 0) take eta = 0, a = 1.
  // One wave: lane = step t (mod 32); the squared key norms were formed at commit.
  auto scalars = [&](int j) __attribute__((always_inline)) {
    const int sb = j & 7;
    const long t0 = (long)j * CS;
    const int c = steps(j);
    const int t = lane & 31;
    const bool live = t < c && !(t0 + t == 0 && kpg == nullptr && a.key_shift);
    const float nrm = sm.knorm[j & 3][t];
    const float bv = sm.beta[j & 3][t];
    float eta = 0.0f, dec = 1.0f;
    if (live) {
      eta = bv * __builtin_amdgcn_rcpf(a.eps + nrm);
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
    const float row0 = lane_value(gsc, 15);
    if (lane >= 16) gsc *= row0;
    const float gprev = dpp_shr<1>(gsc, lane == 16 ? row0 : 1.0f);
    if (__builtin_amdgcn_ballot_w64(gauge_out_of_range(gsc, dec)) != 0 && lane == 0) sm.bad = 1;
    if (lane < CS) {
      const float z = eta * __builtin_amdgcn_rcpf(gsc);
      sm.gam[sb][t] = gsc;
      sm.gm1[sb][t] = gprev;
      sm.zeta[sb][t] = z;
      sm.omega[sb][t] = z * gprev;
    }
  };

  // 16-row fragments of a key or query block: rows 16 b + lr, all k
  struct RowFrags {
    bf16x8 f[2][NKS];
  };
  auto row_frags = [&](const uint16_t (*rows)[SM::XR]) __attribute__((always_inline)) {
    RowFrags r;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) r.f[b][ks] = frag_bf16(&rows[16 * b + lr][32 * ks + 8 * lg]);
    return r;
  };
  // 16x16 product tile sum_k A[16 ba + .][k] B[16 bb + .][k] (exact bf16 operands)
  auto tile_dot = [&](const RowFrags& A, int ba, const RowFrags& B, int bb) __attribute__((always_inline)) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks & 1) acc2 = mfma16(A.f[ba][ks], B.f[bb][ks], acc2);
      else acc = mfma16(A.f[ba][ks], B.f[bb][ks], acc);
    }
    return acc + acc2;
  };
  // Gram of chunk j: G[t][s] = x_t . x_s, all four 16x16 tiles (lane: 4 consecutive s of one t)
  auto gram_store = [&](int j, const RowFrags& X) __attribute__((always_inline)) {
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj) {
        const floatx4 acc = tile_dot(X, tj, X, ti);
        *reinterpret_cast<float4*>(&sm.G[j & 1][16 * ti + lr][16 * tj + 4 * lg]) =
            make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
  };
  // q.x of chunk j: P[t][s] = q_t . x_s for s <= t, split, s in fragment order
  // (tiles (0,0), (1,0), (1,1); tile (0,1) stays zero)
  auto qx_store = [&](int j, const RowFrags& X, const RowFrags& Qf) __attribute__((always_inline)) {
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj <= ti; ++tj) {
        const floatx4 acc = tile_dot(X, tj, Qf, ti);
        const int t = 16 * ti + lr;
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = (16 * tj + 4 * lg + e <= t) ? acc[e] : 0.0f;
        const int p = 8 * lg + 4 * tj;
        store_split4(&sm.Phi[j & 1][t][p], &sm.Plo[j & 1][t][p], pv);
      }
  };
  // keys transposed: XT[k][t] from X[t][k]; item idx moves a 4 (t) x 4 (k) block
  auto transpose_keys = [&](int j, int idx) __attribute__((always_inline)) {
    const int xb = j & 3;
    if (idx < (CS / 4) * (DK / 4)) {
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
  // wave: lanes 0..15 the columns of T_00, lanes 16..47 the 32 columns of block 1
  // (each 16-lane row holds one block; lanes 48..63 repeat block 1).
  auto solve_factors = [&](int j) __attribute__((always_inline)) {
    const int gb = j & 1, sb = j & 7;
    const int blk = lane < 16 ? 0 : 1;
    const int col = lane < 16 ? lane : (lane < 48 ? lane - 16 : 0);   // 0..15 / 0..31
    const int u0 = 16 * blk;
    float rhs[16], acc[16];               // rhs becomes the solution in place
    float om[16], g[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 o4 = *reinterpret_cast<const float4*>(&sm.omega[sb][u0 + 4 * q]);
      om[4 * q] = o4.x; om[4 * q + 1] = o4.y; om[4 * q + 2] = o4.z; om[4 * q + 3] = o4.w;
      const float4 g4 = *reinterpret_cast<const float4*>(&sm.G[gb][u0 + lr][u0 + 4 * q]);
      g[4 * q] = g4.x; g[4 * q + 1] = g4.y; g[4 * q + 2] = g4.z; g[4 * q + 3] = g4.w;
    }
    // -M_10[:, c'] = -omega_{16+m} G[16+m][c'] = -omega_{16+m} G[c'][16+m]
    const int cp = (blk == 1 && col >= 16) ? col - 16 : 0;
    float4 gv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) gv[q] = *reinterpret_cast<const float4*>(&sm.G[gb][cp][16 + 4 * q]);
    const bool ncol = blk == 1 && col >= 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float gq[4] = {gv[q].x, gv[q].y, gv[q].z, gv[q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 4 * q + e;
        rhs[m] = ncol ? -om[m] * gq[e] : (m == col ? 1.0f : 0.0f);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    asm volatile("s_nop 4");              // any EXEC write settles before the DPP sweep
    sweep_from<0>(rhs, acc, g, om);
    if (lane < 48) {
      const int cc = col & 15;
      const int p = 8 * (cc >> 2) + ((col >> 4) << 2) + (cc & 3);
#pragma unroll
      for (int m = 0; m < 16; ++m) sm.SA[gb][blk][m][p] = rhs[m];
    }
    if (lane < 16) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(&sm.TT[gb][lane][4 * q]) = make_float4(rhs[4 * q], rhs[4 * q + 1], rhs[4 * q + 2], rhs[4 * q + 3]);
    }
  };
  // Blocked solve of chunk j as one product.  With the row scales s (omega for
  // the keys, zeta for the values) folded into the factor,
  //   W = F [x | y],   F = T diag(s) = [[T_00 S_0, 0], [N T_00 S_0, T_11 S_1]],
  // N = -T_11 M_10.  Lane (lr, lg) builds rows lr (block 0) and 16 + lr (block 1)
  // of F at fragment slots 8 lg.. (steps 4 lg..) and 8 lg + 4.. (steps 16 + 4 lg..);
  // N T_00 is one small split-bf16 product.  Key tiles give Wt^T rows (lane: 4
  // consecutive k of one t), value tiles Ut rows (lane: 4 consecutive t of one i).
  struct SolveOps {
    float4 s0, s1, t00, t11, n, tt;
    bf16x8 op[2];            // the x or y fragments of the wave's two tiles
  };
  struct FRows {
    HL f[2];
  };
  auto solve_load = [&](int j, bool keys, int tile0, int tile1) __attribute__((always_inline)) {
    const int gb = j & 1, sb = j & 7, xb = j & 3;
    SolveOps o;
    const float* sc = keys ? sm.omega[sb] : sm.zeta[sb];
    o.s0 = *reinterpret_cast<const float4*>(sc + 4 * lg);
    o.s1 = *reinterpret_cast<const float4*>(sc + 16 + 4 * lg);
    o.t00 = *reinterpret_cast<const float4*>(&sm.SA[gb][0][lr][8 * lg]);
    o.t11 = *reinterpret_cast<const float4*>(&sm.SA[gb][1][lr][8 * lg]);
    o.n = *reinterpret_cast<const float4*>(&sm.SA[gb][1][lr][8 * lg + 4]);
    o.tt = *reinterpret_cast<const float4*>(&sm.TT[gb][lr][4 * lg]);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int tile = e ? tile1 : tile0;
      o.op[e] = keys ? frag_bf16(&sm.XT[xb][16 * tile + lr][8 * lg]) : frag_bf16(&sm.YT[gb][16 * tile + lr][8 * lg]);
    }
    return o;
  };
  auto factor_rows = [&](const SolveOps& o) __attribute__((always_inline)) {
    const float z4[4] = {0.f, 0.f, 0.f, 0.f};
    const float av[4] = {o.tt.x, o.tt.y, o.tt.z, o.tt.w};
    const float bv[4] = {o.n.x, o.n.y, o.n.z, o.n.w};
    // (T_00^T N^T)[c][m] with c = 4 lg + e, m = lr: the lane gets (N T_00)[lr][4 lg + e]
    const floatx4 p = mma3(floatx4{0.f, 0.f, 0.f, 0.f}, hl_two(av, z4), hl_two(bv, z4));
    const float f0[4] = {o.t00.x * o.s0.x, o.t00.y * o.s0.y, o.t00.z * o.s0.z, o.t00.w * o.s0.w};
    const float f1a[4] = {p[0] * o.s0.x, p[1] * o.s0.y, p[2] * o.s0.z, p[3] * o.s0.w};
    const float f1b[4] = {o.t11.x * o.s1.x, o.t11.y * o.s1.y, o.t11.z * o.s1.z, o.t11.w * o.s1.w};
    FRows r;
    r.f[0] = hl_two(f0, z4);
    r.f[1] = hl_two(f1a, f1b);
    return r;
  };
  auto solve_tile = [&](int j, bool keys, int tile, const FRows& r, const bf16x8& op) __attribute__((always_inline)) {
    const int gb = j & 1;
    const floatx4 zacc = {0.f, 0.f, 0.f, 0.f};
    if (keys) {
      const int p = fpos(16 * tile + 4 * lg);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const floatx4 w = mma2(zacc, op, r.f[tt]);        // Wt^T[16 tile + 4 lg + e][16 tt + lr]
        const float f[4] = {w[0], w[1], w[2], w[3]};
        store_split4(&sm.Whi[gb][16 * tt + lr][p], &sm.Wlo[gb][16 * tt + lr][p], f);
      }
    } else {
      float* u = &sm.Ut[gb][16 * tile + lr][0];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const floatx4 w = mma2(zacc, r.f[tt], op);        // Ut[16 tile + lr][16 tt + 4 lg + e]
        *reinterpret_cast<float4*>(u + 16 * tt + 4 * lg) = make_float4(w[0], w[1], w[2], w[3]);
      }
    }
  };
  // inner-product family: z_t = zeta_t y_t, kept where the regression keeps Ut;
  // item idx covers 4 steps of one value row
  auto zeta_y = [&](int j, int idx) __attribute__((always_inline)) {
    const int gb = j & 1, sb = j & 7;
    if (idx < RW * (CS / 4)) {
      const int i = idx / (CS / 4), t4 = 4 * (idx % (CS / 4));
      const uint2 yb = *reinterpret_cast<const uint2*>(&sm.YT[gb][i][fpos(t4)]);
      const float4 z = *reinterpret_cast<const float4*>(&sm.zeta[sb][t4]);
      *reinterpret_cast<float4*>(&sm.Ut[gb][i][t4]) =
          make_float4(z.x * __uint_as_float(yb.x << 16), z.y * __uint_as_float(yb.x & 0xFFFF0000u),
                      z.z * __uint_as_float(yb.y << 16), z.w * __uint_as_float(yb.y & 0xFFFF0000u));
    }
  };

  // The state waves and the preparation waves run separate loops with the same
  // barrier count (one per iteration), so neither carries the other's registers.
  // iterations c = -5 .. cend-1 (an even count, for the twice-unrolled loops)
  const int cend = nchunks + ((nchunks + 5) & 1);
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
    // The operands of chunk c+1 (written two or more iterations earlier) are read
    // at the end of iteration c, while the barrier is pending.
    struct StateOps {
      bf16x8 qf[2][NKS], xf[NKT];
      HL wf[2][NKS], pf[2];
      float4 ut4[2];
      float gt[2], gC;
    };
    auto load_ops = [&](int j) __attribute__((always_inline)) {
      StateOps o;
      const int cb = j & 1, xb = j & 3, sb = j & 7;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          if constexpr (REG)
            o.wf[tt][ks] = hl_pair(&sm.Whi[cb][16 * tt + lr][32 * ks + 8 * lg], &sm.Wlo[cb][16 * tt + lr][32 * ks + 8 * lg]);
          o.qf[tt][ks] = frag_bf16(&sm.Q[xb][16 * tt + lr][32 * ks + 8 * lg]);
        }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) o.ut4[tt] = *reinterpret_cast<const float4*>(&sm.Ut[cb][16 * rt + lr][16 * tt + 4 * lg]);
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) o.xf[kt] = frag_bf16(&sm.XT[xb][16 * kt + lr][8 * lg]);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        o.pf[tt] = hl_pair(&sm.Phi[cb][16 * tt + lr][8 * lg], &sm.Plo[cb][16 * tt + lr][8 * lg]);
        o.gt[tt] = sm.gam[sb][16 * tt + lr];
      }
      o.gC = sm.gam[sb][CS - 1];
      return o;
    };
    StateOps ops;
    // output row t of the current chunk, value columns i0 + 16 rt + 4 lg .. (t = lr here)
    float* orow = a.o + v_base + (long)lr * dv + i0 + 16 * rt + 4 * lg;
    for (int c = -5; c < cend; ++c) {
      if (state_wave && c >= 0 && c < nchunks) {
        // ---- state chain of chunk c (registers) ----
        const long t0 = (long)c * CS;
        floatx4 oacc[2], zacc[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          oacc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
          zacc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            if constexpr (REG) zacc[tt] = mma3(zacc[tt], ops.wf[tt][ks], sf[ks]);   // (Wt^T S)[t][i]
            oacc[tt] = mma2(oacc[tt], sf[ks], ops.qf[tt][ks]);                      // (S q)[i][t]
          }
        }
        // z[t][i] = Ut[i][t] - (Wt^T S)[t][i]; lane: t = 16 tt + 4 lg + e, i = lr
        float z[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          z[tt][0] = ops.ut4[tt].x - zacc[tt][0];
          z[tt][1] = ops.ut4[tt].y - zacc[tt][1];
          z[tt][2] = ops.ut4[tt].z - zacc[tt][2];
          z[tt][3] = ops.ut4[tt].w - zacc[tt][3];
        }
        const HL zf = hl_two(z[0], z[1]);                               // rows i, t in fragment order
        // carry: S[i][k] <- g_{C-1} (S[i][k] + sum_t z[i][t] x_t[k])
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          const floatx4 cacc = mma2(floatx4{sv[kt][0], sv[kt][1], sv[kt][2], sv[kt][3]}, ops.xf[kt], zf);
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[kt][e] = ops.gC * cacc[e];
        }
        // readout: o[t][i] = g_t ((S q)[i][t] + sum_{s<=t} z[i][s] (q_t . x_s))
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          oacc[tt] = mma3(oacc[tt], zf, ops.pf[tt]);
          const float gt = ops.gt[tt];
          if (t0 + 16 * tt + lr < L)
            *reinterpret_cast<float4*>(orow + 16 * tt * dv) =
                make_float4(gt * oacc[tt][0], gt * oacc[tt][1], gt * oacc[tt][2], gt * oacc[tt][3]);
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) sf[ks] = hl_two(sv[2 * ks], sv[2 * ks + 1]);
        orow += CS * dv;
      }
      if (state_wave && c + 1 >= 0 && c + 1 < nchunks) ops = load_ops(c + 1);
      __syncthreads();
    }
    if (state_wave && a.S_out && !sm.bad) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
        *reinterpret_cast<float4*>(a.S_out + ((long)chain * dv + i0 + 16 * rt + lr) * DK + 16 * kt + 4 * lg) =
            make_float4(sv[kt][0], sv[kt][1], sv[kt][2], sv[kt][3]);
    }
  } else {
    // ---------------- preparation waves ----------------
    // iteration c:  wave 2  Gram of c+4, q.x of c+2 (inner-product family:
    //                       q.x of c+2, keys of c+3 transposed)
    //               wave 3  Wt tiles 0, 1 of c+2    wave 6  Wt tiles 2, 3 of c+2
    //               wave 7  Ut tiles of c+2
    //               waves 2, 3, 6, 7  commit keys of c+5, queries of c+3
    //               wave 4  scalars of c+4, keys of c+3 transposed (regression
    //                       family), commit gains of c+5 and values of c+3
    //               wave 5  factors of c+3 (inner-product family: part of z of c+2)
    // A wave reads its LDS operands first, then commits, then computes (the LDS
    // round trip overlaps the commit).  Global loads are issued two iterations
    // before their commit, into two register sets used alternately.  Each role
    // runs its own loop (same barrier count), so it carries only its registers.
    // keys and queries move on waves 2, 3, 6, 7 inside their role's own loop
    auto kq_loop = [&](auto&& body) __attribute__((always_inline)) {
      KQSet ps0, ps1;
      prefetch_kq(ps0, 0, -2);
      prefetch_kq(ps1, 1, -1);
      __syncthreads();
      for (int c = -5; c < cend; c += 2) {
        body(c, [&]() __attribute__((always_inline)) {
          commit_kq(ps0, c + 5, c + 3);
          prefetch_kq(ps0, c + 7, c + 5);
        });
        __syncthreads();
        body(c + 1, [&]() __attribute__((always_inline)) {
          commit_kq(ps1, c + 6, c + 4);
          prefetch_kq(ps1, c + 8, c + 6);
        });
        __syncthreads();
      }
    };
    if (wave == 2) {
      kq_loop([&](int c, auto&& move) __attribute__((always_inline)) {
        const RowFrags xg = row_frags(sm.X[(c + 4) & 3]);
        const RowFrags xq = row_frags(sm.X[(c + 2) & 3]);
        const RowFrags qq = row_frags(sm.Q[(c + 2) & 3]);
        move();
        if (REG && live_chunk(c + 4)) gram_store(c + 4, xg);
        if (live_chunk(c + 2)) qx_store(c + 2, xq, qq);
        if constexpr (!REG) {
          if (live_chunk(c + 3)) {
            transpose_keys(c + 3, lane);
            transpose_keys(c + 3, 64 + lane);
          }
        }
      });
    } else if (wave != 4 && wave != 5) {
      kq_loop([&](int c, auto&& move) __attribute__((always_inline)) {
        if constexpr (REG) {
          const bool keys = wave != 7;
          const int t0 = keys ? (wave == 3 ? 0 : 2) : 0;   // first tile of the pair
          const bool two = keys ? (t0 + 1 < NKT) : (nrb > 1);
          const int lt0 = (!keys || t0 < NKT) ? t0 : 0;   // dk = 32: wave 6 has no key tiles
          const SolveOps o = solve_load(c + 2, keys, lt0, two ? lt0 + 1 : lt0);
          move();
          if (live_chunk(c + 2) && (!keys || t0 < NKT)) {
            const FRows r = factor_rows(o);
            solve_tile(c + 2, keys, t0, r, o.op[0]);
            if (two) solve_tile(c + 2, keys, t0 + 1, r, o.op[1]);
          }
        } else {
          move();
          if (live_chunk(c + 2)) zeta_y(c + 2, 64 * (kq_slot - 1) + lane);      // waves 3, 6, 7: items 0..191
        }
      });
    } else if (wave == 4) {
      VBSet ps0, ps1;
      prefetch_vb(ps0, 0, -2);
      prefetch_vb(ps1, 1, -1);
      __syncthreads();
      auto iteration = [&](int c, VBSet& cur) __attribute__((always_inline)) {
        commit_vb(cur, c + 5, c + 3);
        prefetch_vb(cur, c + 7, c + 5);
        if (c + 4 >= 0 && c + 4 < nchunks) scalars(c + 4);
        // regression family: the key transposes leave wave 2 (Gram and q.x, on
        // the SIMD of a solve-tile wave) for this light wave (measured 0.5-2% on
        // 8x12x2048x64); in the inner-product family wave 2 has no Gram and this
        // wave's SIMD carries the critical state wave, so they stay on wave 2
        if constexpr (REG) {
          if (live_chunk(c + 3)) {
            transpose_keys(c + 3, lane);
            transpose_keys(c + 3, 64 + lane);
          }
        }
      };
      for (int c = -5; c < cend; c += 2) {
        iteration(c, ps0);
        __syncthreads();
        iteration(c + 1, ps1);
        __syncthreads();
      }
    } else {
      __syncthreads();
      for (int c = -5; c < cend; ++c) {
        if constexpr (REG) {
          if (c + 3 >= 0 && c + 3 < nchunks) solve_factors(c + 3);
        } else {
          if (c + 2 >= 0 && c + 2 < nchunks) zeta_y(c + 2, 192 + lane);
        }
        __syncthreads();
      }
    }
  }
  // a chain whose decay products left the range of the chunk algebra: its rows
  // again, exactly, by the recurrence (the state was left untouched above)
  __syncthreads();
  if (sm.bad) recurrence_rows<DK, NT, 1>(chain, i0, dv - i0 < RW ? dv - i0 : RW);
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
  // per-chain key, query and value blocks addressed by 32-bit buffer offsets
  const long bytes = (long)a.seqlen * (a.dk > a.dv ? a.dk : a.dv) * 2;
  return a.window == 1 && a.beta_kind != 2 && (a.dk == 32 || a.dk == 64) && bytes < (1L << 30);
}

// Window-1 chunk form with gains shared by the value rows, 32-step chunks.
hipError_t launch_chunk_wy(const SeqArgs& a, hipStream_t stream) {
  if (a.dk == 32) return a.regression ? launch_wy<32, true>(a, stream) : launch_wy<32, false>(a, stream);
  if (a.dk == 64) return a.regression ? launch_wy<64, true>(a, stream) : launch_wy<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace falcon
