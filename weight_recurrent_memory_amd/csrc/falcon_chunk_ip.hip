// falcon_chunk_ip.hip - chunk-parallel forward of the inner-product family
// (Falcon-1A, Falcon-3A: any window B <= 16) with gains shared by the value rows
// (scalar or per-token beta), dk in {64, 128}, bf16 inputs.
//
// Method: explainer of arXiv 2608.27763, section 核心方法 §3 (chunk-parallel form;
// the inner-product write of the A variants) and the 163.com article, section 02
// (2) (only the fixed-size state crosses chunks).  Unrolling the inner-product
// rule S_t = a_t S_{t-1} + eta_t sum_{j in W_t} y_j x_j^T over a chunk that starts
// from S0 (steps t = 0..C-1, samples j, window W_t = {t-B+1..t}):
//   S_t = g_t [S0 + sum_j c_{j,t} y_j x_j^T],   g_t = prod_{r<=t} a_r,
//   c_{j,t} = sum over the steps s <= t whose window holds j of zeta_s
//           = Z(min(j+B-1, t)) - Z(max(j, 0) - 1),   zeta = eta / g, Z = prefix sum,
// so  o_t = g_t [S0 q_t + sum_j c_{j,t} (x_j . q_t) y_j]  and
//     S_C = g_{C-1} [S0 + sum_j c_{j,C-1} y_j x_j^T].
// No triangular system appears, and the state enters a chunk only through
// S0 q_t and one scaled add: the serial part is elementwise, everything else is
// products on the matrix cores.
//
// Structure.  One workgroup = 8 wave64 = one (batch*head) chain x 32 value rows;
// 64-step chunks over a key tile of 80 rows (the 16 samples before the chunk,
// which hold the window's reach back, then the chunk's 64).  Waves 0..3 own the
// state, S^T tiles in registers (row tile w & 1, dk half w >> 1): per chunk they
// form their S0 q partial sums (to LDS) and the carry
// S <- g_{C-1} (S + X^T diag(c_{., C-1}) Y).  Waves 4..7 own a 16-step tile of
// the readout (one specialised code path each): P^T = X Q^T over the key tiles
// up to the diagonal, scaled by c, then Y^T (c o P)^T.  Before the mid-chunk
// barrier every thread also forms the squared-norm partial sums of the next
// chunk's keys from its prefetched registers; after it the readout waves add
// the state partials, scale by g_t and store o, every thread commits the next
// chunk to LDS (the last 16 keys slide into the halo rows) and one wave forms
// the next chunk's scalars (g, the prefix sums of zeta, c_{., C-1}; double
// buffered) for all waves.  Loads run two chunks ahead through per-chain buffer
// resources.  Exact bf16 inputs (q, k, v) meet fp32 values (S, c o P, c y) as
// split-bf16 (hi + lo, two passes; Henry, Tang & Heinecke, ARITH 2019).
#include <type_traits>

#include "falcon_device.h"
#include "falcon_exact.h"
#include "falcon_launch.h"
#include "falcon_mma.h"

namespace falcon {
namespace {

constexpr int IC = 64;         // steps per chunk
constexpr int IK = IC + 16;    // key rows: the 16 samples before the chunk, then its 64
constexpr int IRB = 32;        // value rows per workgroup
constexpr int INW = 8;
constexpr int INT = 64 * INW;

__device__ __forceinline__ int ip_fpos(int k) {
  const int kk = k & 31;
  return (k & ~31) + 8 * ((kk & 15) >> 2) + ((kk >> 4) << 2) + (kk & 3);
}

template <int DK>
struct IpLds {
  static constexpr int XR = DK + 16;   // bf16 row: DK (fragment order) + pad
  static constexpr int KR = IK + 4;    // transposed rows: 80 keys + pad
  static constexpr int NP = DK / 4 + 4;
  static constexpr int OPP = 16 + 4;     // fp32 rows of the partial sums
  uint16_t X[IK][XR];                  // keys, dk in fragment order
  uint16_t XT[DK][KR];                 // keys transposed, keys in natural order
  uint16_t Q[IC][XR];                  // queries, dk in fragment order
  uint16_t YT[IRB][KR];                // values transposed
  float knp[2][IC][NP];                // squared-norm partials [key][dk quad], by chunk parity
  float bnext[2][IC];                  // gains, by chunk parity
  float kn[IK];                        // squared key norms (16 halo rows + the chunk)
  float gs[2][IC];                     // g_t, by chunk parity
  float zs[2][IC];                     // prefix sums Z of zeta, by chunk parity
  float zp[2][IK + 4];                 // [16 + j] = Z_{j-1} (0 for j <= 0), key j = -16..63
  float zq[2][IK + 4];                 // [16 + j] = Z_{min(j+B-1, C-1)}
  float c63[2][IK];                    // c_{m, C-1}, by chunk parity
  float opart[4][IC][OPP];             // S0 q partial sums of the state waves, [t][row]
  int bad;                             // some chunk's decay products left the range
};

struct IpGeom {
  int nrbg;
  int remap;
  int nchunks;
};

template <int N>
__device__ __forceinline__ float ip_shr(float v, float fill) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill), __builtin_bit_cast(int, v),
                                                             0x110 + N, 0xF, 0xF, false));
}
// two groups of 4 bf16 (8-byte reads) as one fragment; the second may be absent
__device__ __forceinline__ bf16x8 ip_frag2(const uint16_t* a, const uint16_t* b) {
  const uint2 x = *reinterpret_cast<const uint2*>(a);
  const uint2 y = *reinterpret_cast<const uint2*>(b);
  return __builtin_bit_cast(bf16x8, make_uint4(x.x, x.y, y.x, y.y));
}
__device__ __forceinline__ bf16x8 ip_frag1(const uint16_t* a) {
  const uint2 x = *reinterpret_cast<const uint2*>(a);
  return __builtin_bit_cast(bf16x8, make_uint4(x.x, x.y, 0u, 0u));
}
__device__ __forceinline__ HL ip_hl(const floatx4& a, const floatx4& b) {
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return hl_vals(v);
}
// element d (0..3) of four rows of 4 bf16 (uint2 each), packed as one uint2
__device__ __forceinline__ uint2 ip_col(const uint2 (&r)[4], int d) {
  const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;
  const uint32_t w0 = d < 2 ? r[0].x : r[0].y, w1 = d < 2 ? r[1].x : r[1].y;
  const uint32_t w2 = d < 2 ? r[2].x : r[2].y, w3 = d < 2 ? r[3].x : r[3].y;
  return make_uint2(__builtin_amdgcn_perm(w1, w0, sel), __builtin_amdgcn_perm(w3, w2, sel));
}

template <int DK>
__global__ __launch_bounds__(INT) void chunk_ip_kernel(SeqArgs a, IpGeom geo) {
  using SM = IpLds<DK>;
  constexpr int NKS = DK / 32;            // 32-wide dk steps
  constexpr int HKT = DK / 32;            // dk tiles per state wave (half of DK / 16)
  constexpr int HKS = HKT / 2 > 0 ? HKT / 2 : 1;
  constexpr int NKB = (IC / 4) * (DK / 4);      // 4 x 4 key blocks per chunk
  constexpr int KQP = IC * DK / 8 / INT;        // 16-byte query pieces per thread
  constexpr int SCW = 4;                        // the wave that forms the scalars (lightest readout)
  static_assert(DK == 64 || DK == 128, "dk in {64, 128}");
  static_assert(KQP >= 1 && NKB <= INT, "loader shape");
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
  const int i0 = rbg * IRB;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int L = a.seqlen;
  const int B = a.window;
  const int ks = a.key_shift;
  const bool fresh = ks == 1 && kpg == nullptr;
  const long qk_base = (long)chain * L * DK;
  const long v_base = (long)chain * L * dv;
  const int nchunks = geo.nchunks;

  // ---------------- zero the key tile (the samples before the sequence) ----------------
  for (int idx = tid; idx < IK * SM::XR; idx += INT) (&sm.X[0][0])[idx] = 0;
  for (int idx = tid; idx < DK * SM::KR; idx += INT) (&sm.XT[0][0])[idx] = 0;
  for (int idx = tid; idx < IRB * SM::KR; idx += INT) (&sm.YT[0][0])[idx] = 0;
  for (int idx = tid; idx < IK; idx += INT) sm.kn[idx] = 0.0f;
  for (int idx = tid; idx < 2 * (IK + 4); idx += INT) (&sm.zp[0][0])[idx] = 0.0f;
  __syncthreads();
  if (a.x_hist) {
    // a resumed sequence: the carried window samples (oldest first) are the
    // last B-1 samples before the first step
    const uint16_t* __restrict__ xhg = static_cast<const uint16_t*>(a.x_hist);
    const uint16_t* __restrict__ yhg = static_cast<const uint16_t*>(a.y_hist);
    const int NH = B - 1;
    for (int idx = tid; idx < NH * DK; idx += INT) {
      const int h = idx / DK, kk = idx % DK, m = 16 - NH + h;
      const uint16_t xv = xhg[((long)chain * NH + h) * DK + kk];
      sm.X[m][ip_fpos(kk)] = xv;
      sm.XT[kk][m] = xv;
    }
    for (int idx = tid; idx < NH * IRB; idx += INT) {
      const int h = idx / IRB, i = idx % IRB, m = 16 - NH + h;
      sm.YT[i][m] = yhg[((long)chain * NH + h) * dv + i0 + i];
    }
    if (tid < NH) {
      float n = 0.0f;
      for (int kk = 0; kk < DK; ++kk) {
        const float xv = bf16_to_f32(xhg[((long)chain * NH + tid) * DK + kk]);
        n = __builtin_fmaf(xv, xv, n);
      }
      sm.kn[16 - NH + tid] = n;
    }
  }

  // ---------------- global loads (buffer resources, range checked) ----------------
  constexpr int BUF_WORD3 = 0x00020000;
  constexpr uint32_t PARKED = 0xC0000000u;
  auto rsrc = [](const void* base, long bytes) __attribute__((always_inline)) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, BUF_WORD3);
  };
  const auto rk = rsrc(kg + qk_base, (long)L * DK * 2);
  const auto rq = rsrc(qg + qk_base, (long)L * DK * 2);
  const auto rv = rsrc(vg + v_base, (long)L * dv * 2);
  const auto rb = a.beta_kind == 1 ? rsrc(bg + (long)chain * L, (long)L * 2) : rsrc(vg, 0);
  // key block of this thread: samples 4 tq .. 4 tq + 3 of the chunk, dk 4 kq .. 4 kq + 3
  const int kq = tid % (DK / 4), tq = tid / (DK / 4);
  const bool kload = tid < NKB;
  // value block (threads 0..127): steps 4 vt .. 4 vt + 3, rows 4 vi .. 4 vi + 3
  const int vt = tid >> 3, vi = tid & 7;
  const bool vload = tid < (IC / 4) * (IRB / 4);
  // per-thread offsets (bytes) of chunk 0; a chunk adds a uniform stride
  uint32_t koff[4], voff[4], qoff[KQP];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // x_s = k_{s - ks}; the row before the sequence (chunk 0, ks = 1) wraps to an
    // offset far out of range, which reads 0, and every later chunk's stride
    // brings it back to the right row
    const int j = 4 * tq + e - ks;
    koff[e] = kload ? (uint32_t)((j * DK + 4 * kq) * 2) : PARKED;
    voff[e] = vload ? (uint32_t)(((4 * vt + e) * dv + i0 + 4 * vi) * 2) : PARKED;
  }
#pragma unroll
  for (int u = 0; u < KQP; ++u) {
    const int p = tid + INT * u;
    qoff[u] = (uint32_t)(((p / (DK / 8)) * DK + 8 * (p % (DK / 8))) * 2);
  }
  const uint32_t KQ_CHUNK = IC * DK * 2, V_CHUNK = (uint32_t)(IC * dv * 2);
  struct Set {
    uint2 k[4];
    uint4 q[KQP];
    uint2 v[4];
    uint16_t b;   // kept 16-bit: widening it at the load would wait for the load there
  };
  // the 32-bit offsets stay below 2^31 past the end (range checked): at most
  // (L + 3 C) * max(dk, dv) * 2 bytes
  auto issue = [&](Set& st, int c) __attribute__((always_inline)) {
    const uint32_t ck = (uint32_t)c * KQ_CHUNK, cv = (uint32_t)c * V_CHUNK;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto r = __builtin_amdgcn_raw_buffer_load_b64(rk, (int)(koff[e] + ck), 0, 0);
      st.k[e] = make_uint2(r[0], r[1]);
    }
#pragma unroll
    for (int u = 0; u < KQP; ++u) {
      const auto r = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(qoff[u] + ck), 0, 0);
      st.q[u] = make_uint4(r[0], r[1], r[2], r[3]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto r = __builtin_amdgcn_raw_buffer_load_b64(rv, (int)(voff[e] + cv), 0, 0);
      st.v[e] = make_uint2(r[0], r[1]);
    }
    st.b = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)((uint32_t)(c * IC + lane) * 2), 0, 0);
  };
  uint2 kprev = make_uint2(0u, 0u);
  if (kpg != nullptr && ks == 1 && kload && tq == 0)
    kprev = *reinterpret_cast<const uint2*>(kpg + (long)chain * DK + 4 * kq);
  auto keyrows = [&](const Set& st, int c, uint2 (&r)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = st.k[e];
    if (c == 0 && tq == 0 && ks == 1) r[0] = kprev;   // x_0 = k_prev (0 on a fresh start)
  };
  // before the barrier: squared-norm partial sums of chunk c's keys (packed bf16
  // dot products over this thread's 4 dk) and its gains
  auto norms_and_gains = [&](const Set& st, int c) __attribute__((always_inline)) {
    if (kload) {
      uint2 r[4];
      keyrows(st, c, r);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, r[e].x), __builtin_bit_cast(bf16x2, r[e].x), 0.0f, false);
        p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, r[e].y), __builtin_bit_cast(bf16x2, r[e].y), p, false);
        sm.knp[c & 1][4 * tq + e][kq] = p;
      }
    }
    if (wave == INW - 1) sm.bnext[c & 1][lane] = a.beta_kind == 1 ? bf16_to_f32(st.b) : a.beta;
  };
  // after the barrier: chunk c to LDS; for c > 0 the previous chunk's last 16
  // samples move to the halo rows first (each thread moves exactly what it then
  // overwrites)
  auto commit = [&](const Set& st, int c) __attribute__((always_inline)) {
    const bool slide = c > 0;
    if (kload) {
      uint2 r[4];
      keyrows(st, c, r);
      const int m0 = 16 + 4 * tq;
      const int xp = ip_fpos(4 * kq);
      if (slide && tq >= 12) {
        const int h0 = m0 - IC;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<uint2*>(&sm.X[h0 + e][xp]) = *reinterpret_cast<const uint2*>(&sm.X[m0 + e][xp]);
#pragma unroll
        for (int d = 0; d < 4; ++d)
          *reinterpret_cast<uint2*>(&sm.XT[4 * kq + d][h0]) = *reinterpret_cast<const uint2*>(&sm.XT[4 * kq + d][m0]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) *reinterpret_cast<uint2*>(&sm.X[m0 + e][xp]) = r[e];
#pragma unroll
      for (int d = 0; d < 4; ++d) *reinterpret_cast<uint2*>(&sm.XT[4 * kq + d][m0]) = ip_col(r, d);
    }
#pragma unroll
    for (int u = 0; u < KQP; ++u) {
      const int p = tid + INT * u;
      const int t = p / (DK / 8), o = p % (DK / 8);
      *reinterpret_cast<uint2*>(&sm.Q[t][ip_fpos(8 * o)]) = make_uint2(st.q[u].x, st.q[u].y);
      *reinterpret_cast<uint2*>(&sm.Q[t][ip_fpos(8 * o + 4)]) = make_uint2(st.q[u].z, st.q[u].w);
    }
    if (vload) {
      const int m0 = 16 + 4 * vt;
      if (slide && vt >= 12) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
          *reinterpret_cast<uint2*>(&sm.YT[4 * vi + d][m0 - IC]) = *reinterpret_cast<const uint2*>(&sm.YT[4 * vi + d][m0]);
      }
      uint2 r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = st.v[e];
#pragma unroll
      for (int d = 0; d < 4; ++d) *reinterpret_cast<uint2*>(&sm.YT[4 * vi + d][m0]) = ip_col(r, d);
    }
  };

  // one wave, after the barrier that made chunk c's partial norms and gains
  // visible (lane t = step t): squared norms (the halo rows keep the previous
  // chunk's last 16), eta, a = 1 - eta lambda, g = prefix product of a,
  // zeta = eta / g and its prefix sum, c_{., C-1}.  Padded steps and the
  // fresh-sequence first step take eta = 0, a = 1.  The shifted copies of the
  // prefix sums and the weights are formed from the register z by lane reads
  // (ds_bpermute, independent of each other), not stored and read back.
  auto lane_read = [](float v, int src) __attribute__((always_inline)) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
  };
  auto scalars = [&](int c) __attribute__((always_inline)) {
    const int t = lane;
    const int pb = c & 1;
    float nsum = 0.0f;
#pragma unroll
    for (int q4 = 0; q4 < DK / 16; ++q4) {
      const float4 v = *reinterpret_cast<const float4*>(&sm.knp[pb][t][4 * q4]);
      nsum += (v.x + v.y) + (v.z + v.w);
    }
    const float hv = (c > 0 && lane < 16) ? sm.kn[IC + lane] : 0.0f;
    wave_sync();
    if (c > 0 && lane < 16) sm.kn[lane] = hv;
    sm.kn[16 + t] = nsum;
    wave_sync();
    float n = 0.0f;
    for (int w = 0; w < B; ++w) n += sm.kn[16 + t - w];
    const int st = c * IC + t;
    const bool live = st < L && !(fresh && st == 0);
    const float eta = live ? sm.bnext[pb][t] * __builtin_amdgcn_rcpf(a.eps + n) : 0.0f;
    const float av = live ? 1.0f - eta * a.lambda : 1.0f;
    float g = av;
    g *= ip_shr<1>(g, 1.0f);
    g *= ip_shr<2>(g, 1.0f);
    g *= ip_shr<4>(g, 1.0f);
    g *= ip_shr<8>(g, 1.0f);
    const float p0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g), 15));
    const float p1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g), 31));
    const float p2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g), 47));
    g *= lg >= 1 ? p0 : 1.0f;
    g *= lg >= 2 ? p1 : 1.0f;
    g *= lg >= 3 ? p2 : 1.0f;
    if (__builtin_amdgcn_ballot_w64(gauge_out_of_range(g, av)) != 0 && lane == 0) sm.bad = 1;
    float z = eta * __builtin_amdgcn_rcpf(g);
    z += ip_shr<1>(z, 0.0f);
    z += ip_shr<2>(z, 0.0f);
    z += ip_shr<4>(z, 0.0f);
    z += ip_shr<8>(z, 0.0f);
    const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, z), 15));
    const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, z), 31));
    const float s2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, z), 47));
    z += lg >= 1 ? s0 : 0.0f;
    z += lg >= 2 ? s1 : 0.0f;
    z += lg >= 3 ? s2 : 0.0f;
    sm.gs[pb][t] = g;
    sm.zs[pb][t] = z;
    // shifted copies for the readout's 4-key reads, and c_{m, C-1} for key rows
    // m = lane and m = 64 + lane: c_{m, C-1} = Z_{min(m-16+B-1, C-1)} - Z_{m-17},
    // zero where that window of steps is empty
    const int j = t - 16 + B - 1;                 // keys -16..47 on lanes 0..63
    const int j2 = 48 + lane + B - 1;             // keys 48..63 on lanes 0..15
    auto cw_lanes = [&](int m, int& hi_l, int& lo_l, bool& use_lo, bool& ok) __attribute__((always_inline)) {
      const int jm = m - 16;
      const int lo = jm > 0 ? jm : 0;
      const int hj = jm + B - 1;
      const int hi = hj < IC - 1 ? hj : IC - 1;
      hi_l = hi > 0 ? hi : 0;
      lo_l = lo > 0 ? lo - 1 : 0;
      use_lo = lo > 0;
      ok = hi >= lo;
    };
    int h1, l1, h2, l2;
    bool u1, o1, u2, o2;
    cw_lanes(lane, h1, l1, u1, o1);
    cw_lanes(IC + lane, h2, l2, u2, o2);
    const float zm1 = lane_read(z, t > 0 ? t - 1 : 0);
    const float zq1 = lane_read(z, j < 0 ? 0 : (j > IC - 1 ? IC - 1 : j));
    const float zq2 = lane_read(z, j2 > IC - 1 ? IC - 1 : j2);
    const float zh1 = lane_read(z, h1), zl1 = lane_read(z, l1);
    const float zh2 = lane_read(z, h2), zl2 = lane_read(z, l2);
    sm.zp[pb][16 + t] = t > 0 ? zm1 : 0.0f;
    sm.zq[pb][t] = zq1;
    if (lane < 16) sm.zq[pb][64 + lane] = zq2;
    sm.c63[pb][lane] = o1 ? zh1 - (u1 ? zl1 : 0.0f) : 0.0f;
    if (lane < 16) sm.c63[pb][IC + lane] = o2 ? zh2 - (u2 ? zl2 : 0.0f) : 0.0f;
  };

  if (threadIdx.x == 0) sm.bad = 0;
  Set s0, s1;
  issue(s0, 0);
  issue(s1, 1);
  norms_and_gains(s0, 0);
  norms_and_gains(s1, 1);
  commit(s0, 0);
  issue(s0, 2);
  __syncthreads();
  if (wave == SCW) scalars(0);
  __syncthreads();

  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  if (wave < 4) {
    // ---------------- state waves ----------------
    const int rt = wave & 1, hh = wave >> 1;
    const int row = i0 + 16 * rt + lr;
    float sv[HKT][4];   // S[row][16 (hh HKT + kt) + 4 lg + e]
#pragma unroll
    for (int kt = 0; kt < HKT; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sv[kt][e] = a.S0 ? a.S0[((long)chain * dv + row) * DK + 16 * (hh * HKT + kt) + 4 * lg + e] : 0.0f;
    HL sf[HKS];
    auto resplit = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < HKS; ++k) sf[k] = ip_hl(floatx4{sv[2 * k][0], sv[2 * k][1], sv[2 * k][2], sv[2 * k][3]},
                                                  floatx4{sv[2 * k + 1][0], sv[2 * k + 1][1], sv[2 * k + 1][2], sv[2 * k + 1][3]});
    };
    resplit();
    auto body = [&](int c, Set& nxt, const Set& far) __attribute__((always_inline)) {
      const int pb = c & 1;
      const float g63 = sm.gs[pb][IC - 1];
      // S0 q partial sums over this wave's dk half: (S Q^T) tiles [row][t]
      {
        floatx4 acc[4] = {zero4, zero4, zero4, zero4};
        bf16x8 qf[HKS][4];
#pragma unroll
        for (int k = 0; k < HKS; ++k)
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) qf[k][tt] = frag_bf16(&sm.Q[16 * tt + lr][32 * (hh * HKS + k) + 8 * lg]);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < HKS; ++k) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) acc[tt] = mfma16(sf[k].hi, qf[k][tt], acc[tt]);
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) acc[tt] = mfma16(sf[k].lo, qf[k][tt], acc[tt]);
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          *reinterpret_cast<float4*>(&sm.opart[wave][16 * tt + lr][4 * lg]) = make_float4(acc[tt][0], acc[tt][1], acc[tt][2], acc[tt][3]);
      }
      // carry: S <- g_{C-1} (S + X^T diag(c) Y) over the 80 key rows
      HL ycf[3];
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int ma = 32 * k + 4 * lg, mb = ma + 16;
        const uint2 ya = *reinterpret_cast<const uint2*>(&sm.YT[16 * rt + lr][ma]);
        const float4 ca = *reinterpret_cast<const float4*>(&sm.c63[pb][ma]);
        float v[8];
        v[0] = ca.x * bf16_to_f32((uint16_t)(ya.x & 0xFFFFu));
        v[1] = ca.y * bf16_to_f32((uint16_t)(ya.x >> 16));
        v[2] = ca.z * bf16_to_f32((uint16_t)(ya.y & 0xFFFFu));
        v[3] = ca.w * bf16_to_f32((uint16_t)(ya.y >> 16));
        if (k < 2) {
          const uint2 yb = *reinterpret_cast<const uint2*>(&sm.YT[16 * rt + lr][mb]);
          const float4 cb = *reinterpret_cast<const float4*>(&sm.c63[pb][mb]);
          v[4] = cb.x * bf16_to_f32((uint16_t)(yb.x & 0xFFFFu));
          v[5] = cb.y * bf16_to_f32((uint16_t)(yb.x >> 16));
          v[6] = cb.z * bf16_to_f32((uint16_t)(yb.y & 0xFFFFu));
          v[7] = cb.w * bf16_to_f32((uint16_t)(yb.y >> 16));
        } else {
          v[4] = v[5] = v[6] = v[7] = 0.0f;
        }
        ycf[k] = hl_vals(v);
      }
      {
        floatx4 acc[HKT];
#pragma unroll
        for (int kt = 0; kt < HKT; ++kt) acc[kt] = floatx4{sv[kt][0], sv[kt][1], sv[kt][2], sv[kt][3]};
        bf16x8 xf[3][HKT];
#pragma unroll
        for (int k = 0; k < 3; ++k)
#pragma unroll
          for (int kt = 0; kt < HKT; ++kt) {
            const int dkr = 16 * (hh * HKT + kt) + lr;
            xf[k][kt] = k < 2 ? ip_frag2(&sm.XT[dkr][32 * k + 4 * lg], &sm.XT[dkr][32 * k + 16 + 4 * lg])
                              : ip_frag1(&sm.XT[dkr][32 * k + 4 * lg]);
          }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < 3; ++k) {
#pragma unroll
          for (int kt = 0; kt < HKT; ++kt) acc[kt] = mfma16(xf[k][kt], ycf[k].hi, acc[kt]);
#pragma unroll
          for (int kt = 0; kt < HKT; ++kt) acc[kt] = mfma16(xf[k][kt], ycf[k].lo, acc[kt]);
        }
#pragma unroll
        for (int kt = 0; kt < HKT; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[kt][e] = g63 * acc[kt][e];
      }
      resplit();
      if (c + 2 < nchunks) norms_and_gains(far, c + 2);
      __syncthreads();
      if (c + 1 < nchunks) commit(nxt, c + 1);
      issue(nxt, c + 3);
      __syncthreads();
    };
    // pairs of chunks, so that each register set keeps its registers (an odd
    // count runs one empty chunk: no live step, no output, the state unchanged)
    for (int c = 0; c < nchunks; c += 2) {
      body(c, s1, s0);
      body(c + 1, s0, s1);
    }
    if (a.S_out && !sm.bad) {
#pragma unroll
      for (int kt = 0; kt < HKT; ++kt)
        *reinterpret_cast<float4*>(a.S_out + ((long)chain * dv + row) * DK + 16 * (hh * HKT + kt) + 4 * lg) =
            make_float4(sv[kt][0], sv[kt][1], sv[kt][2], sv[kt][3]);
    }
  } else {
    // ---------------- readout waves: steps 16 tt .. 16 tt + 15 ----------------
    auto readout = [&](auto TT) __attribute__((always_inline)) {
      constexpr int tt = decltype(TT)::value;
      constexpr int nmb = tt + 2;              // key tiles up to the diagonal
      constexpr int nk = (nmb + 1) / 2;        // 32-key steps over them
      const int t = 16 * tt + lr;
      auto body = [&](int c, Set& nxt, const Set& far) __attribute__((always_inline)) {
        const int pb = c & 1;
        // the step and key indices are made opaque per chunk: otherwise the
        // compiler hoists the weight's lane conditions out of the loop as 40
        // scalar lane masks, which spill
        int tv = t, lgv = lg;
        asm volatile("" : "+v"(tv), "+v"(lgv));
        // P^T tiles (keys x steps): every operand fragment is read first (one
        // LDS round trip), then nmb independent product chains
        bf16x8 qf[NKS], xf[nmb][NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = frag_bf16(&sm.Q[t][32 * ks + 8 * lg]);
#pragma unroll
        for (int mb = 0; mb < nmb; ++mb)
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) xf[mb][ks] = frag_bf16(&sm.X[16 * mb + lr][32 * ks + 8 * lg]);
        asm volatile("" ::: "memory");
        floatx4 p[nmb];
#pragma unroll
        for (int mb = 0; mb < nmb; ++mb) p[mb] = zero4;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int mb = 0; mb < nmb; ++mb) p[mb] = mfma16(xf[mb][ks], qf[ks], p[mb]);
        // weights c_{j,t} = Z_{min(j+B-1,t)} - Z_{j-1} where 0 <= max(j, 0) <= min(j+B-1, t)
        const float zt = sm.zs[pb][tv];
        bf16x8 yf[2][nk];
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
          const uint16_t* yrow = &sm.YT[16 * r2 + lr][0];
#pragma unroll
          for (int k = 0; k < nk; ++k)
            yf[r2][k] = (2 * k + 1 < nmb) ? ip_frag2(yrow + 32 * k + 4 * lg, yrow + 32 * k + 16 + 4 * lg)
                                          : ip_frag1(yrow + 32 * k + 4 * lg);
        }
#pragma unroll
        for (int mb = 0; mb < nmb; ++mb) {
          const int j0 = 16 * mb - 16 + 4 * lgv;
          if (16 * tt >= 16 * mb + B - 2) {
            // the whole tile lies below the window band (t >= j + B - 1): the
            // weight depends on the key only and equals c_{j, C-1}
            const float4 w4 = *reinterpret_cast<const float4*>(&sm.c63[pb][16 + j0]);
            p[mb][0] *= w4.x;
            p[mb][1] *= w4.y;
            p[mb][2] *= w4.z;
            p[mb][3] *= w4.w;
          } else {
            const float4 zp4 = *reinterpret_cast<const float4*>(&sm.zp[pb][16 + j0]);
            const float4 zq4 = *reinterpret_cast<const float4*>(&sm.zq[pb][16 + j0]);
            const float zpv[4] = {zp4.x, zp4.y, zp4.z, zp4.w};
            const float zqv[4] = {zq4.x, zq4.y, zq4.z, zq4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = j0 + r;
              const int hj = j + B - 1;
              const float top = hj >= tv ? zt : zqv[r];
              const bool ok = (hj < tv ? hj : tv) >= (j > 0 ? j : 0);
              p[mb][r] *= ok ? top - zpv[r] : 0.0f;
            }
          }
        }
        // Y^T (c o P)^T: tiles [row][t]; the operand over 32 keys pairs two tiles
        floatx4 oi[2] = {zero4, zero4};
#pragma unroll
        for (int k = 0; k < nk; ++k) {
          const HL pf = ip_hl(p[2 * k], 2 * k + 1 < nmb ? p[2 * k + 1 < nmb ? 2 * k + 1 : 0] : zero4);
#pragma unroll
          for (int r2 = 0; r2 < 2; ++r2) oi[r2] = mfma16(yf[r2][k], pf.hi, oi[r2]);
#pragma unroll
          for (int r2 = 0; r2 < 2; ++r2) oi[r2] = mfma16(yf[r2][k], pf.lo, oi[r2]);
        }
        // the next chunk's scalars (its norms were complete at the last barrier)
        // and the norm partials of the one after
        if (wave == SCW) scalars(c + 1);
        if (c + 2 < nchunks) norms_and_gains(far, c + 2);
        __syncthreads();
        // o_t = g_t (S0 q_t + intra-chunk part)
        const float gt = sm.gs[pb][t];
        const int st = c * IC + t;
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
          const float4 pa = *reinterpret_cast<const float4*>(&sm.opart[r2][t][4 * lg]);
          const float4 pc = *reinterpret_cast<const float4*>(&sm.opart[r2 + 2][t][4 * lg]);
          if (st < L)
            *reinterpret_cast<float4*>(a.o + v_base + (long)st * dv + i0 + 16 * r2 + 4 * lg) =
                make_float4(gt * (oi[r2][0] + pa.x + pc.x), gt * (oi[r2][1] + pa.y + pc.y),
                            gt * (oi[r2][2] + pa.z + pc.z), gt * (oi[r2][3] + pa.w + pc.w));
        }
        if (c + 1 < nchunks) commit(nxt, c + 1);
        issue(nxt, c + 3);
        __syncthreads();
      };
      for (int c = 0; c < nchunks; c += 2) {
        body(c, s1, s0);
        body(c + 1, s0, s1);
      }
    };
    if (wave == 4) readout(std::integral_constant<int, 0>{});
    else if (wave == 5) readout(std::integral_constant<int, 1>{});
    else if (wave == 6) readout(std::integral_constant<int, 2>{});
    else {
      // the readout of steps 48-63 has the most products of the four: its wave
      // issues first on the SIMD it shares (measured: about 2%)
      __builtin_amdgcn_s_setprio(1);
      readout(std::integral_constant<int, 3>{});
      __builtin_amdgcn_s_setprio(0);
    }
  }
  // a chain whose decay products left the range of the chunk algebra: its rows
  // again, exactly, by the recurrence (S_out was left untouched above)
  __syncthreads();
  if (sm.bad) recurrence_rows<DK, INT, 16>(chain, i0, IRB);
}

template <int DK>
hipError_t launch_ip(const SeqArgs& a, hipStream_t stream) {
  static_assert(sizeof(IpLds<DK>) <= 160 * 1024, "LDS budget");
  IpGeom geo;
  const int nchain = a.batch * a.heads;
  geo.nrbg = a.dv / IRB;
  geo.remap = (nchain % 8 == 0) ? 1 : 0;
  geo.nchunks = (int)((a.seqlen + IC - 1) / IC);
  const unsigned nblocks = (unsigned)(nchain * geo.nrbg);
  hipLaunchKernelGGL((chunk_ip_kernel<DK>), dim3(nblocks), dim3(INT), 0, stream, a, geo);
  return hipGetLastError();
}

}  // namespace

bool chunk_ip_supported(const SeqArgs& a) {
  const long bytes = ((long)a.seqlen + 2 * IC) * (a.dk > a.dv ? a.dk : a.dv) * 2;
  return !a.regression && a.beta_kind != 2 && a.dtype == 0 && a.window >= 1 && a.window <= 16 &&
         (a.dk == 64 || a.dk == 128) && a.dv % IRB == 0 && bytes < (1L << 30);
}

// Inner-product family, gains shared by the value rows: 64-step chunks whatever
// the requested chunk.
hipError_t launch_chunk_ip(const SeqArgs& a, hipStream_t stream) {
  if (a.dk == 64) return launch_ip<64>(a, stream);
  if (a.dk == 128) return launch_ip<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace falcon
