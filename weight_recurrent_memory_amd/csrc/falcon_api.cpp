// falcon_api.cpp - the C ABI of libfalcon (declared in include/falcon.h):
// argument validation, kernel selection and launch on the caller's stream.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and can be exercised on a host without a GPU.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "falcon.h"
#include "falcon_launch.h"

#define FALCON_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool finite_nonneg(float x) { return isfinite(x) && x >= 0.0f; }

struct Range {
  const void* p;
  size_t bytes;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

int is_regression(int variant) {
  return variant == FALCON_1 || variant == FALCON_2 || variant == FALCON_3;
}

bool per_channel_variant(int variant) { return variant == FALCON_2 || variant == FALCON_2A; }

bool window_variant(int variant) { return variant == FALCON_3 || variant == FALCON_3A; }

// Validation shared by the recurrent and the chunk form.  hist_api: called from
// an entry point that can carry the window history.
int check_seq(const falcon::SeqArgs& a, bool hist_api) {
  if (a.variant < FALCON_1 || a.variant > FALCON_3A) return FALCON_ERR_INVALID_ARG;
  if (a.window < 1) return FALCON_ERR_INVALID_ARG;
  if (a.window != 1 && !window_variant(a.variant)) return FALCON_ERR_INVALID_ARG;
  if (a.beta_kind < FALCON_BETA_SCALAR || a.beta_kind > FALCON_BETA_CHANNEL)
    return FALCON_ERR_INVALID_ARG;
  if (a.beta_kind == FALCON_BETA_SCALAR) {
    if (a.beta_t != nullptr || !isfinite(a.beta)) return FALCON_ERR_INVALID_ARG;
  } else if (a.beta_t == nullptr) {
    return FALCON_ERR_INVALID_ARG;
  }
  if (a.beta_kind == FALCON_BETA_CHANNEL && !per_channel_variant(a.variant))
    return FALCON_ERR_INVALID_ARG;
  if (!finite_nonneg(a.lambda) || !finite_nonneg(a.eps)) return FALCON_ERR_INVALID_ARG;
  if (a.batch < 1 || a.heads < 1 || a.seqlen < 1 || a.dk < 1 || a.dv < 1)
    return FALCON_ERR_INVALID_ARG;
  if (a.dtype != FALCON_BF16 && a.dtype != FALCON_F32) return FALCON_ERR_INVALID_ARG;
  if (!a.q || !a.k || !a.v || !a.o) return FALCON_ERR_INVALID_ARG;
  // prefix pairing: a live state needs the key it pairs with the first value;
  // same-step pairing has no carried key
  if (a.key_shift && a.S0 && !a.k_prev) return FALCON_ERR_INVALID_ARG;
  if (!a.key_shift && a.k_prev) return FALCON_ERR_INVALID_ARG;
  const void* ptrs[] = {a.q, a.k, a.v, a.k_prev, a.S0, a.o, a.S_out, a.beta_t};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FALCON_ERR_INVALID_ARG;
  const double elems = (double)a.batch * a.heads * a.seqlen * (a.dk > a.dv ? a.dk : a.dv);
  if (elems > 1099511627776.0) return FALCON_ERR_INVALID_ARG;  // 2^40 elements
  const size_t es = a.dtype == FALCON_BF16 ? 2 : 4;
  const size_t BH = (size_t)a.batch * a.heads;
  const size_t L = (size_t)a.seqlen;
  Range o{a.o, BH * L * a.dv * 4};
  Range ins[] = {{a.q, BH * L * a.dk * es},
                 {a.k, BH * L * a.dk * es},
                 {a.v, BH * L * a.dv * es},
                 {a.k_prev, BH * a.dk * es},
                 {a.S0, BH * a.dv * a.dk * 4},
                 {a.S_out, BH * a.dv * a.dk * 4},
                 {a.beta_t, BH * L * (a.beta_kind == FALCON_BETA_CHANNEL ? a.dv : 1) * es}};
  for (const Range& r : ins)
    if (overlap(o, r)) return FALCON_ERR_INVALID_ARG;
  // S_out may equal S0 exactly (in-place carry) but must not partly overlap it or
  // overlap any other input.
  Range so{a.S_out, BH * a.dv * a.dk * 4};
  if (a.S_out && a.S_out != a.S0 && overlap(so, Range{a.S0, BH * a.dv * a.dk * 4}))
    return FALCON_ERR_INVALID_ARG;
  for (int i = 0; i < 4; ++i)
    if (overlap(so, ins[i])) return FALCON_ERR_INVALID_ARG;
  if (overlap(so, ins[6])) return FALCON_ERR_INVALID_ARG;
  if (!supported_dim(a.dk) || !supported_dim(a.dv)) return FALCON_ERR_UNSUPPORTED;
  if (!hist_api && a.window > 1 && a.S0) return FALCON_ERR_UNSUPPORTED;
  return FALCON_OK;
}

// Validation of the window history arguments (after check_seq).
int check_history(const falcon::SeqArgs& a, const void* xo, const void* yo) {
  const bool hin = a.x_hist != nullptr, hout = xo != nullptr;
  if ((a.x_hist == nullptr) != (a.y_hist == nullptr)) return FALCON_ERR_INVALID_ARG;
  if ((xo == nullptr) != (yo == nullptr)) return FALCON_ERR_INVALID_ARG;
  if ((hin || hout) && a.window < 2) return FALCON_ERR_INVALID_ARG;
  if (hin && a.key_shift && !a.k_prev) return FALCON_ERR_INVALID_ARG;
  if (a.window > 1 && a.S0 && !hin) return FALCON_ERR_INVALID_ARG;
  if (!hin && !hout) return FALCON_OK;
  const void* ptrs[] = {a.x_hist, a.y_hist, xo, yo};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FALCON_ERR_INVALID_ARG;
  const size_t es = a.dtype == FALCON_BF16 ? 2 : 4;
  const size_t BH = (size_t)a.batch * a.heads, L = (size_t)a.seqlen, NH = (size_t)a.window - 1;
  const size_t xb = BH * NH * a.dk * es, yb = BH * NH * a.dv * es;
  Range rxh{a.x_hist, xb}, ryh{a.y_hist, yb}, rxo{xo, xb}, ryo{yo, yb};
  Range others[] = {{a.q, BH * L * a.dk * es},
                    {a.k, BH * L * a.dk * es},
                    {a.v, BH * L * a.dv * es},
                    {a.k_prev, BH * a.dk * es},
                    {a.S0, BH * a.dv * a.dk * 4},
                    {a.o, BH * L * a.dv * 4},
                    {a.S_out, BH * a.dv * a.dk * 4},
                    {a.beta_t, BH * L * (a.beta_kind == FALCON_BETA_CHANNEL ? a.dv : 1) * es}};
  // the incoming history is read by the main kernel: no output may overlap it
  // (the history outputs are written afterwards)
  for (int i = 5; i < 7; ++i)
    if (overlap(rxh, others[i]) || overlap(ryh, others[i])) return FALCON_ERR_INVALID_ARG;
  if (overlap(rxh, ryh)) return FALCON_ERR_INVALID_ARG;
  // outputs: equal to their own incoming history or disjoint from it, disjoint
  // from everything else
  for (const Range& r : others)
    if (overlap(rxo, r) || overlap(ryo, r)) return FALCON_ERR_INVALID_ARG;
  if (overlap(rxo, ryo) || overlap(rxo, ryh) || overlap(ryo, rxh)) return FALCON_ERR_INVALID_ARG;
  if (xo != a.x_hist && overlap(rxo, rxh)) return FALCON_ERR_INVALID_ARG;
  if (yo != a.y_hist && overlap(ryo, ryh)) return FALCON_ERR_INVALID_ARG;
  return FALCON_OK;
}

int finish_launch(hipError_t e) { return e == hipSuccess ? FALCON_OK : FALCON_ERR_HIP; }

// The history outputs are written after the main kernel, on the same stream.
int launch_with_history(bool chunk_form, const falcon::SeqArgs& a, void* xo, void* yo,
                        hipStream_t stream, void* ws = nullptr, size_t ws_bytes = 0) {
  hipError_t e = chunk_form ? falcon::launch_chunk(a, stream, ws, ws_bytes) : falcon::launch_recurrent(a, stream);
  if (e == hipSuccess && xo) e = falcon::launch_history_out(a, xo, yo, stream);
  return finish_launch(e);
}

int fwd_recurrent(const falcon::SeqArgs& a, bool hist_api, void* xo, void* yo, hipStream_t stream) {
  int st = check_seq(a, hist_api);
  if (st == FALCON_OK && hist_api) st = check_history(a, xo, yo);
  if (st != FALCON_OK) return st;
  if (a.window > 8) return FALCON_ERR_UNSUPPORTED;
  return launch_with_history(false, a, xo, yo, stream);
}

// The workspace of falcon_fwd_chunk_ws may overlap no other argument.
bool ws_overlaps(const falcon::SeqArgs& a, const void* xo, const void* yo, const void* ws,
                 size_t ws_bytes) {
  const size_t es = a.dtype == FALCON_BF16 ? 2 : 4;
  const size_t BH = (size_t)a.batch * a.heads, L = (size_t)a.seqlen, NH = (size_t)a.window - 1;
  const Range w{ws, ws_bytes};
  const Range others[] = {{a.q, BH * L * a.dk * es},
                          {a.k, BH * L * a.dk * es},
                          {a.v, BH * L * a.dv * es},
                          {a.k_prev, BH * a.dk * es},
                          {a.S0, BH * a.dv * a.dk * 4},
                          {a.o, BH * L * a.dv * 4},
                          {a.S_out, BH * a.dv * a.dk * 4},
                          {a.beta_t, BH * L * (a.beta_kind == FALCON_BETA_CHANNEL ? a.dv : 1) * es},
                          {a.x_hist, BH * NH * a.dk * es},
                          {a.y_hist, BH * NH * a.dv * es},
                          {xo, BH * NH * a.dk * es},
                          {yo, BH * NH * a.dv * es}};
  for (const Range& r : others)
    if (overlap(w, r)) return true;
  return false;
}

int fwd_chunk(const falcon::SeqArgs& a, bool hist_api, void* xo, void* yo, hipStream_t stream,
              void* ws = nullptr, size_t ws_bytes = 0) {
  int st = check_seq(a, hist_api);
  if (st == FALCON_OK && hist_api) st = check_history(a, xo, yo);
  if (st != FALCON_OK) return st;
  if (a.chunk < 1) return FALCON_ERR_INVALID_ARG;
  if (a.chunk != 16 && a.chunk != 32 && a.chunk != 64) return FALCON_ERR_UNSUPPORTED;
  if (a.window > a.chunk) return FALCON_ERR_INVALID_ARG;
  if (a.dtype != FALCON_BF16) return FALCON_ERR_UNSUPPORTED;
  // wider windows: the inner-product kernel takes any window up to 16
  if (a.window > 4 && !falcon::chunk_ip_supported(a)) return FALCON_ERR_UNSUPPORTED;
  if (ws != nullptr) {
    if (!aligned16(ws)) return FALCON_ERR_INVALID_ARG;
    if (ws_overlaps(a, xo, yo, ws, ws_bytes)) return FALCON_ERR_INVALID_ARG;
  }
  return launch_with_history(true, a, xo, yo, stream, ws, ws_bytes);
}

int fwd_masked(const falcon::SeqArgs& a, void* xo, void* yo, hipStream_t stream) {
  int st = check_seq(a, true);
  if (st == FALCON_OK) st = check_history(a, xo, yo);
  if (st != FALCON_OK) return st;
  if (a.seqlen > falcon::kMaskedMaxLen || a.window > 8) return FALCON_ERR_UNSUPPORTED;
  hipError_t e = falcon::launch_masked(a, stream);
  if (e == hipSuccess && xo) e = falcon::launch_history_out(a, xo, yo, stream);
  return finish_launch(e);
}

}  // namespace

FALCON_EXPORT int falcon_abi_version(void) { return FALCON_ABI_VERSION; }

FALCON_EXPORT const char* falcon_status_string(int status) {
  switch (status) {
    case FALCON_OK: return "ok";
    case FALCON_ERR_INVALID_ARG: return "invalid argument";
    case FALCON_ERR_UNSUPPORTED: return "unsupported configuration";
    case FALCON_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

FALCON_EXPORT int falcon_fwd_recurrent(int variant, int window, float beta, const void* beta_t,
                                       int beta_kind, float lambda, float eps, int batch,
                                       int heads, int seqlen, int dk, int dv, int dtype,
                                       const void* q, const void* k, const void* v,
                                       const void* k_prev, const float* S0, float* o,
                                       float* S_out, void* stream) {
  falcon::SeqArgs a{variant, window, is_regression(variant), beta, beta_t, beta_kind, lambda,
                    eps, batch, heads, seqlen, dk, dv, dtype, q, k, v, k_prev, S0, o, S_out,
                    0};
  return fwd_recurrent(a, false, nullptr, nullptr, (hipStream_t)stream);
}

FALCON_EXPORT int falcon_fwd_recurrent_ex(int variant, int window, int flags, float beta,
                                          const void* beta_t, int beta_kind, float lambda,
                                          float eps, int batch, int heads, int seqlen, int dk,
                                          int dv, int dtype, const void* q, const void* k,
                                          const void* v, const void* k_prev, const float* S0,
                                          const void* x_hist, const void* y_hist, float* o,
                                          float* S_out, void* x_hist_out, void* y_hist_out,
                                          void* stream) {
  if (flags & ~FALCON_SAME_STEP) return FALCON_ERR_INVALID_ARG;
  falcon::SeqArgs a{variant, window, is_regression(variant), beta, beta_t, beta_kind, lambda,
                    eps, batch, heads, seqlen, dk, dv, dtype, q, k, v, k_prev, S0, o, S_out,
                    0, x_hist, y_hist, (flags & FALCON_SAME_STEP) ? 0 : 1};
  return fwd_recurrent(a, true, x_hist_out, y_hist_out, (hipStream_t)stream);
}

FALCON_EXPORT int falcon_fwd_chunk(int variant, int window, float beta, const void* beta_t,
                                   int beta_kind, float lambda, float eps, int batch, int heads,
                                   int seqlen, int dk, int dv, int dtype, const void* q,
                                   const void* k, const void* v, const void* k_prev,
                                   const float* S0, float* o, float* S_out, int chunk,
                                   void* stream) {
  falcon::SeqArgs a{variant, window, is_regression(variant), beta, beta_t, beta_kind, lambda,
                    eps, batch, heads, seqlen, dk, dv, dtype, q, k, v, k_prev, S0, o, S_out,
                    chunk};
  return fwd_chunk(a, false, nullptr, nullptr, (hipStream_t)stream);
}

FALCON_EXPORT int falcon_fwd_chunk_ex(int variant, int window, int flags, float beta,
                                      const void* beta_t, int beta_kind, float lambda, float eps,
                                      int batch, int heads, int seqlen, int dk, int dv, int dtype,
                                      const void* q, const void* k, const void* v,
                                      const void* k_prev, const float* S0, const void* x_hist,
                                      const void* y_hist, float* o, float* S_out,
                                      void* x_hist_out, void* y_hist_out, int chunk,
                                      void* stream) {
  if (flags & ~FALCON_SAME_STEP) return FALCON_ERR_INVALID_ARG;
  falcon::SeqArgs a{variant, window, is_regression(variant), beta, beta_t, beta_kind, lambda,
                    eps, batch, heads, seqlen, dk, dv, dtype, q, k, v, k_prev, S0, o, S_out,
                    chunk, x_hist, y_hist, (flags & FALCON_SAME_STEP) ? 0 : 1};
  return fwd_chunk(a, true, x_hist_out, y_hist_out, (hipStream_t)stream);
}

FALCON_EXPORT unsigned long long falcon_fwd_workspace_bytes(int variant, int window, int beta_kind,
                                                            int batch, int heads, int seqlen,
                                                            int dk, int dv, int dtype) {
  if (variant < FALCON_1 || variant > FALCON_3A || window < 1 || batch < 1 || heads < 1 ||
      seqlen < 1 || dk < 1 || dv < 1 || dtype != FALCON_BF16)
    return 0;
  if (beta_kind < FALCON_BETA_SCALAR || beta_kind > FALCON_BETA_CHANNEL) return 0;
  if (window != 1 && !window_variant(variant)) return 0;
  falcon::SeqArgs a{variant, window, is_regression(variant), 0.0f, nullptr, beta_kind, 0.0f, 0.0f,
                    batch, heads, seqlen, dk, dv, dtype, nullptr, nullptr, nullptr, nullptr,
                    nullptr, nullptr, nullptr, 64};
  return (unsigned long long)falcon::chunk_wyb2_workspace_bytes(a);
}

FALCON_EXPORT int falcon_fwd_chunk_ws(int variant, int window, int flags, float beta,
                                      const void* beta_t, int beta_kind, float lambda, float eps,
                                      int batch, int heads, int seqlen, int dk, int dv, int dtype,
                                      const void* q, const void* k, const void* v,
                                      const void* k_prev, const float* S0, const void* x_hist,
                                      const void* y_hist, float* o, float* S_out,
                                      void* x_hist_out, void* y_hist_out, void* workspace,
                                      unsigned long long workspace_bytes, int chunk,
                                      void* stream) {
  if (flags & ~FALCON_SAME_STEP) return FALCON_ERR_INVALID_ARG;
  falcon::SeqArgs a{variant, window, is_regression(variant), beta, beta_t, beta_kind, lambda,
                    eps, batch, heads, seqlen, dk, dv, dtype, q, k, v, k_prev, S0, o, S_out,
                    chunk, x_hist, y_hist, (flags & FALCON_SAME_STEP) ? 0 : 1};
  return fwd_chunk(a, true, x_hist_out, y_hist_out, (hipStream_t)stream, workspace,
                   (size_t)workspace_bytes);
}

FALCON_EXPORT int falcon_fwd_masked(int variant, int window, int flags, float beta,
                                    const void* beta_t, int beta_kind, float lambda, float eps,
                                    int batch, int heads, int seqlen, int dk, int dv, int dtype,
                                    const void* q, const void* k, const void* v,
                                    const void* k_prev, const float* S0, const void* x_hist,
                                    const void* y_hist, float* o, float* S_out, void* x_hist_out,
                                    void* y_hist_out, void* stream) {
  if (flags & ~FALCON_SAME_STEP) return FALCON_ERR_INVALID_ARG;
  falcon::SeqArgs a{variant, window, is_regression(variant), beta, beta_t, beta_kind, lambda,
                    eps, batch, heads, seqlen, dk, dv, dtype, q, k, v, k_prev, S0, o, S_out,
                    0, x_hist, y_hist, (flags & FALCON_SAME_STEP) ? 0 : 1};
  return fwd_masked(a, x_hist_out, y_hist_out, (hipStream_t)stream);
}

namespace {

int decode_step(int variant, int window, int flags, float beta, const void* beta_t,
                int beta_kind, float lambda, float eps, int nseq, int heads, int dk, int dv,
                int dtype, float* S, void* k_prev, void* x_hist, void* y_hist, const void* q,
                const void* k, const void* v, float* o, bool hist_api, void* stream) {
  if (variant < FALCON_1 || variant > FALCON_3A) return FALCON_ERR_INVALID_ARG;
  if (flags & ~FALCON_SAME_STEP) return FALCON_ERR_INVALID_ARG;
  const int key_shift = (flags & FALCON_SAME_STEP) ? 0 : 1;
  if ((k_prev != nullptr) != (key_shift == 1)) return FALCON_ERR_INVALID_ARG;
  if (window < 1 || (window != 1 && !window_variant(variant))) return FALCON_ERR_INVALID_ARG;
  if ((x_hist == nullptr) != (y_hist == nullptr)) return FALCON_ERR_INVALID_ARG;
  if ((x_hist != nullptr) != (window > 1)) return FALCON_ERR_INVALID_ARG;
  if (beta_kind < FALCON_BETA_SCALAR || beta_kind > FALCON_BETA_CHANNEL)
    return FALCON_ERR_INVALID_ARG;
  if (beta_kind == FALCON_BETA_SCALAR) {
    if (beta_t != nullptr || !isfinite(beta)) return FALCON_ERR_INVALID_ARG;
  } else if (beta_t == nullptr) {
    return FALCON_ERR_INVALID_ARG;
  }
  if (beta_kind == FALCON_BETA_CHANNEL && !per_channel_variant(variant))
    return FALCON_ERR_INVALID_ARG;
  if (!finite_nonneg(lambda) || !finite_nonneg(eps)) return FALCON_ERR_INVALID_ARG;
  if (nseq < 1 || heads < 1 || dk < 1 || dv < 1) return FALCON_ERR_INVALID_ARG;
  if (dtype != FALCON_BF16 && dtype != FALCON_F32) return FALCON_ERR_INVALID_ARG;
  if (!S || !q || !k || !v || !o) return FALCON_ERR_INVALID_ARG;
  const void* ptrs[] = {S, k_prev, q, k, v, o, beta_t, x_hist, y_hist};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FALCON_ERR_INVALID_ARG;
  const size_t es = dtype == FALCON_BF16 ? 2 : 4;
  const size_t NH = (size_t)nseq * heads, W1 = (size_t)window - 1;
  if ((double)NH * dk * dv > 1099511627776.0) return FALCON_ERR_INVALID_ARG;
  Range rS{S, NH * dv * dk * 4}, rkp{k_prev, NH * dk * es}, rq{q, NH * dk * es},
      rk{k, NH * dk * es}, rv{v, NH * dv * es}, ro{o, NH * dv * 4},
      rb{beta_t, NH * (beta_kind == FALCON_BETA_CHANNEL ? dv : 1) * es},
      rxh{x_hist, NH * W1 * dk * es}, ryh{y_hist, NH * W1 * dv * es};
  Range all[] = {rS, rkp, rq, rk, rv, ro, rb, rxh, ryh};
  for (int i = 0; i < 9; ++i)
    for (int j = i + 1; j < 9; ++j)
      if (overlap(all[i], all[j])) return FALCON_ERR_INVALID_ARG;
  if (!supported_dim(dk) || !supported_dim(dv)) return FALCON_ERR_UNSUPPORTED;
  if (!hist_api && window_variant(variant)) return FALCON_ERR_UNSUPPORTED;
  if (window > 8) return FALCON_ERR_UNSUPPORTED;
  falcon::DecodeArgs a{is_regression(variant), window, x_hist, y_hist, beta, beta_t, beta_kind,
                       lambda, eps, nseq, heads, dk, dv, dtype, S, k_prev, q, k, v, o,
                       key_shift};
  return finish_launch(falcon::launch_decode(a, (hipStream_t)stream));
}

}  // namespace

FALCON_EXPORT int falcon_decode_step(int variant, float beta, const void* beta_t, int beta_kind,
                                     float lambda, float eps, int nseq, int heads, int dk,
                                     int dv, int dtype, float* S, void* k_prev, const void* q,
                                     const void* k, const void* v, float* o, void* stream) {
  return decode_step(variant, 1, 0, beta, beta_t, beta_kind, lambda, eps, nseq, heads, dk, dv,
                     dtype, S, k_prev, nullptr, nullptr, q, k, v, o, false, stream);
}

FALCON_EXPORT int falcon_decode_step_ex(int variant, int window, int flags, float beta,
                                        const void* beta_t, int beta_kind, float lambda,
                                        float eps, int nseq, int heads, int dk, int dv,
                                        int dtype, float* S, void* k_prev, void* x_hist,
                                        void* y_hist, const void* q, const void* k,
                                        const void* v, float* o, void* stream) {
  return decode_step(variant, window, flags, beta, beta_t, beta_kind, lambda, eps, nseq, heads,
                     dk, dv, dtype, S, k_prev, x_hist, y_hist, q, k, v, o, true, stream);
}

namespace {
bool bwd_window(int window) { return window >= 1 && window <= 8; }
}  // namespace

FALCON_EXPORT unsigned long long falcon_bwd_workspace_bytes(int batch, int heads, int seqlen, int dk,
                                                            int dv, int window) {
  if (batch < 1 || heads < 1 || seqlen < 1 || !supported_dim(dk) || !supported_dim(dv) ||
      !bwd_window(window))
    return 0;
  return (unsigned long long)falcon::backward_workspace_bytes(batch, heads, seqlen, dk, dv, window);
}

namespace {

// Validation of a backward call, everything but the workspace.  On success
// fills *b (workspace left null) and *need (workspace bytes).
int check_bwd(int variant, int window, int flags, float beta, const void* beta_t, int beta_kind,
              float lambda, float eps, int batch, int heads, int seqlen, int dk, int dv, int dtype,
              const void* q, const void* k, const void* v, const void* k_prev, const float* S0,
              const float* dO, const float* dS_L, const float* dk_last, float* dq, float* dk_out,
              float* dv_out, float* dbeta_t, float* dk_prev, float* dS0, falcon::BwdArgs* b,
              size_t* need) {
  if (flags & ~FALCON_SAME_STEP) return FALCON_ERR_INVALID_ARG;
  const int key_shift = (flags & FALCON_SAME_STEP) ? 0 : 1;
  // the forward arguments are checked as the forward checks them (dO takes the
  // place of o: same shape, and it must not overlap an input either)
  falcon::SeqArgs a{variant, window, is_regression(variant), beta, beta_t, beta_kind, lambda, eps,
                    batch, heads, seqlen, dk, dv, dtype, q, k, v, k_prev, S0,
                    const_cast<float*>(dO), nullptr, 0, nullptr, nullptr, key_shift};
  int st = check_seq(a, true);
  if (st != FALCON_OK) return st;
  if (!dq || !dk_out || !dv_out) return FALCON_ERR_INVALID_ARG;
  if (dbeta_t && beta_kind == FALCON_BETA_SCALAR) return FALCON_ERR_INVALID_ARG;
  if (dk_prev && (!k_prev || !key_shift)) return FALCON_ERR_INVALID_ARG;
  if (dS0 && !S0) return FALCON_ERR_INVALID_ARG;
  const void* ptrs[] = {dS_L, dk_last, dq, dk_out, dv_out, dbeta_t, dk_prev, dS0};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FALCON_ERR_INVALID_ARG;
  // windows 1..8; a windowed start state would need its window history,
  // which this entry point does not take
  if (!bwd_window(window)) return FALCON_ERR_UNSUPPORTED;
  if (window > 1 && S0) return FALCON_ERR_UNSUPPORTED;
  // a chain's inputs and workspace record are addressed with 32-bit offsets
  if (falcon::backward_chain_bytes(seqlen, dk, dv, window, dtype) >= (1ull << 30))
    return FALCON_ERR_UNSUPPORTED;
  const size_t es = dtype == FALCON_BF16 ? 2 : 4;
  const size_t BH = (size_t)batch * heads, L = (size_t)seqlen;
  Range outs[] = {{dq, BH * L * dk * 4},
                  {dk_out, BH * L * dk * 4},
                  {dv_out, BH * L * dv * 4},
                  {dbeta_t, BH * L * (beta_kind == FALCON_BETA_CHANNEL ? dv : 1) * 4},
                  {dk_prev, BH * dk * 4},
                  {dS0, BH * dv * dk * 4}};
  Range ins[] = {{q, BH * L * dk * es},
                 {k, BH * L * dk * es},
                 {v, BH * L * dv * es},
                 {k_prev, BH * dk * es},
                 {S0, BH * dv * dk * 4},
                 {beta_t, BH * L * (beta_kind == FALCON_BETA_CHANNEL ? dv : 1) * es},
                 {dO, BH * L * dv * 4},
                 {dS_L, BH * dv * dk * 4},
                 {dk_last, BH * dk * 4}};
  for (int i = 0; i < 6; ++i) {
    for (int j = i + 1; j < 6; ++j)
      if (overlap(outs[i], outs[j])) return FALCON_ERR_INVALID_ARG;
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return FALCON_ERR_INVALID_ARG;
  }
  *need = falcon::backward_workspace_bytes(batch, heads, seqlen, dk, dv, window);
  *b = falcon::BwdArgs{is_regression(variant), window, key_shift, beta, beta_t, beta_kind, lambda,
                       eps, batch, heads, (long)seqlen, dk, dv, dtype, q, k, v, k_prev, S0, dO,
                       dS_L, dk_last, dq, dk_out, dv_out, dbeta_t, dk_prev, dS0, nullptr};
  return FALCON_OK;
}

}  // namespace

FALCON_EXPORT int falcon_bwd_chunk(int variant, int window, int flags, float beta, const void* beta_t,
                                   int beta_kind, float lambda, float eps, int batch, int heads,
                                   int seqlen, int dk, int dv, int dtype, const void* q,
                                   const void* k, const void* v, const void* k_prev,
                                   const float* S0, const float* dO, const float* dS_L,
                                   const float* dk_last, float* dq, float* dk_out, float* dv_out,
                                   float* dbeta_t, float* dk_prev, float* dS0, void* workspace,
                                   unsigned long long workspace_bytes, void* stream) {
  falcon::BwdArgs b;
  size_t need = 0;
  int st = check_bwd(variant, window, flags, beta, beta_t, beta_kind, lambda, eps, batch, heads,
                     seqlen, dk, dv, dtype, q, k, v, k_prev, S0, dO, dS_L, dk_last, dq, dk_out,
                     dv_out, dbeta_t, dk_prev, dS0, &b, &need);
  if (st != FALCON_OK) return st;
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return FALCON_ERR_INVALID_ARG;
  const size_t es = dtype == FALCON_BF16 ? 2 : 4;
  const size_t BH = (size_t)batch * heads, L = (size_t)seqlen;
  const Range ws{workspace, need};
  const Range others[] = {{dq, BH * L * dk * 4},
                          {dk_out, BH * L * dk * 4},
                          {dv_out, BH * L * dv * 4},
                          {dbeta_t, BH * L * (beta_kind == FALCON_BETA_CHANNEL ? dv : 1) * 4},
                          {dk_prev, BH * dk * 4},
                          {dS0, BH * dv * dk * 4},
                          {q, BH * L * dk * es},
                          {k, BH * L * dk * es},
                          {v, BH * L * dv * es},
                          {k_prev, BH * dk * es},
                          {S0, BH * dv * dk * 4},
                          {beta_t, BH * L * (beta_kind == FALCON_BETA_CHANNEL ? dv : 1) * es},
                          {dO, BH * L * dv * 4},
                          {dS_L, BH * dv * dk * 4},
                          {dk_last, BH * dk * 4}};
  for (const Range& r : others)
    if (overlap(ws, r)) return FALCON_ERR_INVALID_ARG;
  b.workspace = static_cast<float*>(workspace);
  return finish_launch(falcon::launch_backward(b, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// Backward without a caller workspace: the workspace is a file-scope device
// array of FALCON_BWD_SCRATCH_BYTES.  In host code `scratch` names a host-side
// stand-in, not device memory; its device address is looked up once per device
// (with that device current) and only that address is passed to kernels.

namespace {

__device__ __align__(256) float scratch[FALCON_BWD_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once known

// Device address of this device's `scratch`, or nullptr if it cannot be found.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

FALCON_EXPORT int falcon_bwd_chunk_noalloc(int variant, int window, int flags, float beta,
                                           const void* beta_t, int beta_kind, float lambda,
                                           float eps, int batch, int heads, int seqlen, int dk,
                                           int dv, int dtype, const void* q, const void* k,
                                           const void* v, const void* k_prev, const float* S0,
                                           const float* dO, const float* dS_L,
                                           const float* dk_last, float* dq, float* dk_out,
                                           float* dv_out, float* dbeta_t, float* dk_prev,
                                           float* dS0, void* stream) {
  falcon::BwdArgs b;
  size_t need = 0;
  int st = check_bwd(variant, window, flags, beta, beta_t, beta_kind, lambda, eps, batch, heads,
                     seqlen, dk, dv, dtype, q, k, v, k_prev, S0, dO, dS_L, dk_last, dq, dk_out,
                     dv_out, dbeta_t, dk_prev, dS0, &b, &need);
  if (st != FALCON_OK) return st;
  if (need > FALCON_BWD_SCRATCH_BYTES) return FALCON_ERR_UNSUPPORTED;
  void* ws = scratch_on_current_device();
  if (!ws) return FALCON_ERR_HIP;
  // every workspace element the kernels read is written earlier in the same
  // call, so nothing is cleared
  b.workspace = static_cast<float*>(ws);
  return finish_launch(falcon::launch_backward(b, (hipStream_t)stream));
}
