// falcon_api.cpp - the C ABI of libfalcon (declared in include/falcon.h):
// argument validation, kernel selection and launch on the caller's stream.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and can be exercised on a host without a GPU.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

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

// Validation shared by the recurrent and the chunk form.
int check_seq(const falcon::SeqArgs& a) {
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
  if (a.S0 && !a.k_prev) return FALCON_ERR_INVALID_ARG;
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
  if (a.window > 1 && a.S0) return FALCON_ERR_UNSUPPORTED;
  return FALCON_OK;
}

int finish_launch(hipError_t e) { return e == hipSuccess ? FALCON_OK : FALCON_ERR_HIP; }

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
  int st = check_seq(a);
  if (st != FALCON_OK) return st;
  if (window > 8) return FALCON_ERR_UNSUPPORTED;
  return finish_launch(falcon::launch_recurrent(a, (hipStream_t)stream));
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
  int st = check_seq(a);
  if (st != FALCON_OK) return st;
  if (chunk < 1) return FALCON_ERR_INVALID_ARG;
  if (chunk != 16 && chunk != 32 && chunk != 64) return FALCON_ERR_UNSUPPORTED;
  if (window > chunk) return FALCON_ERR_INVALID_ARG;
  if (window > 4) return FALCON_ERR_UNSUPPORTED;
  if (dtype != FALCON_BF16) return FALCON_ERR_UNSUPPORTED;
  return finish_launch(falcon::launch_chunk(a, (hipStream_t)stream));
}

FALCON_EXPORT int falcon_decode_step(int variant, float beta, const void* beta_t, int beta_kind,
                                     float lambda, float eps, int nseq, int heads, int dk,
                                     int dv, int dtype, float* S, void* k_prev, const void* q,
                                     const void* k, const void* v, float* o, void* stream) {
  if (variant < FALCON_1 || variant > FALCON_3A) return FALCON_ERR_INVALID_ARG;
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
  if (!S || !k_prev || !q || !k || !v || !o) return FALCON_ERR_INVALID_ARG;
  const void* ptrs[] = {S, k_prev, q, k, v, o, beta_t};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FALCON_ERR_INVALID_ARG;
  const size_t es = dtype == FALCON_BF16 ? 2 : 4;
  const size_t NH = (size_t)nseq * heads;
  if ((double)NH * dk * dv > 1099511627776.0) return FALCON_ERR_INVALID_ARG;
  Range rS{S, NH * dv * dk * 4}, rkp{k_prev, NH * dk * es}, rq{q, NH * dk * es},
      rk{k, NH * dk * es}, rv{v, NH * dv * es}, ro{o, NH * dv * 4},
      rb{beta_t, NH * (beta_kind == FALCON_BETA_CHANNEL ? dv : 1) * es};
  Range all[] = {rS, rkp, rq, rk, rv, ro, rb};
  for (int i = 0; i < 7; ++i)
    for (int j = i + 1; j < 7; ++j)
      if (overlap(all[i], all[j])) return FALCON_ERR_INVALID_ARG;
  if (!supported_dim(dk) || !supported_dim(dv)) return FALCON_ERR_UNSUPPORTED;
  if (window_variant(variant)) return FALCON_ERR_UNSUPPORTED;
  falcon::DecodeArgs a{is_regression(variant), beta, beta_t, beta_kind, lambda, eps, nseq,
                       heads, dk, dv, dtype, S, k_prev, q, k, v, o};
  return finish_launch(falcon::launch_decode(a, (hipStream_t)stream));
}
