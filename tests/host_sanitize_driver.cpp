// Host-side check of the C-ABI layer under AddressSanitizer and
// UndefinedBehaviorSanitizer (built and run by tests/test_host_sanitize.py on a
// machine without a GPU).  Every entry point of include/falcon.h is called with
// arguments that validation must reject and with well-formed ones that reach
// the HIP launch, which then fails for want of a device (FALCON_ERR_HIP).  The
// pointers are host allocations standing in for device buffers: the layer only
// compares and aligns them, it never reads through them.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstdint>
#include <cstring>
#include <functional>
#include <string>
#include <vector>

#include "falcon.h"

namespace {

int g_failures = 0;
int g_checks = 0;

void expect(const std::string& what, long got, long want) {
  ++g_checks;
  if (got != want) {
    ++g_failures;
    std::printf("FAIL %s: got %ld, want %ld\n", what.c_str(), got, want);
  }
}

// one aligned host buffer per tensor, so that no two arguments overlap
struct Buffers {
  std::vector<void*> owned;
  void* get(size_t bytes) {
    void* p = std::aligned_alloc(256, (bytes + 255) / 256 * 256);
    std::memset(p, 0, (bytes + 255) / 256 * 256);
    owned.push_back(p);
    return p;
  }
  ~Buffers() {
    for (void* p : owned) std::free(p);
  }
};

// arguments of the sequence entry points
struct Seq {
  int variant = FALCON_1, window = 1, flags = 0;
  float beta = 0.5f;
  const void* beta_t = nullptr;
  int beta_kind = FALCON_BETA_SCALAR;
  float lambda = 0.01f, eps = 1e-6f;
  int batch = 1, heads = 2, seqlen = 40, dk = 64, dv = 64, dtype = FALCON_BF16;
  const void *q = nullptr, *k = nullptr, *v = nullptr, *k_prev = nullptr;
  const float* S0 = nullptr;
  const void *x_hist = nullptr, *y_hist = nullptr;
  float *o = nullptr, *S_out = nullptr;
  void *x_hist_out = nullptr, *y_hist_out = nullptr;
  void* ws = nullptr;
  unsigned long long ws_bytes = 0;
  int chunk = 64;
};

Seq base_seq(Buffers& b) {
  Seq s;
  const size_t tok = (size_t)s.batch * s.heads * s.seqlen;
  s.q = b.get(tok * s.dk * 2);
  s.k = b.get(tok * s.dk * 2);
  s.v = b.get(tok * s.dv * 2);
  s.o = static_cast<float*>(b.get(tok * s.dv * 4));
  s.S_out = static_cast<float*>(b.get((size_t)s.batch * s.heads * s.dv * s.dk * 4));
  return s;
}

int call_recurrent(const Seq& s) {
  return falcon_fwd_recurrent(s.variant, s.window, s.beta, s.beta_t, s.beta_kind, s.lambda, s.eps, s.batch,
                              s.heads, s.seqlen, s.dk, s.dv, s.dtype, s.q, s.k, s.v, s.k_prev, s.S0, s.o,
                              s.S_out, nullptr);
}
int call_chunk(const Seq& s) {
  return falcon_fwd_chunk(s.variant, s.window, s.beta, s.beta_t, s.beta_kind, s.lambda, s.eps, s.batch, s.heads,
                          s.seqlen, s.dk, s.dv, s.dtype, s.q, s.k, s.v, s.k_prev, s.S0, s.o, s.S_out, s.chunk,
                          nullptr);
}
int call_recurrent_ex(const Seq& s) {
  return falcon_fwd_recurrent_ex(s.variant, s.window, s.flags, s.beta, s.beta_t, s.beta_kind, s.lambda, s.eps,
                                 s.batch, s.heads, s.seqlen, s.dk, s.dv, s.dtype, s.q, s.k, s.v, s.k_prev, s.S0,
                                 s.x_hist, s.y_hist, s.o, s.S_out, s.x_hist_out, s.y_hist_out, nullptr);
}
int call_chunk_ex(const Seq& s) {
  return falcon_fwd_chunk_ex(s.variant, s.window, s.flags, s.beta, s.beta_t, s.beta_kind, s.lambda, s.eps,
                             s.batch, s.heads, s.seqlen, s.dk, s.dv, s.dtype, s.q, s.k, s.v, s.k_prev, s.S0,
                             s.x_hist, s.y_hist, s.o, s.S_out, s.x_hist_out, s.y_hist_out, s.chunk, nullptr);
}
int call_chunk_ws(const Seq& s) {
  return falcon_fwd_chunk_ws(s.variant, s.window, s.flags, s.beta, s.beta_t, s.beta_kind, s.lambda, s.eps,
                             s.batch, s.heads, s.seqlen, s.dk, s.dv, s.dtype, s.q, s.k, s.v, s.k_prev, s.S0,
                             s.x_hist, s.y_hist, s.o, s.S_out, s.x_hist_out, s.y_hist_out, s.ws, s.ws_bytes,
                             s.chunk, nullptr);
}
int call_masked(const Seq& s) {
  return falcon_fwd_masked(s.variant, s.window, s.flags, s.beta, s.beta_t, s.beta_kind, s.lambda, s.eps,
                           s.batch, s.heads, s.seqlen, s.dk, s.dv, s.dtype, s.q, s.k, s.v, s.k_prev, s.S0,
                           s.x_hist, s.y_hist, s.o, s.S_out, s.x_hist_out, s.y_hist_out, nullptr);
}

using SeqFn = std::function<int(const Seq&)>;

// validation cases shared by every sequence entry point
void seq_cases(const char* name, const SeqFn& fn, Buffers& b, bool chunk_form) {
  const Seq s0 = base_seq(b);
  auto run = [&](const char* label, const std::function<void(Seq&)>& edit, int want) {
    Seq s = s0;
    edit(s);
    expect(std::string(name) + " " + label, fn(s), want);
  };
  void* beta_tok = b.get((size_t)s0.batch * s0.heads * s0.seqlen * 2);
  void* kp = b.get((size_t)s0.batch * s0.heads * s0.dk * 2);
  void* s_in = b.get((size_t)s0.batch * s0.heads * s0.dv * s0.dk * 4);
  run("variant 6", [](Seq& s) { s.variant = 6; }, FALCON_ERR_INVALID_ARG);
  run("variant -1", [](Seq& s) { s.variant = -1; }, FALCON_ERR_INVALID_ARG);
  run("window 0", [](Seq& s) { s.window = 0; }, FALCON_ERR_INVALID_ARG);
  run("window 2 on Falcon-1", [](Seq& s) { s.window = 2; }, FALCON_ERR_INVALID_ARG);
  run("null q", [](Seq& s) { s.q = nullptr; }, FALCON_ERR_INVALID_ARG);
  run("null o", [](Seq& s) { s.o = nullptr; }, FALCON_ERR_INVALID_ARG);
  run("misaligned q", [](Seq& s) { s.q = static_cast<const char*>(s.q) + 2; }, FALCON_ERR_INVALID_ARG);
  run("seqlen 0", [](Seq& s) { s.seqlen = 0; }, FALCON_ERR_INVALID_ARG);
  run("batch -3", [](Seq& s) { s.batch = -3; }, FALCON_ERR_INVALID_ARG);
  run("lambda -0.1", [](Seq& s) { s.lambda = -0.1f; }, FALCON_ERR_INVALID_ARG);
  run("eps nan", [](Seq& s) { s.eps = std::nanf(""); }, FALCON_ERR_INVALID_ARG);
  run("beta inf", [](Seq& s) { s.beta = INFINITY; }, FALCON_ERR_INVALID_ARG);
  run("per-token kind, no pointer", [](Seq& s) { s.beta_kind = FALCON_BETA_TOKEN; }, FALCON_ERR_INVALID_ARG);
  run("pointer with scalar kind", [&](Seq& s) { s.beta_t = beta_tok; }, FALCON_ERR_INVALID_ARG);
  run("per-channel beta on Falcon-1", [&](Seq& s) { s.beta_t = beta_tok; s.beta_kind = FALCON_BETA_CHANNEL; },
      FALCON_ERR_INVALID_ARG);
  run("beta kind 3", [&](Seq& s) { s.beta_t = beta_tok; s.beta_kind = 3; }, FALCON_ERR_INVALID_ARG);
  run("state without carried key", [&](Seq& s) { s.S0 = static_cast<const float*>(s_in); },
      FALCON_ERR_INVALID_ARG);
  run("o aliases q", [](Seq& s) { s.o = static_cast<float*>(const_cast<void*>(s.q)); }, FALCON_ERR_INVALID_ARG);
  run("dtype 7", [](Seq& s) { s.dtype = 7; }, FALCON_ERR_INVALID_ARG);
  run("dk 48", [](Seq& s) { s.dk = 48; }, FALCON_ERR_UNSUPPORTED);
  run("dv 256", [](Seq& s) { s.dv = 256; }, FALCON_ERR_UNSUPPORTED);
  if (chunk_form) {
    run("chunk 0", [](Seq& s) { s.chunk = 0; }, FALCON_ERR_INVALID_ARG);
    run("chunk 48", [](Seq& s) { s.chunk = 48; }, FALCON_ERR_UNSUPPORTED);
    run("fp32 inputs", [](Seq& s) { s.dtype = FALCON_F32; }, FALCON_ERR_UNSUPPORTED);
    run("window 32 above chunk 16", [](Seq& s) { s.variant = FALCON_3; s.window = 32; s.chunk = 16; },
        FALCON_ERR_INVALID_ARG);
  }
  // well-formed: validation passes, the launch fails without a device
  run("well-formed", [](Seq&) {}, FALCON_ERR_HIP);
  run("well-formed, carried key and state", [&](Seq& s) { s.k_prev = kp; s.S0 = static_cast<const float*>(s_in); },
      FALCON_ERR_HIP);
  run("well-formed, per-token beta", [&](Seq& s) { s.beta_t = beta_tok; s.beta_kind = FALCON_BETA_TOKEN; },
      FALCON_ERR_HIP);
  run("well-formed, in-place state", [&](Seq& s) {
        s.k_prev = kp;
        s.S0 = static_cast<const float*>(s_in);
        s.S_out = static_cast<float*>(s_in);
      },
      FALCON_ERR_HIP);
}

void history_cases(const char* name, const SeqFn& fn, Buffers& b, bool masked) {
  Seq s0 = base_seq(b);
  s0.variant = FALCON_3;
  s0.window = 4;
  const size_t ch = (size_t)s0.batch * s0.heads;
  void* xh = b.get(ch * 3 * s0.dk * 2);
  void* yh = b.get(ch * 3 * s0.dv * 2);
  void* xo = b.get(ch * 3 * s0.dk * 2);
  void* yo = b.get(ch * 3 * s0.dv * 2);
  void* kp = b.get(ch * s0.dk * 2);
  void* s_in = b.get(ch * s0.dv * s0.dk * 4);
  auto run = [&](const char* label, const std::function<void(Seq&)>& edit, int want) {
    Seq s = s0;
    edit(s);
    expect(std::string(name) + " " + label, fn(s), want);
  };
  run("flags 2", [](Seq& s) { s.flags = 2; }, FALCON_ERR_INVALID_ARG);
  run("same step with carried key", [&](Seq& s) { s.flags = FALCON_SAME_STEP; s.k_prev = kp; },
      FALCON_ERR_INVALID_ARG);
  run("one history pointer", [&](Seq& s) { s.x_hist = xh; }, FALCON_ERR_INVALID_ARG);
  run("history output aliases input", [&](Seq& s) {
        s.x_hist = xh;
        s.y_hist = yh;
        s.x_hist_out = const_cast<void*>(s.q);
        s.y_hist_out = yo;
      },
      FALCON_ERR_INVALID_ARG);
  if (masked) run("seqlen 65", [](Seq& s) { s.seqlen = 65; }, FALCON_ERR_UNSUPPORTED);
  run("well-formed resume", [&](Seq& s) {
        s.k_prev = kp;
        s.S0 = static_cast<const float*>(s_in);
        s.x_hist = xh;
        s.y_hist = yh;
        s.x_hist_out = xo;
        s.y_hist_out = yo;
      },
      FALCON_ERR_HIP);
  run("well-formed same step", [&](Seq& s) { s.flags = FALCON_SAME_STEP; }, FALCON_ERR_HIP);
}

void workspace_cases(Buffers& b) {
  Seq s0 = base_seq(b);
  s0.variant = FALCON_3;
  s0.window = 4;
  const unsigned long long need = falcon_fwd_workspace_bytes(FALCON_3, 4, 0, s0.batch, s0.heads, s0.seqlen,
                                                             s0.dk, s0.dv, FALCON_BF16);
  expect("workspace bytes", (long)need, (long)((size_t)s0.batch * s0.heads * ((s0.seqlen + 15) / 16) * 12416));
  expect("workspace bytes, Falcon-3A", (long)falcon_fwd_workspace_bytes(FALCON_3A, 4, 0, 1, 1, 64, 64, 64, 0), 0);
  expect("workspace bytes, batch 0", (long)falcon_fwd_workspace_bytes(FALCON_3, 4, 0, 0, 1, 64, 64, 64, 0), 0);
  void* ws = b.get(need);
  auto run = [&](const char* label, const std::function<void(Seq&)>& edit, int want) {
    Seq s = s0;
    s.ws = ws;
    s.ws_bytes = need;
    edit(s);
    expect(std::string("falcon_fwd_chunk_ws ") + label, call_chunk_ws(s), want);
  };
  run("misaligned workspace", [](Seq& s) { s.ws = static_cast<char*>(s.ws) + 8; }, FALCON_ERR_INVALID_ARG);
  run("workspace overlaps q", [](Seq& s) { s.ws = const_cast<void*>(s.q); }, FALCON_ERR_INVALID_ARG);
  run("window 4 on Falcon-1", [](Seq& s) { s.variant = FALCON_1; }, FALCON_ERR_INVALID_ARG);
  run("well-formed", [](Seq&) {}, FALCON_ERR_HIP);
  run("workspace one byte short", [](Seq& s) { s.ws_bytes -= 1; }, FALCON_ERR_HIP);
}

void decode_cases(Buffers& b) {
  const int nseq = 3, heads = 2, dk = 64, dv = 64;
  const size_t ch = (size_t)nseq * heads;
  float* S = static_cast<float*>(b.get(ch * dv * dk * 4));
  void* kp = b.get(ch * dk * 2);
  void* q = b.get(ch * dk * 2);
  void* k = b.get(ch * dk * 2);
  void* v = b.get(ch * dv * 2);
  float* o = static_cast<float*>(b.get(ch * dv * 4));
  void* xh = b.get(ch * 3 * dk * 2);
  void* yh = b.get(ch * 3 * dv * 2);
  expect("decode null S", falcon_decode_step(FALCON_1, 0.5f, nullptr, 0, 0.01f, 1e-6f, nseq, heads, dk, dv, 0,
                                             nullptr, kp, q, k, v, o, nullptr),
         FALCON_ERR_INVALID_ARG);
  expect("decode k_prev aliases k", falcon_decode_step(FALCON_1, 0.5f, nullptr, 0, 0.01f, 1e-6f, nseq, heads, dk,
                                                       dv, 0, S, k, q, k, v, o, nullptr),
         FALCON_ERR_INVALID_ARG);
  expect("decode window variant", falcon_decode_step(FALCON_3, 0.5f, nullptr, 0, 0.01f, 1e-6f, nseq, heads, dk,
                                                     dv, 0, S, kp, q, k, v, o, nullptr),
         FALCON_ERR_UNSUPPORTED);
  expect("decode well-formed", falcon_decode_step(FALCON_1, 0.5f, nullptr, 0, 0.01f, 1e-6f, nseq, heads, dk, dv, 0,
                                                  S, kp, q, k, v, o, nullptr),
         FALCON_ERR_HIP);
  expect("decode_ex window 4 without history",
         falcon_decode_step_ex(FALCON_3, 4, 0, 0.5f, nullptr, 0, 0.01f, 1e-6f, nseq, heads, dk, dv, 0, S, kp,
                               nullptr, nullptr, q, k, v, o, nullptr),
         FALCON_ERR_INVALID_ARG);
  expect("decode_ex window 4 well-formed",
         falcon_decode_step_ex(FALCON_3, 4, 0, 0.5f, nullptr, 0, 0.01f, 1e-6f, nseq, heads, dk, dv, 0, S, kp, xh,
                               yh, q, k, v, o, nullptr),
         FALCON_ERR_HIP);
}

struct Bwd {
  int variant = FALCON_1, window = 1, flags = 0;
  int batch = 1, heads = 2, seqlen = 40, dk = 64, dv = 64;
  const void *q, *k, *v;
  const float* dO;
  float *dq, *dk_out, *dv_out;
};

void backward_cases(Buffers& b) {
  Bwd s;
  const size_t tok = (size_t)s.batch * s.heads * s.seqlen;
  s.q = b.get(tok * s.dk * 2);
  s.k = b.get(tok * s.dk * 2);
  s.v = b.get(tok * s.dv * 2);
  s.dO = static_cast<const float*>(b.get(tok * s.dv * 4));
  s.dq = static_cast<float*>(b.get(tok * s.dk * 4));
  s.dk_out = static_cast<float*>(b.get(tok * s.dk * 4));
  s.dv_out = static_cast<float*>(b.get(tok * s.dv * 4));
  const unsigned long long need = falcon_bwd_workspace_bytes(s.batch, s.heads, s.seqlen, s.dk, s.dv, s.window);
  expect("bwd workspace bytes positive", need > 0, 1);
  void* ws = b.get(need);
  auto bwd = [&](const Bwd& a, void* w, unsigned long long wb) {
    return falcon_bwd_chunk(a.variant, a.window, a.flags, 0.5f, nullptr, 0, 0.01f, 1e-6f, a.batch, a.heads,
                            a.seqlen, a.dk, a.dv, 0, a.q, a.k, a.v, nullptr, nullptr, a.dO, nullptr, nullptr, a.dq,
                            a.dk_out, a.dv_out, nullptr, nullptr, nullptr, w, wb, nullptr);
  };
  auto noalloc = [&](const Bwd& a) {
    return falcon_bwd_chunk_noalloc(a.variant, a.window, a.flags, 0.5f, nullptr, 0, 0.01f, 1e-6f, a.batch,
                                    a.heads, a.seqlen, a.dk, a.dv, 0, a.q, a.k, a.v, nullptr, nullptr, a.dO,
                                    nullptr, nullptr, a.dq, a.dk_out, a.dv_out, nullptr, nullptr, nullptr,
                                    nullptr);
  };
  expect("bwd null workspace", bwd(s, nullptr, need), FALCON_ERR_INVALID_ARG);
  expect("bwd short workspace", bwd(s, ws, need - 1), FALCON_ERR_INVALID_ARG);
  Bwd t = s;
  t.dq = static_cast<float*>(const_cast<void*>(s.q));
  expect("bwd dq aliases q", bwd(t, ws, need), FALCON_ERR_INVALID_ARG);
  t = s;
  t.window = 9;
  t.variant = FALCON_3;
  expect("bwd window 9", bwd(t, ws, need), FALCON_ERR_UNSUPPORTED);
  expect("bwd well-formed", bwd(s, ws, need), FALCON_ERR_HIP);
  t = s;
  t.seqlen = 1 << 30;
  expect("bwd sizes beyond the buffers overlap", noalloc(t), FALCON_ERR_INVALID_ARG);
  // a sequence whose workspace exceeds the fixed scratch array: stand-in
  // addresses 2^36 bytes apart (compared, never dereferenced)
  t = s;
  t.seqlen = 1 << 16;
  const unsigned long long big = falcon_bwd_workspace_bytes(t.batch, t.heads, t.seqlen, t.dk, t.dv, t.window);
  expect("bwd workspace of 65536 steps above the scratch", big > FALCON_BWD_SCRATCH_BYTES, 1);
  auto far = [](int i) { return reinterpret_cast<void*>((uintptr_t)(1ull << 44) + (uintptr_t)i * (1ull << 36)); };
  t.q = far(0);
  t.k = far(1);
  t.v = far(2);
  t.dO = static_cast<const float*>(far(3));
  t.dq = static_cast<float*>(far(4));
  t.dk_out = static_cast<float*>(far(5));
  t.dv_out = static_cast<float*>(far(6));
  expect("noalloc above its scratch", noalloc(t), FALCON_ERR_UNSUPPORTED);
  expect("bwd with a caller workspace, same sizes", bwd(t, far(7), big), FALCON_ERR_HIP);
  expect("noalloc well-formed (no device address)", noalloc(s), FALCON_ERR_HIP);
}

}  // namespace

int main() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    // stand-in pointers are host memory: never reach a real launch
    std::printf("a GPU is present: this host-only check does not run here\n");
    return 77;
  }
  expect("abi version", falcon_abi_version(), FALCON_ABI_VERSION);
  for (int st = -1; st <= 4; ++st) expect("status string non-null", falcon_status_string(st) != nullptr, 1);
  {
    Buffers b;
    seq_cases("falcon_fwd_recurrent", call_recurrent, b, false);
    seq_cases("falcon_fwd_chunk", call_chunk, b, true);
    seq_cases("falcon_fwd_recurrent_ex", call_recurrent_ex, b, false);
    seq_cases("falcon_fwd_chunk_ex", call_chunk_ex, b, true);
    seq_cases("falcon_fwd_masked", call_masked, b, false);
    history_cases("falcon_fwd_recurrent_ex", call_recurrent_ex, b, false);
    history_cases("falcon_fwd_chunk_ex", call_chunk_ex, b, false);
    history_cases("falcon_fwd_masked", call_masked, b, true);
    workspace_cases(b);
    decode_cases(b);
    backward_cases(b);
  }
  std::printf("%d checks, %d failures\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}
