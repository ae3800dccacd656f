// falcon_launch.h - internal interface between the C-ABI layer (falcon_api.cpp)
// and the kernel launchers.  Arguments are already validated when these run.
#pragma once
#include <hip/hip_runtime.h>

namespace falcon {

// Arguments of one sequence call (recurrent or chunk form).
struct SeqArgs {
  int variant;       // falcon_variant
  int window;        // B
  int regression;    // 1: Falcon-1/2/3, 0: Falcon-1A/2A/3A
  float beta;        // scalar gain (beta_kind == 0)
  const void* beta_t;
  int beta_kind;     // 0 scalar, 1 per token, 2 per token and value channel
  float lambda, eps;
  int batch, heads, seqlen, dk, dv;
  int dtype;         // 0 bf16, 1 fp32
  const void* q;
  const void* k;
  const void* v;
  const void* k_prev;  // may be null
  const float* S0;     // may be null
  float* o;
  float* S_out;        // may be null
  int chunk;           // chunk form only
  // window history of a resumed Falcon-3/3A sequence: the window-1 samples
  // (x_j, y_j) before step 1, oldest first, [chain][window-1][dk or dv]; null:
  // none (zero samples)
  const void* x_hist = nullptr;
  const void* y_hist = nullptr;
  // sample pairing: x_t = k_{t - key_shift}; 1 = the previous key (x_1 = k_prev
  // or 0), 0 = the same step's key
  int key_shift = 1;
};

struct DecodeArgs {
  int regression;
  int window;        // 1, or B > 1 with x_hist / y_hist
  void* x_hist;      // [nseq*heads][window-1][dk], oldest first, updated in place
  void* y_hist;      // [nseq*heads][window-1][dv]
  float beta;
  const void* beta_t;
  int beta_kind;
  float lambda, eps;
  int nseq, heads, dk, dv;
  int dtype;
  float* S;
  void* k_prev;
  const void* q;
  const void* k;
  const void* v;
  float* o;
  int key_shift;     // 1: x = k_prev (then k_prev <- k); 0: x = k, k_prev unused
};

// Backward of the chunk form, windows 1..8 (falcon_backward.hip).
struct BwdArgs {
  int regression;
  int window;        // 1..8
  int key_shift;
  float beta;
  const void* beta_t;
  int beta_kind;
  float lambda, eps;
  int batch, heads;
  long seqlen;
  int ndk, ndv;      // sizes
  int dtype;
  const void* q;
  const void* k;
  const void* v;
  const void* k_prev;
  const float* S0;
  const float* dO;
  const float* dS_L;     // may be null
  const float* dk_last;  // may be null
  float* dq;
  float* dk;
  float* dv;
  float* dbeta_t;        // may be null
  float* dk_prev;        // may be null
  float* dS0;            // may be null
  float* workspace;      // backward_workspace_bytes(...)
};
size_t backward_workspace_bytes(int batch, int heads, long seqlen, int dk, int dv, int window);
// Largest per-chain buffer range the backward kernel addresses (bytes); the
// kernel needs it below 2^30.
size_t backward_chain_bytes(long seqlen, int dk, int dv, int window, int dtype);
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream);

hipError_t launch_recurrent(const SeqArgs& a, hipStream_t stream);
// masked-parallel form, the whole call one masked system (falcon_masked.hip):
// seqlen 1..kMaskedMaxLen, window 1..8
constexpr int kMaskedMaxLen = 64;
hipError_t launch_masked(const SeqArgs& a, hipStream_t stream);
// workspace (optional): the two-kernel sliding-window form runs where it applies and
// ws_bytes >= chunk_wyb2_workspace_bytes(a)
hipError_t launch_chunk(const SeqArgs& a, hipStream_t stream, void* ws = nullptr, size_t ws_bytes = 0);
// window-1 chunk form, per-channel gains (falcon_chunk_w1.hip); cs = sub-chunk length
hipError_t launch_chunk_w1(const SeqArgs& a, hipStream_t stream, int cs);
// window-1 chunk form, gains shared by the value rows, dk in {32, 64}
// (falcon_chunk_wy.hip); 32-step chunks whatever the requested chunk
bool chunk_wy_supported(const SeqArgs& a);
hipError_t launch_chunk_wy(const SeqArgs& a, hipStream_t stream);
// sliding-window chunk form (window 2 or 4), gains shared by the value rows, dk in
// {64, 128} (falcon_chunk_wyb.hip); 16-step sub-chunks whatever the requested chunk
bool chunk_wyb_supported(const SeqArgs& a);
hipError_t launch_chunk_wyb(const SeqArgs& a, hipStream_t stream);
// the same in two kernels (regression family): a pre-pass writes every
// sub-chunk's folds to a workspace, a state kernel runs the sequential part;
// the workspace bytes it needs (0 where it does not apply) and its launch
size_t chunk_wyb2_workspace_bytes(const SeqArgs& a);
hipError_t launch_chunk_wyb2(const SeqArgs& a, void* workspace, hipStream_t stream);
// inner-product family, any window up to 16, gains shared by the value rows, dk in
// {64, 128}, dv a multiple of 32 (falcon_chunk_ip.hip); 64-step chunks
bool chunk_ip_supported(const SeqArgs& a);
hipError_t launch_chunk_ip(const SeqArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// the window-1 latest samples after a sequence call, written to x_out / y_out
// (which may equal a.x_hist / a.y_hist); enqueue after the call's kernel
hipError_t launch_history_out(const SeqArgs& a, void* x_out, void* y_out, hipStream_t stream);

}  // namespace falcon
