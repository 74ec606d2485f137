// Launcher interfaces of the training backward (attention core, FFN
// sublayer) between the C-ABI layer and their HIP kernels.
#pragma once
#include "kernels.hpp"

namespace llatte {

// ------------------------------------------------------------------ attention backward
// Gradients of the latent attention core (bf16 q / c, fp32 out, lse, dout;
// fp32 dq [Mtot, h, r] and dc [Ktot, r]); rows and masks as the forward.
struct AttnBwdParams {
  const void* q = nullptr;     // [Mtot, h, r] bf16
  const void* c = nullptr;     // [Ktot, r] bf16
  const float* out = nullptr;  // [Mtot, h, r]
  const float* lse = nullptr;  // [Mtot, h] natural log
  const float* dout = nullptr; // [Mtot, h, r]
  float* dq = nullptr;
  float* dc = nullptr;
  const int* kv_off = nullptr;
  const int* hq_off = nullptr;
  int B = 0, n_cand = 0, h = 0, r = 0;
  long long Mtot = 0;
  float scale = 1.f;
  // set by attention_backward from the workspace: d_out as bf16 high and
  // low parts [Mtot, h, r], D = d_out . out [Mtot, h]
  bf16* ws_ghi = nullptr;
  bf16* ws_glo = nullptr;
  float* ws_d = nullptr;
  bool dc_accumulate = false;  // d_C from two head groups, added onto zero
};
// Workspace bytes of attention_backward.
size_t attention_backward_workspace(long long Mtot, int h, int r);
hipError_t attention_backward(AttnBwdParams p, int max_len, void* ws, hipStream_t s);

// ------------------------------------------------------------------ FFN backward
// Gradients of R2 = R1 + GELU(RMSNorm(R1) g2 W1) W2 over M rows (bf16
// operands, fp32 accumulation and outputs).
struct FfnBwdParams {
  const float* r1 = nullptr;    // [M, d]
  const float* g2 = nullptr;    // [d]
  const void* w1 = nullptr;     // [d, F] bf16
  const void* w2 = nullptr;     // [F, d] bf16
  const float* dout = nullptr;  // [M, d]
  float* dr1 = nullptr;         // [M, d]
  float* dg2 = nullptr;         // [d]
  float* dW1 = nullptr;         // [d, F]
  float* dW2 = nullptr;         // [F, d]
  long long M = 0;
  int d = 0, F = 0;
  float eps = 0.f;
};
constexpr long long kFfnSkPart = 1ll << 22;  // split-K scratch (floats)
size_t ffn_backward_workspace(long long M, int d, int F);
hipError_t ffn_backward(const FfnBwdParams& p, void* ws, hipStream_t s);

}  // namespace llatte
