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
  bf16* dq_bf16 = nullptr;  // when set, d_q goes here rounded to bf16 instead of to dq
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
constexpr long long kFfnSkPart = 1ll << 23;  // split-K scratch (floats)
size_t ffn_backward_workspace(long long M, int d, int F);
hipError_t ffn_backward(const FfnBwdParams& p, void* ws, hipStream_t s);


// ------------------------------------------------------------------ shared pieces
// RMSNorm backward over M rows of width d (<= 1024, multiple of 4):
// dx = dres + s (dh g - xh mean(dh g xh)) with s from ss = sum(x^2) per
// row (dres optional), and per-block partial column sums of dh * xh in
// dg_part [rmsnorm_backward_parts(M), d]. With qmap, row i with
// qmap[i] >= 0 adds row qmap[i] of dh_q to dh and of dres_q to dres.
int rmsnorm_backward_parts(long long M);
hipError_t rmsnorm_backward(const float* x, const float* ss, const float* dh, const float* g,
                            const float* dres, float eps, long long M, int d, float* dx,
                            float* dg_part, hipStream_t s, const int* qmap = nullptr,
                            const float* dh_q = nullptr, const float* dres_q = nullptr);
// out[c] = sum over p < np of part[p][c] in a fixed order.
hipError_t column_sum(const float* part, int np, int d, float* out, hipStream_t s);
hipError_t zero_f32(float* p, long long n, hipStream_t s);

// ------------------------------------------------------------------ weight gradients
// C [N1, N2] (float, row stride ldc) = X^T Y over M rows, X [M, N1] and
// Y [M, N2] bf16 row-major (row strides ldx, ldy; multiples of 8, as are N1
// and N2), for `batch` problems whose operands advance by sX, sY, sC
// elements. With part (part_cap floats of scratch) the rows split across
// the GPU and the splits are added in order.
struct WgradParams {
  const bf16* X = nullptr;
  int ldx = 0;
  long long sX = 0;
  const bf16* Y = nullptr;
  int ldy = 0;
  long long sY = 0;
  long long M = 0;
  int N1 = 0, N2 = 0, batch = 1;
  float* C = nullptr;
  int ldc = 0;
  long long sC = 0;
  float* part = nullptr;
  long long part_cap = 0;
  const char* name = "wgrad";
};
hipError_t wgrad(WgradParams p, hipStream_t s);

// ------------------------------------------------------------------ attention sublayer
// Hq [Mtot, d] (bf16) = the candidate rows Hc [B*n_cand, d], then user u's
// last n_u rows of H (H row kv_off[u] + K_u - n_u + t goes to row
// B*n_cand + hq_off[u] + t); qmap[H row] = that query row, or -1 for the
// user's other rows (every H row is written). d is a multiple of 8.
hipError_t gather_query_rows(const bf16* Hc, const bf16* H, const int* kv_off, const int* hq_off,
                             int B, int n_cand, int d, bf16* Hq, int* qmap, hipStream_t s);

}  // namespace llatte
