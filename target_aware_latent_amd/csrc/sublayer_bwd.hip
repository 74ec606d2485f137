// Row movement of the attention-sublayer backward ([LLaTTE] Appendix A.3,
// pre-norm layer of Appendix A.2): the query rows of a layer are each
// user's last n_u history rows plus its candidate rows; the forward reads
// them from the normed rows of every history row, and the backward sends
// their gradients back to those rows.
#include "backward.hpp"

namespace llatte {

// Block (u, g): user u's candidate rows and history query rows g, g + G, ...
// of it, in 16-byte pieces.
__global__ __launch_bounds__(256) void gather_query_rows_kernel(const bf16* Hc, const bf16* H,
                                                                const int* kv_off, const int* hq_off,
                                                                int B, int n_cand, int d, bf16* Hq,
                                                                int* hist_map) {
  const int u = blockIdx.x, G = gridDim.y, g = blockIdx.y;
  const int kv0 = kv_off[u], K = kv_off[u + 1] - kv0, hq0 = hq_off[u], n = hq_off[u + 1] - hq0;
  const int pieces = d / 8, nc = B * n_cand;
  const int rows = n + n_cand;
  for (int t = g; t < rows; t += G) {
    const bf16* src;
    size_t dst;
    if (t < n) {
      const int hrow = kv0 + K - n + t;
      src = H + (size_t)hrow * d;
      dst = (size_t)(nc + hq0 + t) * d;
      if (threadIdx.x == 0) hist_map[hq0 + t] = hrow;
    } else {
      const int crow = u * n_cand + (t - n);
      src = Hc + (size_t)crow * d;
      dst = (size_t)crow * d;
    }
    for (int c = threadIdx.x; c < pieces; c += 256) *(bf16x8*)(Hq + dst + c * 8) = *(const bf16x8*)(src + c * 8);
  }
}

hipError_t gather_query_rows(const bf16* Hc, const bf16* H, const int* kv_off, const int* hq_off,
                             int B, int n_cand, int d, bf16* Hq, int* hist_map, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  timing_begin("gather_q", s);
  hipLaunchKernelGGL(gather_query_rows_kernel, dim3(B, 32), dim3(256), 0, s, Hc, H, kv_off, hq_off, B,
                     n_cand, d, Hq, hist_map);
  timing_end(s);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void scatter_query_rows_kernel(const float* dHq, const float* dRq,
                                                                 const int* hist_map, long long nh,
                                                                 long long nc, int d, float* dH,
                                                                 float* dres) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const int q4 = d / 4;
  if (e >= nh * q4) return;
  const long long j = e / q4;
  const int c = (int)(e % q4) * 4;
  const size_t dst = (size_t)hist_map[j] * d + c, src = (size_t)(nc + j) * d + c;
  *(f32x4*)(dH + dst) += *(const f32x4*)(dHq + src);
  *(f32x4*)(dres + dst) = *(const f32x4*)(dRq + src);
}

hipError_t scatter_query_rows(const float* dHq, const float* dRq, const int* hist_map, long long nh,
                              long long nc, int d, float* dH, float* dres, hipStream_t s) {
  if (nh <= 0) return hipSuccess;
  const long long n = nh * (d / 4);
  timing_begin("scatter_q", s);
  hipLaunchKernelGGL(scatter_query_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     dHq, dRq, hist_map, nh, nc, d, dH, dres);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace llatte
