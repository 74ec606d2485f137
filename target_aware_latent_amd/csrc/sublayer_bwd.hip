// Row movement of the attention-sublayer backward ([LLaTTE] Appendix A.3,
// pre-norm layer of Appendix A.2): the query rows of a layer are each
// user's last n_u history rows plus its candidate rows; the forward reads
// them from the normed rows of every history row, and the backward sends
// their gradients back to those rows.
#include "backward.hpp"

namespace llatte {

// Block (u, g): user u's rows g, g + G, ... of its K_u history rows (query
// rows copied, every row's qmap entry written) and of its candidates, in
// 16-byte pieces.
__global__ __launch_bounds__(256) void gather_query_rows_kernel(const bf16* Hc, const bf16* H,
                                                                const int* kv_off, const int* hq_off,
                                                                int B, int n_cand, int d, bf16* Hq,
                                                                int* qmap) {
  const int u = blockIdx.x, G = gridDim.y, g = blockIdx.y;
  const int kv0 = kv_off[u], K = kv_off[u + 1] - kv0, hq0 = hq_off[u], n = hq_off[u + 1] - hq0;
  const int pieces = d / 8, nc = B * n_cand;
  for (int j = g; j < K + n_cand; j += G) {
    const bf16* src;
    size_t dst;
    if (j < K) {
      const int t = j - (K - n);  // query row index within the user, if >= 0
      if (threadIdx.x == 0) qmap[kv0 + j] = t >= 0 ? nc + hq0 + t : -1;
      if (t < 0) continue;
      src = H + (size_t)(kv0 + j) * d;
      dst = (size_t)(nc + hq0 + t) * d;
    } else {
      const int crow = u * n_cand + (j - K);
      src = Hc + (size_t)crow * d;
      dst = (size_t)crow * d;
    }
    for (int c = threadIdx.x; c < pieces; c += 256) *(bf16x8*)(Hq + dst + c * 8) = *(const bf16x8*)(src + c * 8);
  }
}

hipError_t gather_query_rows(const bf16* Hc, const bf16* H, const int* kv_off, const int* hq_off,
                             int B, int n_cand, int d, bf16* Hq, int* qmap, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  timing_begin("gather_q", s);
  hipLaunchKernelGGL(gather_query_rows_kernel, dim3(B, 32), dim3(256), 0, s, Hc, H, kv_off, hq_off, B,
                     n_cand, d, Hq, qmap);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace llatte
