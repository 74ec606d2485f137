// Sequence summaries ([LLaTTE] Appendix A.2 item 4: LoRAMLP_k over the
// flattened readout). With base weights shared by the summaries and rank-rho
// adapters per summary,
//   LoRAMLP_k(x) = GELU(x (W1 + A1_k B1_k)) (W2 + A2_k B2_k),
// the adapted weights are merged once at packing time, transposed into the
// tiled products' K-contiguous layout; a forward is then two batched
// products over the K summaries.
#include "kernels.hpp"

namespace llatte {

// out[k][i][j] = W[j][i] + sum_r A[k][j][r] Bm[k][r][i]   (fp32 sums, stored
// in the dtype). W [rows, cols], A [K, rows, rank], Bm [K, rank, cols];
// out [K, cols, rows]. 32 x 32 tiles: W and Bm are read along i, out is
// written along j, through an LDS transpose (33-float rows: no bank
// conflicts on the column reads).
template <typename T>
__global__ __launch_bounds__(256) void lora_merge_kernel(const T* W, const T* A, const T* Bm,
                                                         int rows, int cols, int rank, T* out) {
  __shared__ float tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int i0 = blockIdx.x * 32, j0 = blockIdx.y * 32, k = blockIdx.z;
  const T* Ak = A + (size_t)k * rows * rank;
  const T* Bk = Bm + (size_t)k * rank * cols;
  const int i = i0 + tx;
#pragma unroll
  for (int jj = ty; jj < 32; jj += 8) {
    const int j = j0 + jj;
    float v = 0.f;
    if (i < cols && j < rows) {
      v = tof(W[(size_t)j * cols + i]);
      for (int r = 0; r < rank; ++r)
        v = fmaf(tof(Ak[(size_t)j * rank + r]), tof(Bk[(size_t)r * cols + i]), v);
    }
    tile[jj][tx] = v;
  }
  __syncthreads();
  T* ok = out + (size_t)k * cols * rows;
  const int j = j0 + tx;
#pragma unroll
  for (int ii = ty; ii < 32; ii += 8) {
    const int i2 = i0 + ii;
    if (i2 < cols && j < rows) ok[(size_t)i2 * rows + j] = cvt<T>(tile[tx][ii]);
  }
}

hipError_t lora_merge(const void* W, const void* A, const void* Bm, int rows, int cols,
                      int rank, int K, void* out, bool is_bf16, hipStream_t s) {
  if (rows <= 0 || cols <= 0 || K <= 0) return hipSuccess;
  const dim3 grid((cols + 31) / 32, (rows + 31) / 32, K);
  timing_begin("lora_merge", s);
  if (is_bf16)
    hipLaunchKernelGGL(lora_merge_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)W,
                       (const bf16*)A, (const bf16*)Bm, rows, cols, rank, (bf16*)out);
  else
    hipLaunchKernelGGL(lora_merge_kernel<float>, grid, dim3(256), 0, s, (const float*)W,
                       (const float*)A, (const float*)Bm, rows, cols, rank, (float*)out);
  timing_end(s);
  return hipGetLastError();
}

// dst (dtype) = src (float32), n elements, four per thread (16-byte loads
// where src is 16-byte aligned and n a multiple of four; one by one for the
// tail otherwise).
template <typename T>
__global__ __launch_bounds__(256) void cast_kernel(const float* src, T* dst, long long n) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  if (i + 4 <= n && ((uintptr_t)(src + i) & 15) == 0) {
    const f32x4 v = *(const f32x4*)(src + i);
    typedef T T4 __attribute__((ext_vector_type(4)));
    T4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = cvt<T>(v[k]);
    if (((uintptr_t)(dst + i) & (4 * sizeof(T) - 1)) == 0) {
      *(T4*)(dst + i) = o;
      return;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[i + k] = o[k];
    return;
  }
  for (long long k = i; k < n && k < i + 4; ++k) dst[k] = cvt<T>(src[k]);
}

hipError_t cast_f32(const float* src, void* dst, long long n, bool is_bf16, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 1023) / 1024);
  timing_begin("cast", s);
  if (is_bf16)
    hipLaunchKernelGGL(cast_kernel<bf16>, dim3(grid), dim3(256), 0, s, src, (bf16*)dst, n);
  else
    hipLaunchKernelGGL(cast_kernel<float>, dim3(grid), dim3(256), 0, s, src, (float*)dst, n);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace llatte
