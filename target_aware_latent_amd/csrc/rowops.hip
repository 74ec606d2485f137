// Row-wise, HBM-bound kernels: RMSNorm / cast of residual rows, weight
// transposes, and the small assembly copies around the layer stack.
#include "kernels.hpp"

namespace llatte {

// One wave per row, four rows per workgroup. Each lane owns float4 chunks
// lane*4 + 256*j of the row, so a row of d floats is read once, reduced with
// wave shuffles, and written as dtype and/or float (and its sum of squares).
// RMSNorm (Root Mean Square Layer Normalization): x / sqrt(mean(x^2) + eps) * g.
template <typename T>
__global__ __launch_bounds__(256) void norm_rows_kernel(
    RowSrc src, int rows_cap, const int* rows_dev, const float* gain,
    float eps, float* out_f32, int ld_f32, T* out_t, int ld_t, int d,
    float* ss_out) {
  constexpr int MAXV = 4;  // d <= 4 * 256 = 1024
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= dev_count(rows_dev, rows_cap)) return;
  const float* x = src.row(row);
  f32x4 v[MAXV];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int idx = j * 256 + lane * 4;
    v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (idx < d) {
      v[j] = *(const f32x4*)(x + idx);
      ss += v[j][0] * v[j][0] + v[j][1] * v[j][1] + v[j][2] * v[j][2] +
            v[j][3] * v[j][3];
    }
  }
  float scale = 1.f;
  if (gain || ss_out) {
    ss = wave_sum(ss);
    if (gain) scale = 1.f / sqrtf(ss / (float)d + eps);
    if (ss_out && lane == 0) ss_out[row] = ss;
  }
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int idx = j * 256 + lane * 4;
    if (idx >= d) continue;
    f32x4 y = v[j];
    if (gain) {
      f32x4 g = *(const f32x4*)(gain + idx);
      y = f32x4{y[0] * scale * g[0], y[1] * scale * g[1], y[2] * scale * g[2],
                y[3] * scale * g[3]};
    }
    if (out_f32) *(f32x4*)(out_f32 + (size_t)row * ld_f32 + idx) = y;
    if (out_t) {
      typedef T T4 __attribute__((ext_vector_type(4)));
      *(T4*)(out_t + (size_t)row * ld_t + idx) =
          T4{cvt<T>(y[0]), cvt<T>(y[1]), cvt<T>(y[2]), cvt<T>(y[3])};
    }
  }
}

hipError_t norm_rows(RowSrc src, int rows_cap, const int* rows_dev,
                     const float* gain, float eps, float* out_f32, int ld_f32,
                     void* out_t, int ld_t, int d, int t_kind, hipStream_t s,
                     float* ss_out) {
  if (rows_cap <= 0) return hipSuccess;
  dim3 grid((rows_cap + 3) / 4);
  timing_begin("norm_rows", s);
  if (t_kind == K_BF16)
    hipLaunchKernelGGL(norm_rows_kernel<bf16>, grid, dim3(256), 0, s, src,
                       rows_cap, rows_dev, gain, eps, out_f32, ld_f32,
                       (bf16*)out_t, ld_t, d, ss_out);
  else if (t_kind == K_F16)
    hipLaunchKernelGGL(norm_rows_kernel<f16>, grid, dim3(256), 0, s, src,
                       rows_cap, rows_dev, gain, eps, out_f32, ld_f32,
                       (f16*)out_t, ld_t, d, ss_out);
  else
    hipLaunchKernelGGL(norm_rows_kernel<float>, grid, dim3(256), 0, s, src,
                       rows_cap, rows_dev, gain, eps, out_f32, ld_f32,
                       (float*)out_t, ld_t, d, ss_out);
  timing_end(s);
  return hipGetLastError();
}

// 32x32 tiles through LDS (one padding column against bank conflicts).
template <typename S, typename T>
__global__ __launch_bounds__(256) void transpose_kernel(
    const S* src, int rows, int cols, int ld_src, long long s_src, T* dst,
    int ld_dst, long long s_dst, const float* row_scale) {
  __shared__ T tile[32][33];
  src += (size_t)blockIdx.z * s_src;
  dst += (size_t)blockIdx.z * s_dst;
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols)
      tile[i][tx] = cvt<T>(tof(src[(size_t)r * ld_src + c]) * (row_scale ? row_scale[r] : 1.f));
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    int c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) dst[(size_t)c * ld_dst + r] = tile[tx][i];
  }
}

hipError_t transpose(const void* src, int rows, int cols, int ld_src,
                     long long s_src, void* dst, int ld_dst, long long s_dst,
                     int batch, int s_kind, int d_kind, hipStream_t s,
                     const float* row_scale) {
  if (rows <= 0 || cols <= 0 || batch <= 0) return hipSuccess;
  dim3 grid((cols + 31) / 32, (rows + 31) / 32, batch);
  timing_begin("transpose", s);
  if (s_kind == K_BF16 && d_kind == K_BF16)
    hipLaunchKernelGGL((transpose_kernel<bf16, bf16>), grid, dim3(256), 0, s,
                       (const bf16*)src, rows, cols, ld_src, s_src, (bf16*)dst,
                       ld_dst, s_dst, row_scale);
  else if (s_kind == K_BF16 && d_kind == K_F16)
    hipLaunchKernelGGL((transpose_kernel<bf16, f16>), grid, dim3(256), 0, s,
                       (const bf16*)src, rows, cols, ld_src, s_src, (f16*)dst,
                       ld_dst, s_dst, row_scale);
  else if (s_kind == K_F32 && d_kind == K_F32)
    hipLaunchKernelGGL((transpose_kernel<float, float>), grid, dim3(256), 0, s,
                       (const float*)src, rows, cols, ld_src, s_src,
                       (float*)dst, ld_dst, s_dst, row_scale);
  else
    return hipErrorInvalidValue;
  timing_end(s);
  return hipGetLastError();
}

template <typename T>
__global__ void concat_kernel(const float* cand, const float* ctx, int B,
                              int n_q, int d, int d_c, T* xc) {
  const int w = d + d_c;
  const long long total = (long long)B * n_q * w;
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const int row = (int)(e / w), k = (int)(e % w);
    const float v = k < d ? cand[(size_t)row * d + k]
                          : ctx[(size_t)(row / n_q) * d_c + (k - d)];
    xc[e] = cvt<T>(v);
  }
}

hipError_t concat_queries(const float* cand, const float* ctx, int B, int n_q,
                          int d, int d_c, void* xc, bool is_bf16,
                          hipStream_t s) {
  const long long total = (long long)B * n_q * (d + d_c);
  if (total == 0) return hipSuccess;
  int blocks = (int)std::min<long long>((total + 255) / 256, 65536);
  timing_begin("concat_queries", s);
  if (is_bf16)
    hipLaunchKernelGGL(concat_kernel<bf16>, dim3(blocks), dim3(256), 0, s, cand,
                       ctx, B, n_q, d, d_c, (bf16*)xc);
  else
    hipLaunchKernelGGL(concat_kernel<float>, dim3(blocks), dim3(256), 0, s,
                       cand, ctx, B, n_q, d, d_c, (float*)xc);
  timing_end(s);
  return hipGetLastError();
}

__global__ void broadcast_kernel(const float* seeds, int n_s, int d, int B,
                                 float* out) {
  const long long total = (long long)B * n_s * d;
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x)
    out[e] = seeds[e % ((long long)n_s * d)];
}

hipError_t broadcast_rows(const float* seeds, int n_s, int d, int B, float* out,
                          hipStream_t s) {
  const long long total = (long long)B * n_s * d;
  if (total == 0) return hipSuccess;
  int blocks = (int)std::min<long long>((total + 255) / 256, 65536);
  timing_begin("broadcast_rows", s);
  hipLaunchKernelGGL(broadcast_kernel, dim3(blocks), dim3(256), 0, s, seeds,
                     n_s, d, B, out);
  timing_end(s);
  return hipGetLastError();
}

__global__ void copy_rows_kernel(const float* src, int ld, float* dst,
                                 int count_cap, const int* count_dev, int d) {
  const int rows = dev_count(count_dev, count_cap);
  const long long total = (long long)rows * d;
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const long long r = e / d, k = e % d;
    dst[e] = src[r * ld + k];
  }
}

hipError_t copy_rows_f32(const float* src, int ld, float* dst, int count_cap,
                         const int* count_dev, int d, hipStream_t s) {
  const long long total = (long long)count_cap * d;
  if (total == 0) return hipSuccess;
  int blocks = (int)std::min<long long>((total + 255) / 256, 65536);
  timing_begin("copy_rows", s);
  hipLaunchKernelGGL(copy_rows_kernel, dim3(blocks), dim3(256), 0, s, src, ld,
                     dst, count_cap, count_dev, d);
  timing_end(s);
  return hipGetLastError();
}

// out[a][c] = sum over b < nb of src[(a sa + b sb) ld + col0 + c], c < width,
// a < na, b in increasing order (one thread per output element).
__global__ void group_sum_kernel(const float* src, int ld, int col0, int na, int sa, int nb,
                                 int sb, int width, float* out) {
  const long long total = (long long)na * width;
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const long long a = e / width, c = e % width;
    float t = 0.f;
    for (int b = 0; b < nb; ++b) t += src[(a * sa + (long long)b * sb) * ld + col0 + c];
    out[e] = t;
  }
}

hipError_t group_sum_rows(const float* src, int ld, int col0, int na, int sa, int nb, int sb,
                          int width, float* out, hipStream_t s) {
  const long long total = (long long)na * width;
  if (total == 0) return hipSuccess;
  int blocks = (int)std::min<long long>((total + 255) / 256, 65536);
  timing_begin("group_sum_rows", s);
  hipLaunchKernelGGL(group_sum_kernel, dim3(blocks), dim3(256), 0, s, src, ld, col0, na, sa, nb,
                     sb, width, out);
  timing_end(s);
  return hipGetLastError();
}

__global__ void add_kernel(float* dst, const float* src, long long n) {
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x)
    dst[e] += src[e];
}

hipError_t add_f32(float* dst, const float* src, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int blocks = (int)std::min<long long>((n + 255) / 256, 65536);
  timing_begin("add", s);
  hipLaunchKernelGGL(add_kernel, dim3(blocks), dim3(256), 0, s, dst, src, n);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace llatte
