// Backward of the pre-norm FFN sublayer ([LLaTTE] Appendix A.2 layer
// equation, pre-norm reading): R2 = R1 + GELU(RMSNorm(R1) g2 W1) W2, over M
// independent rows. Given d_out = dL/dR2 it produces dR1, dg2, dW1 and dW2:
//   s = (mean(R1^2) + eps)^-1/2,  xh = R1 s,  H2 = xh g2,  A = H2 W1,
//   dW2 = GELU(A)^T d_out,   dG = d_out W2^T,   dA = dG GELU'(A),
//   dW1 = H2^T dA,           dH2 = dA W1^T,
//   dg2 = sum_rows dH2 xh,   dR1 = d_out + s (dH2 g2 - xh mean(dH2 g2 xh)).
// The forward's H2 and A are recomputed (the row norm, one product). The
// recomputation and the input gradients run on the tiled bf16 GEMM (both
// operands K-contiguous), the input gradients with W1 [d, d_ff] and
// W2 [d_ff, d] in their natural row-major layout; the product dG writes
// dA = dG GELU'(A) and GELU(A) from its epilogue (A recomputed as bf16).
// The weight gradients contract over the rows on the weight-gradient
// kernel, which reads the row-major activations directly. The norm
// backward is an HBM-bound kernel of its own.
#include "backward.hpp"

namespace llatte {

// RMSNorm backward with the residual (dres, optional), one wave per row,
// kNormRows rows per block; with qmap, row i also takes dh_q and dres_q of
// row qmap[i] when that is >= 0 (a layer's query rows feeding back into
// its input rows): s = 1 / sqrt(ss / d + eps), xh = x s, dxh = dh g,
// dx = dres + s (dxh - xh mean(dxh xh)); and the block's partial sums of
// dh * xh per column (the gain's gradient), summed over the block's rows in
// row order and then over its waves in wave order.
constexpr int kNormRows = 64;
// G row groups per wave (64 / G lanes per row; G = 2 for rows of at most
// 128), two rows per group in flight at a time: a wave's 16 rows take 8 / G
// iterations, each loading its rows before reducing them. A lane holds MAXV
// chunks of four columns per row (rows of at most 4 MAXV 64 / G), so that
// narrower rows keep fewer registers and more waves per SIMD.
template <int G, int MAXV>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const float* x, const float* ss,
                                                         const float* dh, const float* g,
                                                         const float* dres, float eps, int M,
                                                         int d, float* dx, float* dg_part,
                                                         const int* qmap, const float* dh_q,
                                                         const float* dres_q) {
  constexpr int LG = 64 / G;               // lanes per row
  constexpr int STRIDE = 4 * LG;           // columns between a lane's chunks
  __shared__ float red[4][1024];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = lane / LG, gl = lane % LG;
  f32x4 acc[MAXV], gv[MAXV];
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    acc[j] = f32x4{};
    const int idx = j * STRIDE + gl * 4;
    gv[j] = idx < d ? *(const f32x4*)(g + idx) : f32x4{};
  }
  const int r0 = blockIdx.x * kNormRows + wave * (kNormRows / 4);
  // the row map of the wave's 16 rows, loaded once (lane j holds row r0 + j),
  // so that no iteration waits for it before loading the mapped rows
  constexpr int WR = kNormRows / 4;
  const int qm = qmap && lane < WR && r0 + lane < M ? qmap[r0 + lane] : -1;
  for (int i = 0; i < kNormRows / 4 / (2 * G); ++i) {
    int row[2], qi[2];
    float sc[2];
    f32x4 xh[2][MAXV], hv[2][MAXV], rs[2][MAXV];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      row[u] = r0 + (2 * i + u) * G + grp;
      const bool ok = row[u] < M;
      sc[u] = ok ? 1.f / sqrtf(ss[row[u]] / (float)d + eps) : 0.f;
      qi[u] = __shfl(qm, row[u] - r0, 64);
      if (!ok) qi[u] = -1;
#pragma unroll
      for (int j = 0; j < MAXV; ++j) {
        const int idx = j * STRIDE + gl * 4;
        xh[u][j] = hv[u][j] = rs[u][j] = f32x4{};
        if (ok && idx < d) {
          const size_t o = (size_t)row[u] * d + idx;
          xh[u][j] = *(const f32x4*)(x + o) * sc[u];
          hv[u][j] = *(const f32x4*)(dh + o);
          if (dres) rs[u][j] = *(const f32x4*)(dres + o);
          if (qi[u] >= 0) {
            const size_t oq = (size_t)qi[u] * d + idx;
            hv[u][j] += *(const f32x4*)(dh_q + oq);
            rs[u][j] += *(const f32x4*)(dres_q + oq);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float dot = 0.f;
#pragma unroll
      for (int j = 0; j < MAXV; ++j) {
        const f32x4 dxh = hv[u][j] * gv[j];
#pragma unroll
        for (int k = 0; k < 4; ++k) dot = fmaf(dxh[k], xh[u][j][k], dot);
      }
#pragma unroll
      for (int o = 1; o < LG; o <<= 1) dot += __shfl_xor(dot, o, 64);
      const float mean = dot / (float)d;
      if (row[u] >= M) continue;
#pragma unroll
      for (int j = 0; j < MAXV; ++j) {
        const int idx = j * STRIDE + gl * 4;
        if (idx >= d) continue;
        *(f32x4*)(dx + (size_t)row[u] * d + idx) = rs[u][j] + (hv[u][j] * gv[j] - xh[u][j] * mean) * sc[u];
        acc[j] += hv[u][j] * xh[u][j];
      }
    }
  }
  if constexpr (G == 2) {
#pragma unroll
    for (int j = 0; j < MAXV; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[j][k] += __shfl_xor(acc[j][k], 32, 64);
  }
  if (grp == 0) {
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
      const int idx = j * STRIDE + gl * 4;
      if (idx < d) *(f32x4*)&red[wave][idx] = acc[j];
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += 256)
    dg_part[(size_t)blockIdx.x * d + c] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
}

// out[c] = sum over p of part[p][c]: 64 columns per block; each of sixteen
// thread rows sums a contiguous sixteenth of the partials in order, then the
// sixteen sums are added in order (a fixed order: the result is
// reproducible).
__global__ __launch_bounds__(1024) void colsum_kernel(const float* part, int np, int d, float* out) {
  __shared__ float q[16][64];
  const int t = threadIdx.x & 63, ty = threadIdx.x >> 6, c = blockIdx.x * 64 + t;
  const int per = (np + 15) / 16, p0 = ty * per, p1 = min(np, p0 + per);
  float v = 0.f;
  if (c < d) {
#pragma unroll 8
    for (int p = p0; p < p1; ++p) v += part[(size_t)p * d + c];
  }
  q[ty][t] = v;
  __syncthreads();
  if (ty == 0 && c < d) {
    float acc = 0.f;
    for (int i = 0; i < 16; ++i) acc += q[i][t];
    out[c] = acc;
  }
}

__global__ __launch_bounds__(256) void zero_kernel(float* p, long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

namespace {

size_t up256(size_t b) { return (b + 255) & ~(size_t)255; }

struct FfnWs {
  bf16 *H2, *W1T, *dOb, *A, *dA, *G;
  float *ss, *dH2, *dg_part, *sk;
  size_t bytes;
};

FfnWs ffn_ws(char* base, long long M, int d, int F) {
  const size_t nb = (size_t)((M + kNormRows - 1) / kNormRows);
  FfnWs w{};
  size_t o = 0;
  auto take = [&](size_t b) {
    char* p = base ? base + o : nullptr;
    o += up256(b);
    return p;
  };
  w.H2 = (bf16*)take((size_t)M * d * 2);
  w.W1T = (bf16*)take((size_t)F * d * 2);
  w.dOb = (bf16*)take((size_t)M * d * 2);
  w.A = (bf16*)take((size_t)M * F * 2);
  w.dA = (bf16*)take((size_t)M * F * 2);
  w.G = (bf16*)take((size_t)M * F * 2);
  w.ss = (float*)take((size_t)M * 4);
  w.dH2 = (float*)take((size_t)M * d * 4);
  w.dg_part = (float*)take(nb * d * 4);
  w.sk = (float*)take((size_t)kFfnSkPart * 4);
  w.bytes = o;
  return w;
}

GemmParams plain_gemm(const void* A, int lda, const void* B, int ldb, int M, int N, int K, void* C,
                      int ldc, const char* name, float* sk) {
  GemmParams g;
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.M_cap = M;
  g.N = N;
  g.K = K;
  g.epi = EPI_STORE_F32;
  g.C = C;
  g.ldc = ldc;
  g.name = name;
  g.sk_part = sk;
  g.sk_part_cap = kFfnSkPart;
  return g;
}

}  // namespace

size_t ffn_backward_workspace(long long M, int d, int F) { return ffn_ws(nullptr, M, d, F).bytes; }

int rmsnorm_backward_parts(long long M) { return (int)((M + kNormRows - 1) / kNormRows); }

// The instance for the row width: two row groups per wave for d <= 128,
// else one, with the fewest column chunks per lane that cover d.
static void launch_rmsnorm_bwd(const float* x, const float* ss, const float* dh, const float* g,
                               const float* dres, float eps, long long M, int d, float* dx,
                               float* dg_part, const int* qmap, const float* dh_q,
                               const float* dres_q, hipStream_t s) {
  const dim3 grid(rmsnorm_backward_parts(M));
  if (d <= 128)
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<2, 1>), grid, dim3(256), 0, s, x, ss, dh, g, dres, eps,
                       (int)M, d, dx, dg_part, qmap, dh_q, dres_q);
  else if (d <= 512)
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<1, 2>), grid, dim3(256), 0, s, x, ss, dh, g, dres, eps,
                       (int)M, d, dx, dg_part, qmap, dh_q, dres_q);
  else
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<1, 4>), grid, dim3(256), 0, s, x, ss, dh, g, dres, eps,
                       (int)M, d, dx, dg_part, qmap, dh_q, dres_q);
}

hipError_t rmsnorm_backward(const float* x, const float* ss, const float* dh, const float* g,
                            const float* dres, float eps, long long M, int d, float* dx,
                            float* dg_part, hipStream_t s, const int* qmap, const float* dh_q,
                            const float* dres_q) {
  if (M <= 0) return hipSuccess;
  timing_begin("rmsnorm_bwd", s);
  launch_rmsnorm_bwd(x, ss, dh, g, dres, eps, M, d, dx, dg_part, qmap, dh_q, dres_q, s);
  timing_end(s);
  return hipGetLastError();
}

hipError_t column_sum(const float* part, int np, int d, float* out, hipStream_t s) {
  hipLaunchKernelGGL(colsum_kernel, dim3((d + 63) / 64), dim3(1024), 0, s, part, np, d, out);
  return hipGetLastError();
}

hipError_t zero_f32(float* p, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t ffn_backward(const FfnBwdParams& p, void* ws, hipStream_t s) {
  const long long M = p.M;
  const int d = p.d, F = p.F;
  if (M <= 0) {
    // no rows: the weight gradients are zero (a fill kernel, so that the
    // call stays capturable in a graph)
    const long long n = (long long)d * F;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p.dW1, n);
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p.dW2, n);
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((d + 255) / 256)), dim3(256), 0, s, p.dg2,
                       (long long)d);
    return hipGetLastError();
  }
  FfnWs w = ffn_ws((char*)ws, M, d, F);
  hipError_t e;
  // H2 = RMSNorm(R1) g2 (bf16) and the rows' sums of squares
  if ((e = norm_rows(RowSrc{p.r1, p.r1, 0, d}, (int)M, nullptr, p.g2, p.eps, nullptr, 0, w.H2, d,
                     d, K_BF16, s, w.ss)))
    return e;
  // W1^T [F, d] for the recomputed A = H2 W1
  if ((e = transpose(p.w1, d, F, F, 0, w.W1T, d, 0, 1, K_BF16, K_BF16, s))) return e;
  {
    // the pre-activation A (bf16)
    GemmParams g = plain_gemm(w.H2, d, w.W1T, d, (int)M, F, d, w.A, F, "gemm_bwd_a", nullptr);
    g.epi = EPI_STORE;
    if ((e = gemm(g, true, s))) return e;
  }
  // d_out as bf16; dG = d_out W2^T (B = W2 [F, d] as stored), whose
  // epilogue writes dA = dG GELU'(A) and GELU(A)
  if ((e = cast_f32(p.dout, w.dOb, M * d, true, s))) return e;
  {
    GemmParams g = plain_gemm(w.dOb, d, p.w2, d, (int)M, F, d, w.dA, F, "gemm_bwd_dg", nullptr);
    g.epi = EPI_GELU_BWD;
    g.nt = true;  // dA and GELU(A) stream to HBM (read by later kernels, not this one)
    g.table = w.A;
    g.ld_table = F;
    g.cast_out = w.G;
    g.ld_cast = F;
    if ((e = gemm(g, true, s))) return e;
  }
  // dW2 [F, d] = GELU(A)^T d_out and dW1 [d, F] = H2^T dA (over the rows)
  auto wg = [&](const bf16* X, int n1, const bf16* Y, int n2, float* C, const char* name) {
    WgradParams g;
    g.X = X;
    g.ldx = n1;
    g.Y = Y;
    g.ldy = n2;
    g.M = M;
    g.N1 = n1;
    g.N2 = n2;
    g.C = C;
    g.ldc = n2;
    g.part = w.sk;
    g.part_cap = kFfnSkPart;
    g.name = name;
    return wgrad(g, s);
  };
  if ((e = wg(w.G, F, w.dOb, d, p.dW2, "gemm_bwd_dw2"))) return e;
  if ((e = wg(w.H2, d, w.dA, F, p.dW1, "gemm_bwd_dw1"))) return e;
  // dH2 = dA W1^T: B = W1 [d, F] as stored
  if ((e = gemm(plain_gemm(w.dA, F, p.w1, F, (int)M, d, F, w.dH2, d, "gemm_bwd_dh", nullptr), true, s)))
    return e;
  const int nb = (int)((M + kNormRows - 1) / kNormRows);
  timing_begin("rmsnorm_bwd", s);
  launch_rmsnorm_bwd(p.r1, w.ss, w.dH2, p.g2, p.dout, p.eps, M, d, p.dr1, w.dg_part, nullptr, nullptr,
                     nullptr, s);
  hipLaunchKernelGGL(colsum_kernel, dim3((d + 63) / 64), dim3(1024), 0, s, w.dg_part, nb, d, p.dg2);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace llatte
