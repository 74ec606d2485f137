// Weight gradients of the backward: C[i][j] = sum over rows m of X[m][i] Y[m][j]
// (C = X^T Y), for X [M, N1] and Y [M, N2] bf16 row-major, C float. The
// contraction runs over the rows, so both MFMA operands are read from
// row-major LDS tiles with the gfx950 transpose load: within each 16-lane
// group, lane i receives column i of the 4 x 16 block whose rows (here:
// consecutive m) the group's lanes address. Two such reads (rows 4g.. and
// 16 + 4g.. of a 32-row step) give a lane eight m values of one column, in
// the same order for both operands, which is all a contraction needs. No
// transposed copy of X or Y is written.
//
// Block: 256 threads, a 128 x 128 tile of C, four waves of 64 x 64 (4 x 4
// blocks of the 16x16x32 bf16 MFMA); 32 rows per step, double-buffered LDS
// with register prefetch. The rows split across blocks (grid.y) when the
// tiles alone leave the GPU idle; each split stores its fp32 tile and a
// second kernel adds the splits in order (reproducible) and writes C.
// grid.z runs over a batch (e.g. heads) with element strides.
#include "backward.hpp"

namespace llatte {

namespace {

constexpr int kWT = 128;        // C tile edge
constexpr int kWK = 32;         // rows per step
constexpr int kWLD = kWT + 16;  // LDS row (bf16): 72 banks, 8 modulo 64

typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 wg_hx4;
typedef __attribute__((address_space(3))) wg_hx4 wg_lds_hx4;
typedef __attribute__((address_space(3))) f16 wg_lds_f16;

__device__ __forceinline__ bf16x4 wg_tr(const bf16* p) {
  auto q = (wg_lds_hx4*)((wg_lds_f16*)(f16*)p);
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(q));
}

}  // namespace

__global__ __launch_bounds__(256, 2) void wgrad_kernel(WgradParams p) {
  __shared__ __attribute__((aligned(16))) bf16 Xs[2][kWK * kWLD];
  __shared__ __attribute__((aligned(16))) bf16 Ys[2][kWK * kWLD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int tiles2 = (p.N2 + kWT - 1) / kWT;
  const int i0 = (blockIdx.x / tiles2) * kWT, j0 = (blockIdx.x % tiles2) * kWT;
  const int b = blockIdx.z;
  const bf16* X = p.X + (size_t)b * p.sX;
  const bf16* Y = p.Y + (size_t)b * p.sY;
  // this split's rows
  const int nsteps_all = (p.M + kWK - 1) / kWK;
  const int per = (nsteps_all + gridDim.y - 1) / gridDim.y;
  const int s0 = blockIdx.y * per, s1 = min(nsteps_all, s0 + per);
  const int nsteps = max(0, s1 - s0);

  // staging: a 32 x 128 tile is 512 pieces of 8 elements, two per thread
  bf16x8 rx[2], ry[2];
  auto gload = [&](int st) {
    const int m0 = (s0 + st) * kWK;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = tid + 256 * k, r = e >> 4, c = (e & 15) * 8, m = m0 + r;
      const bool okm = m < p.M;
      rx[k] = okm && i0 + c < p.N1 ? *(const bf16x8*)(X + (size_t)m * p.ldx + i0 + c) : bf16x8{};
      ry[k] = okm && j0 + c < p.N2 ? *(const bf16x8*)(Y + (size_t)m * p.ldy + j0 + c) : bf16x8{};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = tid + 256 * k, r = e >> 4, c = (e & 15) * 8;
      *(bf16x8*)&Xs[buf][r * kWLD + c] = rx[k];
      *(bf16x8*)&Ys[buf][r * kWLD + c] = ry[k];
    }
  };
  const int wi = (wave >> 1) * 64, wj = (wave & 1) * 64;  // the wave's 64 x 64 corner
  const int trow = 4 * lg + (lr >> 2), tcol = (lr & 3) * 4;
  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = f32x4{};

  if (nsteps > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    if (st + 1 < nsteps) gload(st + 1);
    const bf16* xs = Xs[buf];
    const bf16* ys = Ys[buf];
    bf16x8 ya[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = wj + c * 16 + tcol;
      ya[c] = bf16x8{};
      const bf16x4 lo = wg_tr(ys + trow * kWLD + col), hi = wg_tr(ys + (16 + trow) * kWLD + col);
      ya[c] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int col = wi + a * 16 + tcol;
      const bf16x4 lo = wg_tr(xs + trow * kWLD + col), hi = wg_tr(xs + (16 + trow) * kWLD + col);
      const bf16x8 xa{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, ya[c], acc[a][c], 0, 0, 0);
    }
    if (st + 1 < nsteps) lstore(buf ^ 1);
    __syncthreads();
  }
  // lane holds C[i0 + wi + 16a + 4lg + e][j0 + wj + 16c + lr]
  if (gridDim.y > 1) {
    const size_t tile = (size_t)b * gridDim.x + blockIdx.x;
    f32x4* mine = (f32x4*)(p.part + (tile * gridDim.y + blockIdx.y) * (size_t)(kWT * kWT)) + tid * 16;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) mine[a * 4 + c] = acc[a][c];
    return;
  }
  float* C = p.C + (size_t)b * p.sC;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = j0 + wj + 16 * c + lr;
      if (j >= p.N2) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + wi + 16 * a + 4 * lg + e;
        if (i < p.N1) C[(size_t)i * p.ldc + j] = acc[a][c][e];
      }
    }
}

// Sums the splits of each tile in split order and writes C. The partial
// tiles hold each thread's 16 accumulators contiguously; reduce block
// (tile, part) takes the accumulators of the sixteen threads
// 16 part .. 16 part + 15, one f32x4 per thread, so a tile's sum spreads
// over sixteen workgroups.
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(WgradParams p, int nsplit) {
  const int tiles2 = (p.N2 + kWT - 1) / kWT;
  const int i0 = (blockIdx.x / tiles2) * kWT, j0 = (blockIdx.x % tiles2) * kWT;
  const int b = blockIdx.z;
  const size_t tile = (size_t)b * gridDim.x + blockIdx.x;
  const int ot = blockIdx.y * 16 + (threadIdx.x >> 4), k = threadIdx.x & 15;  // owner thread, slot
  const f32x4* src = (const f32x4*)(p.part + tile * nsplit * (size_t)(kWT * kWT)) + ot * 16 + k;
  f32x4 acc = src[0];
  for (int sp = 1; sp < nsplit; ++sp) acc += src[(size_t)sp * (kWT * kWT / 4)];
  // the owner's lane mapping: C[i0 + wi + 16a + 4lg + e][j0 + wj + 16c + lr], k = 4a + c
  const int lane = ot & 63, wave = ot >> 6, lr = lane & 15, lg = lane >> 4;
  const int a = k >> 2, c = k & 3;
  const int j = j0 + (wave & 1) * 64 + 16 * c + lr;
  if (j >= p.N2) return;
  float* C = p.C + (size_t)b * p.sC;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = i0 + (wave >> 1) * 64 + 16 * a + 4 * lg + e;
    if (i < p.N1) C[(size_t)i * p.ldc + j] = acc[e];
  }
}

int wgrad_splits(long long M, int N1, int N2, int batch, long long part_cap) {
  const long long tiles = (long long)((N1 + kWT - 1) / kWT) * ((N2 + kWT - 1) / kWT) * batch;
  const long long steps = (M + kWK - 1) / kWK;
  long long sp = std::max<long long>(1, 512 / std::max<long long>(tiles, 1));
  sp = std::min<long long>({sp, 64, std::max<long long>(1, steps / 8)});
  while (sp > 1 && tiles * sp * kWT * kWT > part_cap) --sp;
  return (int)sp;
}

hipError_t wgrad(WgradParams p, hipStream_t s) {
  if (p.N1 <= 0 || p.N2 <= 0 || p.batch <= 0) return hipSuccess;
  const int tiles = ((p.N1 + kWT - 1) / kWT) * ((p.N2 + kWT - 1) / kWT);
  const int sp = p.part ? wgrad_splits(p.M, p.N1, p.N2, p.batch, p.part_cap) : 1;
  timing_begin(p.name, s);
  hipLaunchKernelGGL(wgrad_kernel, dim3(tiles, sp, p.batch), dim3(256), 0, s, p);
  if (sp > 1) hipLaunchKernelGGL(wgrad_reduce_kernel, dim3(tiles, 16, p.batch), dim3(256), 0, s, p, sp);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace llatte
