// Attention in latent space: the core of the absorbed MLA form (LLaTTE,
// Appendix A.3: MLA equals multi-query attention on the latent). Every head
// scores its latent query against the same latent rows C and averages C
// itself, so one C tile in LDS serves all heads of a query block.
//
// bf16 kernel (MFMA), one workgroup per work item (a block of query rows of
// one user, all heads of a head group), four waves, each wave owning EPW
// (query row, head) pairs ("effective rows"):
//   S^T = C_tile . Q^T          v_mfma_f32_16x16x32_bf16, A = C rows from LDS,
//                               B = latent queries held in registers
//   online softmax per column   (fp32, exp2, max/sum over the four lane
//                               groups of a column with two xor shuffles)
//   O^T += C_tile^T . P^T       A = C^T from a transposed LDS copy, B = P^T
//                               straight from the S^T accumulators
// Computing the transposed products keeps each lane's softmax column and its
// output column the same effective row, so the rescale needs no shuffles,
// and P never goes through LDS. The C tile is staged twice per step
// (row-major for S^T, transposed for O^T), double-buffered; the transpose is
// done while writing LDS from registers. Masks: history rows attend keys up
// to their own position (causal, LLaTTE Appendix A.2); candidate rows attend
// every key of their user.
//
// fp32 kernel: one wave per (query row, head), keys 64 at a time, plain
// online softmax. It serves the fp32 path only.
#include "kernels.hpp"

namespace llatte {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

template <int R, int EPW, typename OutT>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnParams p, int HG,
                                                        int hg_shift) {
  constexpr int BN = kAttnBN;        // keys per tile
  constexpr int LDC = R + 8;         // row-major C tile pitch (elements)
  constexpr int LDT = BN + 8;        // transposed C tile pitch
  constexpr int NEB = EPW / 16;      // effective-row blocks per wave
  constexpr int NKS = R / 32;        // 32-wide r steps
  constexpr int NRB = R / 16;        // 16-wide r blocks of the output
  constexpr int NLD = (2 * R + 255) / 256;  // 4-key x 8-r load blocks/thread

  __shared__ __attribute__((aligned(16))) bf16 Cs[2][BN * LDC];
  __shared__ __attribute__((aligned(16))) bf16 Ct[2][R * LDT];

  const int nitems = min(*p.n_items, p.items_cap);
  if ((int)blockIdx.x >= nitems) return;
  const i32x4 it = p.items[blockIdx.x];
  const int qrow0 = it[0], kvb = it[1];
  const bool cand = it[2] < 0;
  const int nr = it[2] & 0x7fffffff;
  const int pos0 = it[3];
  const int h0 = blockIdx.y * HG;
  const int max_pos = cand ? pos0 : pos0 + nr - 1;
  const int nkeys = max_pos + 1;
  const int ntiles = (nkeys + BN - 1) / BN;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;

  const bf16* Q = (const bf16*)p.q;
  const bf16* Cg = (const bf16*)p.c + (size_t)kvb * R;

  // Effective rows of this lane (one per block eb): e = wave*EPW + eb*16 + l16
  // -> query row ql = e >> hg_shift, head h0 + (e & (HG-1)).
  int pos[NEB];
  bool valid[NEB];
  bf16x8 qf[NEB][NKS];
  int pmin = 0x7fffffff;
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) {
    const int e = wave * EPW + eb * 16 + l16;
    const int ql = e >> hg_shift, hl = e & (HG - 1);
    valid[eb] = ql < nr;
    const int qc = min(ql, nr - 1);
    pos[eb] = cand ? pos0 : pos0 + qc;
    pmin = min(pmin, pos[eb]);
    const bf16* qp = Q + ((size_t)(qrow0 + qc) * p.h + h0 + hl) * R + g * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[eb][ks] = *(const bf16x8*)(qp + ks * 32);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) pmin = min(pmin, __shfl_xor(pmin, o, 64));

  // Tile loads: block b covers keys 4*kq .. 4*kq+3 and r 8*rc .. 8*rc+7.
  i32x4 ld[NLD][4];
  auto load_tile = [&](int t) {
    const int k0 = t * BN;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int b = tid + i * 256;
      const int rc = b % (R / 8), kq = b / (R / 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = k0 + kq * 4 + j;
        ld[i][j] = (b < 2 * R && key < nkeys)
                       ? *(const i32x4*)(Cg + (size_t)key * R + rc * 8)
                       : i32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int b = tid + i * 256;
      if (b >= 2 * R) continue;
      const int rc = b % (R / 8), kq = b / (R / 8);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *(i32x4*)&Cs[buf][(kq * 4 + j) * LDC + rc * 8] = ld[i][j];
      bf16x8 v0 = __builtin_bit_cast(bf16x8, ld[i][0]);
      bf16x8 v1 = __builtin_bit_cast(bf16x8, ld[i][1]);
      bf16x8 v2 = __builtin_bit_cast(bf16x8, ld[i][2]);
      bf16x8 v3 = __builtin_bit_cast(bf16x8, ld[i][3]);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *(bf16x4*)&Ct[buf][(rc * 8 + e) * LDT + kq * 4] =
            bf16x4{v0[e], v1[e], v2[e], v3[e]};
    }
  };

  f32x4 acc_o[NRB][NEB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) acc_o[rb][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NEB], l_run[NEB];
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) {
    m_run[eb] = -INFINITY;
    l_run[eb] = 0.f;
  }
  const float sc = p.scale * kLog2e;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const bf16* cs = Cs[cur];
    const bf16* ct = Ct[cur];

    // S^T[key][e] for the 64 keys of this tile
    f32x4 s[4][NEB];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) s[kb][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 a = *(const bf16x8*)&cs[(kb * 16 + l16) * LDC + ks * 32 + g * 8];
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb)
          s[kb][eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[eb][ks], s[kb][eb], 0, 0, 0);
      }
    }

    // online softmax per effective row (this lane's column of S^T)
    const bool need_mask = t * BN + BN - 1 > pmin;
    bf16x8 pf[2][NEB];
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float x = s[kb][eb][v] * sc;
          if (need_mask) {
            const int key = t * BN + kb * 16 + g * 4 + v;
            if (key > pos[eb]) x = -INFINITY;
          }
          s[kb][eb][v] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[eb], mx);
      const float alpha = fast_exp2(m_run[eb] - m_new);
      m_run[eb] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float e = fast_exp2(s[kb][eb][v] - m_new);
          rs += e;
          pf[kb >> 1][eb][(kb & 1) * 4 + v] = to_bf16(e);
        }
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      l_run[eb] = l_run[eb] * alpha + rs;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) acc_o[rb][eb] *= alpha;
      }
    }

    // O^T[r][e] += sum over keys of C^T[r][key] * P^T[key][e]
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16* row = &ct[(rb * 16 + l16) * LDT + kk * 32 + g * 4];
        const bf16x4 lo = *(const bf16x4*)row;
        const bf16x4 hi = *(const bf16x4*)(row + 16);
        const bf16x8 a = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb)
          acc_o[rb][eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[kk][eb], acc_o[rb][eb], 0, 0, 0);
      }
    }

    if (t + 1 < ntiles) store_tile(cur ^ 1);
    __syncthreads();
  }

  // normalise and store: lane holds out[e][rb*16 + 4g .. +3]
  OutT* O = (OutT*)p.out;
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) {
    if (!valid[eb]) continue;
    const int e = wave * EPW + eb * 16 + l16;
    const int ql = e >> hg_shift, hl = e & (HG - 1);
    const size_t orow = (size_t)(qrow0 + ql) * p.h + h0 + hl;
    const float inv = 1.f / l_run[eb];
    OutT* op = O + orow * R + g * 4;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const f32x4 v = acc_o[rb][eb];
      if constexpr (sizeof(OutT) == 2)
        *(bf16x4*)(op + rb * 16) =
            bf16x4{to_bf16(v[0] * inv), to_bf16(v[1] * inv), to_bf16(v[2] * inv),
                   to_bf16(v[3] * inv)};
      else
        *(f32x4*)(op + rb * 16) = v * inv;
    }
    if (p.lse && g == 0) p.lse[orow] = (m_run[eb] + __log2f(l_run[eb])) * kLn2;
  }
}

// fp32: one wave per (query row, head).
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnParams p) {
  constexpr int RV = 4;  // r <= 256
  __shared__ float sq[256];
  __shared__ float sp[64];
  const int i = blockIdx.x, hh = blockIdx.y, lane = threadIdx.x;
  if (i >= dev_count(p.M_dev, p.M_cap)) return;
  const int r = p.r;
  const int2 info = p.qinfo[i];
  const int kvb = info.x, nkeys = info.y + 1;
  const float* q = (const float*)p.q + ((size_t)i * p.h + hh) * r;
  const float* C = (const float*)p.c + (size_t)kvb * r;
  for (int k = lane; k < r; k += 64) sq[k] = q[k];
  __syncthreads();
  float m = -INFINITY, l = 0.f;
  float o[RV] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < nkeys; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (j < nkeys) {
      const float* c = C + (size_t)j * r;
      float acc = 0.f;
      for (int k = 0; k < r; ++k) acc += sq[k] * c[k];
      s = acc * p.scale;
    }
    const float m_new = fmaxf(m, wave_max(s));
    const float alpha = expf(m - m_new);
    const float pj = j < nkeys ? expf(s - m_new) : 0.f;
    l = l * alpha + wave_sum(pj);
    m = m_new;
#pragma unroll
    for (int v = 0; v < RV; ++v) o[v] *= alpha;
    sp[lane] = pj;
    __syncthreads();
    const int nj = min(64, nkeys - j0);
    for (int jj = 0; jj < nj; ++jj) {
      const float w = sp[jj];
      const float* c = C + (size_t)(j0 + jj) * r;
#pragma unroll
      for (int v = 0; v < RV; ++v) {
        const int k = lane + 64 * v;
        if (k < r) o[v] += w * c[k];
      }
    }
    __syncthreads();
  }
  float* out = (float*)p.out + ((size_t)i * p.h + hh) * r;
  const float inv = 1.f / l;
#pragma unroll
  for (int v = 0; v < RV; ++v) {
    const int k = lane + 64 * v;
    if (k < r) out[k] = o[v] * inv;
  }
  if (p.lse && lane == 0) p.lse[(size_t)i * p.h + hh] = m + logf(l);
}

// Effective rows per wave and query rows per item of the bf16 kernel.
static int attn_epw(int r) { return r == 256 ? 32 : 64; }

static int heads_per_group(int h, int r) {
  // all heads of a query row in one workgroup when at least one query row
  // fits; otherwise the largest power-of-two divisor of h that fits
  const int eff = 4 * attn_epw(r);
  int hg = 1;
  while (hg * 2 <= h && h % (hg * 2) == 0 && hg * 2 <= eff) hg *= 2;
  return hg;
}

int attn_bq(int h, int r) {
  if (r != 64 && r != 128 && r != 256) return 0;
  return 4 * attn_epw(r) / heads_per_group(h, r);
}

template <int R, int EPW>
static void launch_bf16(const AttnParams& p, hipStream_t s) {
  const int hg = heads_per_group(p.h, R);
  int shift = 0;
  while ((1 << shift) < hg) ++shift;
  dim3 grid(p.items_cap, p.h / hg);
  if (p.out_f32)
    hipLaunchKernelGGL((attn_bf16_kernel<R, EPW, float>), grid, dim3(256), 0, s,
                       p, hg, shift);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<R, EPW, bf16>), grid, dim3(256), 0, s,
                       p, hg, shift);
}

hipError_t attention(const AttnParams& p, bool is_bf16, hipStream_t s) {
  if (p.M_cap <= 0) return hipSuccess;
  timing_begin(is_bf16 ? "attention_bf16" : "attention_f32", s);
  if (is_bf16) {
    if (p.items_cap > 0) {
      switch (p.r) {
        case 64: launch_bf16<64, 64>(p, s); break;
        case 128: launch_bf16<128, 64>(p, s); break;
        case 256: launch_bf16<256, 32>(p, s); break;
        default: timing_end(s); return hipErrorInvalidValue;
      }
    }
  } else {
    hipLaunchKernelGGL(attn_f32_kernel, dim3(p.M_cap, p.h), dim3(64), 0, s, p);
  }
  timing_end(s);
  return hipGetLastError();
}

}  // namespace llatte
