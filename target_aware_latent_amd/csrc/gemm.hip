// Tiled matrix product on the gfx950 matrix cores, with fused epilogues.
//
// Both operands are K-contiguous (A [M, K], B [N, K]); weights are brought to
// this layout once by the packing step. A workgroup of four waves computes a
// BM x BN tile; K advances in BK steps through a double-buffered LDS stage.
// A tile row is 128 bytes (eight 16-byte chunks) with chunk c of row r
// stored at c ^ ((r >> 1) & 7): with 64 four-byte banks, a 16-lane pass of
// fragment reads (16 rows, one chunk) and of staging writes (2 rows, 8
// chunks) each covers all 64 banks once. The MFMA is
// issued with the operands swapped (B fragment first) so that each lane ends
// up holding four consecutive output columns of one row: the epilogue then
// reads residuals and writes results as 8- or 16-byte vectors.
//
// bf16 operands use v_mfma_f32_16x16x32_bf16; fp32 operands use
// v_mfma_f32_16x16x4_f32. Accumulation is fp32 in both cases.
#include <algorithm>
#include <type_traits>
#include <vector>

#include "kernels.hpp"

namespace llatte {

template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
  static constexpr int KSTEP = 32;   // k per instruction
  static constexpr int VEC = 8;      // k values per lane
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static constexpr int KSTEP = 4;
  static constexpr int VEC = 1;
  typedef float frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// erf by Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26 (|error| <= 1.5e-7): for z >= 0, erf(z) = 1 - t (a1 + t (a2 + t (a3
// + t (a4 + t a5)))) exp(-z^2), t = 1 / (1 + p z); odd in z.
__device__ __forceinline__ float erf_as(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(1.f + 0.3275911f * az);
  const float poly =
      t * (0.254829592f +
           t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float e = __builtin_amdgcn_exp2f(-az * az * 1.4426950408889634f);
  return copysignf(1.f - poly * e, z);
}

// GELU with the exact (erf) form, x * Phi(x).
__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.f + erf_as(x * 0.70710678118654752f));
}

// The same on the bf16 path, written as x Phi(x) = max(x, 0) - |x| Q(|x|)
// with the normal tail Q(u) = erfc(u / sqrt 2) / 2 from Abramowitz & Stegun
// formula 7.1.25 (erfc(z) = t (a1 + t (a2 + t a3)) exp(-z^2), t = 1 / (1 +
// p z), |error| <= 2.5e-5, far below the bf16 rounding of the result): nine
// VALU operations and two transcendentals per element. p and a_i are
// pre-scaled for z = u / sqrt 2 and the factor 1/2.
__device__ __forceinline__ float gelu_erf_bf16(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.47047f * 0.70710678118654752f, ax, 1.f));
  const float q = t * fmaf(t, fmaf(t, 0.5f * 0.7478556f, 0.5f * -0.0958798f), 0.5f * 0.3480242f);
  const float e = __builtin_amdgcn_exp2f(x * x * (-0.5f * 1.4426950408889634f));
  return fmaf(-(ax * q), e, __builtin_elementwise_maximum(x, 0.f));  // no quieting pass
}
template <typename T> __device__ __forceinline__ float gelu_t(float x) {
  if constexpr (__is_same(T, bf16)) return gelu_erf_bf16(x);
  else return gelu_erf(x);
}

// GELU(a) = a Phi(a) and its derivative Phi(a) + a phi(a) (erf form),
// elementwise: dg = d GELU'(a), g = GELU(a). On the bf16 path the normal
// tail Q(|a|) = q e comes from the same Abramowitz & Stegun 7.1.25 form as
// gelu_erf_bf16, and e = exp(-a^2 / 2) also gives the density
// phi(a) = e / sqrt(2 pi): Phi(a) = 1 - Q for a >= 0, else Q. Otherwise
// Phi from erf_as (formula 7.1.26).
template <typename T>
__device__ __forceinline__ void gelu_bwd4(f32x4 d, f32x4 a, f32x4& dg, f32x4& g) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float x = a[k];
    const float e = __builtin_amdgcn_exp2f(x * x * (-0.5f * 1.4426950408889634f));
    float Phi;
    if constexpr (__is_same(T, bf16)) {
      const float ax = fabsf(x);
      const float t = __builtin_amdgcn_rcpf(fmaf(0.47047f * 0.70710678118654752f, ax, 1.f));
      const float Q = t * fmaf(t, fmaf(t, 0.5f * 0.7478556f, 0.5f * -0.0958798f), 0.5f * 0.3480242f) * e;
      Phi = x >= 0.f ? 1.f - Q : Q;
    } else {
      Phi = 0.5f * (1.f + erf_as(x * 0.70710678118654752f));
    }
    dg[k] = d[k] * fmaf(x, e * 0.39894228040143268f, Phi);
    g[k] = x * Phi;
  }
}

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *(f32x4*)p = f32x4{a, b, c, d};
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, float a, float b, float c, float d) {
  *(bf16x4*)p = bf16x4{to_bf16(a), to_bf16(b), to_bf16(c), to_bf16(d)};
}
// The same with the non-temporal hint (streamed to memory, not kept in the
// caches); NT selects it at compile time.
template <bool NT, typename T>
__device__ __forceinline__ void store4h(T* p, float a, float b, float c, float d) {
  if constexpr (!NT) {
    store4<T>(p, a, b, c, d);
  } else if constexpr (__is_same(T, bf16)) {
    __builtin_nontemporal_store(bf16x4{to_bf16(a), to_bf16(b), to_bf16(c), to_bf16(d)}, (bf16x4*)p);
  } else {
    __builtin_nontemporal_store(f32x4{a, b, c, d}, (f32x4*)p);
  }
}
template <typename T> __device__ __forceinline__ f32x4 load4(const T* p);
template <> __device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *(const f32x4*)p;
}
template <> __device__ __forceinline__ f32x4 load4<bf16>(const bf16* p) {
  bf16x4 v = *(const bf16x4*)p;
  return f32x4{from_bf16(v[0]), from_bf16(v[1]), from_bf16(v[2]), from_bf16(v[3])};
}
// Four elements as stored (converted only where used, so that a load can
// stay in flight past a barrier).
template <typename T> struct Raw4 { typedef f32x4 type; };
template <> struct Raw4<bf16> { typedef bf16x4 type; };
__device__ __forceinline__ f32x4 widen4(f32x4 v) { return v; }
__device__ __forceinline__ f32x4 widen4(bf16x4 v) {
  return f32x4{from_bf16(v[0]), from_bf16(v[1]), from_bf16(v[2]), from_bf16(v[3])};
}

// Timestamp encoding of the action tokens ([LLaTTE] Appendix A.2, additive
// timestamp encodings on a subset of the hidden dimensions): columns
// 2i, 2i+1 < enc_dims of row m get sin / cos of
// (age / 3600) * 10000^(-2i / enc_dims). Ages span months, where an fp32
// angle would be off by 1e-3 rad: the angle is formed and reduced to a
// fraction of a turn in fp64, and the hardware sine / cosine (argument in
// turns) takes the reduced fp32 value.
__device__ __forceinline__ f32x4 add_time_enc(f32x4 x, const GemmParams& p, int m, int n) {
  if (!p.enc_age || n >= p.enc_dims) return x;
  const double turns_h = (double)p.enc_age[m] * (1.0 / (3600.0 * 6.283185307179586));
#pragma unroll
  for (int c = 0; c < 4; c += 2) {
    const int col = n + c;  // even: (sin, cos) of one frequency in col, col + 1
    if (col < p.enc_dims) {
      const double w = exp2(-(double)col / p.enc_dims * 13.287712379549449);  // log2 1e4
      double t = turns_h * w;
      t -= floor(t);
      const float tf = (float)t;
      x[c] += __builtin_amdgcn_sinf(tf);
      x[c + 1] += __builtin_amdgcn_cosf(tf);
    }
  }
  return x;
}

// Row-major epilogue. The fp32 accumulator tile goes through LDS (16-byte
// chunk c of row r stored at chunk c ^ (r & 15), so that both the fragment
// writes and the row reads below are free of bank conflicts) and comes back
// with LPR lanes per row, each lane holding chunks q and q + LPR of its row:
// every 16-lane group then reads and writes whole 256-byte runs of a row,
// and each row's RMSNorm sums reduce within its lane group.
template <typename T, int BM, int BN, int WM, int WN, int NW, bool NTS>
__device__ __forceinline__ void epilogue_rowmajor(const GemmParams p, const f32x4 (&acc)[WM / 16][WN / 16],
                                                  float* Cs, const float* rs_lds,
                                                  const int (&rrow)[BM / (64 * NW / (BN / 8))],
                                                  int m0, int n0, int M, int wm0, int wn0,
                                                  int lane, int tid) {
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int NT = 64 * NW;
  constexpr int CPR = BN / 4;       // 16-byte chunks per row
  constexpr int LPR = CPR / 2;      // lanes per row
  constexpr int RPP = NT / LPR;     // rows per pass
  constexpr int NPASS = BM / RPP;
  static_assert(LPR <= 64 && (LPR & (LPR - 1)) == 0 && BM % RPP == 0, "row-major epilogue shape");
  auto cidx = [](int row, int chunk) { return row * BN + ((chunk ^ (row & 15)) << 2); };
  const int lr = lane & 15;
  const int q = tid % LPR, rsub = tid / LPR;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      *(f32x4*)&Cs[cidx(wm0 + i * 16 + lr, ((wn0 + j * 16) >> 2) + (lane >> 4))] = acc[i][j];
  // Inputs the epilogue reads from memory (residual rows, gathered table
  // rows, the stored pre-activation) are loaded once the accumulators are in
  // LDS (their registers free) and before the barrier, so that their latency
  // overlaps the wait for the other waves.
  using R4 = typename Raw4<T>::type;
  f32x4 in[NPASS][2];  // residual rows (fp32)
  R4 tin[NPASS][2];    // table rows, as stored
  if (p.epi == EPI_RESID_F32) {
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int m = m0 + ps * RPP + rsub;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = n0 + (q + h * LPR) * 4;
        in[ps][h] = f32x4{};
        if (m < M && n < p.N) in[ps][h] = *(const f32x4*)(p.res.row(rrow[ps]) + n);
      }
    }
  } else if (p.epi == EPI_GATHER_ADD_F32 || p.epi == EPI_GELU_BWD) {
    const bool gather = p.epi == EPI_GATHER_ADD_F32;
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int m = m0 + ps * RPP + rsub;
      const size_t trow = (size_t)(gather ? rrow[ps] : m) * p.ld_table;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = n0 + (q + h * LPR) * 4;
        tin[ps][h] = R4{};
        if (m < M && n < p.N) tin[ps][h] = *(const R4*)((const T*)p.table + trow + n);
      }
    }
  }
  __syncthreads();

  const bool has_rs = p.rs.ss != nullptr;
  // values of this lane, scaled by the row scale
  f32x4 v[NPASS][2];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int row = ps * RPP + rsub;
    const float sc = has_rs ? rs_lds[row] : 1.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) v[ps][h] = *(const f32x4*)&Cs[cidx(row, q + h * LPR)] * sc;
  }
  auto each = [&](auto&& f) {  // f(ps, h, m, n) over this lane's valid outputs
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int m = m0 + ps * RPP + rsub;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = n0 + (q + h * LPR) * 4;
        if (m < M && n < p.N) f(ps, h, m, n);
      }
    }
  };
  // sum over the LPR lanes of a row (aligned groups of LPR lanes)
  auto row_sum = [&](float x) {
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) x += __shfl_xor(x, o, 64);
    return x;
  };
  auto coff = [&](int m, int n) { return (size_t)blockIdx.z * p.sC + (size_t)m * p.ldc + n; };
  switch (p.epi) {
    case EPI_STORE:
      each([&](int ps, int h, int m, int n) {
        const f32x4 x = v[ps][h] * p.alpha;
        store4h<NTS, T>((T*)p.C + coff(m, n), x[0], x[1], x[2], x[3]);
      });
      break;
    case EPI_STORE_F32:
      each([&](int ps, int h, int m, int n) {
        const f32x4 x = add_time_enc(v[ps][h] * p.alpha, p, m, n);
        store4<float>((float*)p.C + coff(m, n), x[0], x[1], x[2], x[3]);
      });
      break;
    case EPI_GELU:
      each([&](int ps, int h, int m, int n) {
        const f32x4 x = v[ps][h];
        store4h<NTS, T>((T*)p.C + coff(m, n), gelu_t<T>(x[0]), gelu_t<T>(x[1]), gelu_t<T>(x[2]),
                       gelu_t<T>(x[3]));
      });
      break;
    case EPI_RESID_F32: {
      float ssp[NPASS];
#pragma unroll
      for (int ps = 0; ps < NPASS; ++ps) ssp[ps] = 0.f;
      each([&](int ps, int h, int m, int n) {
        const f32x4 x = v[ps][h] + in[ps][h];
        store4h<NTS, float>((float*)p.C + coff(m, n), x[0], x[1], x[2], x[3]);
        if (p.cast_out)
          store4<T>((T*)p.cast_out + (size_t)m * p.ld_cast + n, x[0], x[1], x[2], x[3]);
        ssp[ps] += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
      });
      if (p.ss_out) {
        // one slot per (row, tile column)
        const int slot = n0 / BN;
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
          const float t = row_sum(ssp[ps]);
          const int m = m0 + ps * RPP + rsub;
          if (q == 0 && m < M) p.ss_out[(size_t)slot * p.ss_ld + m] = t;
        }
      }
    } break;
    case EPI_GATHER_ADD_F32: {
      each([&](int ps, int h, int m, int n) {
        const f32x4 x = v[ps][h] + widen4(tin[ps][h]);
        store4<float>((float*)p.C + coff(m, n), x[0], x[1], x[2], x[3]);
      });
    } break;
    case EPI_GELU_BWD: {
      each([&](int ps, int h, int m, int n) {
        f32x4 dg, g;
        gelu_bwd4<T>(v[ps][h], widen4(tin[ps][h]), dg, g);
        store4h<NTS, T>((T*)p.C + coff(m, n), dg[0], dg[1], dg[2], dg[3]);
        store4h<NTS, T>((T*)p.cast_out + (size_t)m * p.ld_cast + n, g[0], g[1], g[2], g[3]);
      });
    } break;
    case EPI_ROWNORM: {
      // RMSNorm over the row's N columns (with a gain this tile spans them)
      float sc[NPASS];
#pragma unroll
      for (int ps = 0; ps < NPASS; ++ps) {
        sc[ps] = 1.f;
        if (p.gain) {
          float t = 0.f;
#pragma unroll
          for (int h = 0; h < 2; ++h)
            if (n0 + (q + h * LPR) * 4 < p.N)
              t += v[ps][h][0] * v[ps][h][0] + v[ps][h][1] * v[ps][h][1] +
                   v[ps][h][2] * v[ps][h][2] + v[ps][h][3] * v[ps][h][3];
          sc[ps] = 1.f / sqrtf(row_sum(t) / (float)p.N + p.eps);
        }
      }
      each([&](int ps, int h, int m, int n) {
        f32x4 x = v[ps][h] * sc[ps];
        if (p.gain) x *= *(const f32x4*)(p.gain + n);
        const size_t off = (size_t)m * p.ldc + n;
        if (p.out_kind == K_F16)
          *(f16x4*)((f16*)p.C + off) = f16x4{(f16)x[0], (f16)x[1], (f16)x[2], (f16)x[3]};
        else if (p.out_kind == K_BF16)
          store4<bf16>((bf16*)p.C + off, x[0], x[1], x[2], x[3]);
        else
          store4<float>((float*)p.C + off, x[0], x[1], x[2], x[3]);
      });
    } break;
  }
}

// Operand staging without registers (bf16, PF = 0): each wave instruction
// copies 64 x 16 bytes from global memory straight into LDS, lane i's bytes
// landing at LDS byte address `lds` + 16 i (gfx950 LDS DMA,
// global_load_lds_dwordx4; the LDS address travels in M0). Issued as inline
// assembly: the compiler's own wait insertion would otherwise make every LDS
// read wait for all outstanding copies, i.e. for the next tile's. The
// kernel waits for its copies itself (dma_wait_all, then a barrier) before it
// reads them. Nothing else in these kernels uses M0; the compiler's waits
// for its own loads stay correct, since the counter retires operations in
// issue order and extra copies only make those waits longer.
__device__ __forceinline__ void lds_dma16(const void* g, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory");
}
__device__ __forceinline__ void dma_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector memory operations of this wave are in flight
// (they retire in issue order: every older copy has landed).
template <int N> __device__ __forceinline__ void dma_wait_but() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Eight-wave 128-wide tiles keep two workgroups per CU (LDS allows it): at
// most 128 VGPRs, i.e. four waves per SIMD.
template <int BN, int NW> constexpr int gemm_min_waves() { return NW == 8 && BN <= 128 ? 4 : 1; }
// The 64x128 tile's four 32x64 waves fit the same 128 VGPRs.
template <int BM, int BN, int NW> constexpr int gemm_min_waves3() {
  return BM == 64 && BN == 128 && NW == 4 ? 4 : gemm_min_waves<BN, NW>();
}

// SK = 0: the whole product. Split K: SK = 1 computes the K steps of split
// blockIdx.y (of gridDim.y) and stores its fp32 tile in p.sk_part; SK = 2,
// launched after it, sums the splits' tiles in split order and runs the
// epilogue (the kernel boundary makes the tiles visible; no cross-workgroup
// synchronisation). SA: LDS stages of the A operand (DMA staging). With 3
// the A copies run two K steps ahead of the MFMAs and B's one (A streams
// from HBM, the weights mostly hit L2); the 128 x 128 tile's LDS is then
// exactly half a CU's, and fused row scales wait in a register until the
// output tile's LDS is laid out.
//
// PH: the diagnostic copy (SK = 0, LDS DMA). Each workgroup stamps the 100 MHz
// real-time clock at its start, once its first operands have landed (the
// first K step's barrier), once its last products have landed, and after
// its last store; thread 0 writes the four stamps to p.clk at the
// workgroup's launch index. Workgroups past the row count write none.
template <typename T, int BM, int BN, int WM, int WN, int NW, int PF, int SK, int SA = 2,
          bool PH = false, int MINW = gemm_min_waves3<BM, BN, NW>()>
__global__ __launch_bounds__(64 * NW, MINW) void gemm_kernel(GemmParams p) {
  static_assert(!PH || (SK == 0 && PF == 0), "phase stamps: whole products, LDS DMA");
  unsigned long long clk0 = 0, clk1 = 0, clk2 = 0;
  if constexpr (PH) clk0 = clk1 = __builtin_amdgcn_s_memrealtime();
  using MF = Mfma<T>;
  constexpr int NT = 64 * NW;              // threads
  constexpr int CE = 16 / sizeof(T);       // elements per 16-byte chunk
  constexpr int BK = 8 * CE;               // 8 chunks per tile row
  constexpr int LDK = BK;                  // LDS row (elements), swizzled
  constexpr int WAVES_N = BN / WN;
  static_assert((BM / WM) * (BN / WN) == NW, "wave grid");
  constexpr int AI = BM * 8 / NT;          // A chunks per thread
  constexpr int BI = BN * 8 / NT;
  constexpr int TM = WM / 16, TN = WN / 16;

  // One LDS block: the operand tile stages during the main loop, then
  // (kShuffle) the fp32 output tile for the row-major epilogue. The row
  // scales of a fused RMSNorm of A follow the operands; with SA = 3 (no room
  // there) they follow the output tile, written once the main loop is done.
  static_assert(SA == 2 || (SA == 3 && PF == 0), "A stages");
  constexpr int kOpBytes = (SA * BM + 2 * BN) * LDK * (int)sizeof(T);
  constexpr bool kShuffle = BM * BN * 4 <= kOpBytes;
  static_assert(SA == 2 || (kShuffle && BM * BN * 4 + BM * 4 <= kOpBytes), "row scales with SA = 3");
  __shared__ __attribute__((aligned(16))) char smem[kOpBytes + (SA == 3 ? 0 : BM * 4)];
  T (*As)[BM * LDK] = (T (*)[BM * LDK])smem;
  T (*Bs)[BN * LDK] = (T (*)[BN * LDK])(smem + SA * BM * LDK * sizeof(T));
  float* rs_lds = (float*)(smem + (SA == 3 ? BM * BN * 4 : kOpBytes));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int M = dev_count(p.M_dev, p.M_cap);

  // Tile index, regrouped so that consecutive tiles of one XCD (workgroups
  // are dealt to the eight XCDs round-robin) share the same A rows.
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tiles_m = (p.M_cap + BM - 1) / BM;
  const int G = tiles_n * tiles_m;
  int bid = blockIdx.x;
  const int per = G / 8;
  if (bid < per * 8) bid = (bid & 7) * per + (bid >> 3);
  const int tm = bid / tiles_n, tn = bid % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  if (m0 >= M) return;
  // K steps [kb0, kb0 + nk) of nk_all: all of them, or split blockIdx.y's
  const int nk_all = (p.K + BK - 1) / BK;
  const int nsplit = SK == 1 ? (int)gridDim.y : 1;
  const int kper = (nk_all + nsplit - 1) / nsplit;
  const int kb0 = SK == 1 ? (int)blockIdx.y * kper : 0;

  const T* A = (const T*)p.A + (size_t)blockIdx.z * p.sA;
  const T* Bm = (const T*)p.B + (size_t)blockIdx.z * p.sB;

  // PF = 0: operands staged by LDS DMA (bf16, K a multiple of BK, rows of
  // 16-byte multiples). Instruction i of a wave stages tile rows
  // 8 (i NW + wave) .. + 7; lane l takes row + l / 8 and the global chunk that
  // the swizzle places at physical chunk l % 8. Rows past M (N) read row
  // M - 1 (N - 1): finite data whose results are never stored.
  constexpr bool DMA = PF == 0;
  static_assert(!DMA || sizeof(T) == 2, "LDS DMA staging is for 16-bit operands");
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const unsigned lds_base = (unsigned)(size_t)((__attribute__((address_space(3))) char*)smem);
  const T* adma[DMA ? AI : 1];
  const T* bdma[DMA ? BI : 1];
  if constexpr (DMA) {
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int row = (i * NW + wave_u) * 8 + lane / 8;
      const int r = min(m0 + row, M - 1);
      const int src = p.a_rows ? p.a_rows[r] : r;
      adma[i] = A + (size_t)src * p.lda + (((lane & 7) ^ ((row >> 1) & 7)) * CE);
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int row = (i * NW + wave_u) * 8 + lane / 8;
      const int r = min(n0 + row, p.N - 1);
      bdma[i] = Bm + (size_t)r * p.ldb + (((lane & 7) ^ ((row >> 1) & 7)) * CE);
    }
  }
  auto dma_tile = [&](int kt, int buf) {
    const int k0 = (kb0 + kt) * BK;
#pragma unroll
    for (int i = 0; i < AI; ++i)
      lds_dma16(adma[i] + k0, lds_base + (unsigned)((buf * BM * LDK + (i * NW + wave_u) * 8 * LDK) * 2));
#pragma unroll
    for (int i = 0; i < BI; ++i)
      lds_dma16(bdma[i] + k0, lds_base + (unsigned)((SA * BM * LDK + buf * BN * LDK +
                                                      (i * NW + wave_u) * 8 * LDK) * 2));
  };
  // the same for one operand (SA = 3)
  auto dma_a = [&](int kt, int buf) {
    const int k0 = (kb0 + kt) * BK;
#pragma unroll
    for (int i = 0; i < AI; ++i)
      lds_dma16(adma[i] + k0, lds_base + (unsigned)((buf * BM * LDK + (i * NW + wave_u) * 8 * LDK) * 2));
  };
  auto dma_b = [&](int kt, int buf) {
    const int k0 = (kb0 + kt) * BK;
#pragma unroll
    for (int i = 0; i < BI; ++i)
      lds_dma16(bdma[i] + k0, lds_base + (unsigned)((SA * BM * LDK + buf * BN * LDK +
                                                      (i * NW + wave_u) * 8 * LDK) * 2));
  };

  // Per-thread global source rows (fixed across the K loop).
  const T* arow[AI];
  bool aok[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    int c = tid + i * NT;
    int r = m0 + c / 8;
    aok[i] = r < M;
    int src = aok[i] ? (p.a_rows ? p.a_rows[r] : r) : 0;
    arow[i] = A + (size_t)src * p.lda + (c % 8) * CE;
  }
  const T* brow[BI];
  bool bok[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    int c = tid + i * NT;
    int r = n0 + c / 8;
    bok[i] = r < p.N;
    brow[i] = Bm + (size_t)(bok[i] ? r : 0) * p.ldb + (c % 8) * CE;
  }

  // Two register sets: the loads of K step k+2 are issued while step k is
  // computed from LDS and step k+1 waits in the other set, so each load has
  // two compute phases to arrive.
  i32x4 ra[PF > 0 ? PF : 1][AI], rb[PF > 0 ? PF : 1][BI];
  auto load_tile = [&](int kt, auto set) {
    constexpr int S = decltype(set)::value;
    const int k0 = (kb0 + kt) * BK;
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      int kc = ((tid + i * NT) % 8) * CE;
      bool ok = aok[i] && (k0 + kc < p.K);
      ra[S][i] = ok ? *(const i32x4*)(arow[i] + k0) : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      int kc = ((tid + i * NT) % 8) * CE;
      bool ok = bok[i] && (k0 + kc < p.K);
      rb[S][i] = ok ? *(const i32x4*)(brow[i] + k0) : i32x4{0, 0, 0, 0};
    }
  };
  auto sw = [](int row, int chunk) { return row * LDK + ((chunk ^ ((row >> 1) & 7)) * CE); };
  auto store_lds = [&](int buf, auto set) {
    constexpr int S = decltype(set)::value;
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      int c = tid + i * NT;
      *(i32x4*)&As[buf][sw(c / 8, c % 8)] = ra[S][i];
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      int c = tid + i * NT;
      *(i32x4*)&Bs[buf][sw(c / 8, c % 8)] = rb[S][i];
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int wm0 = (wave / WAVES_N) * WM;
  const int wn0 = (wave % WAVES_N) * WN;
  const int lr = lane & 15;                 // fragment row
  const int lk = (lane >> 4) * MF::VEC;     // fragment k offset
  // swizzled in-row offset of each k step (fragment rows are 16-aligned, so
  // the swizzle depends on lr only)
  constexpr int NKK = BK / MF::KSTEP;
  int koff[NKK];
#pragma unroll
  for (int x = 0; x < NKK; ++x) {
    const int e = x * MF::KSTEP + lk;
    koff[x] = ((e / CE) ^ ((lr >> 1) & 7)) * CE + e % CE;
  }

  const int nk = SK == 2 ? 0 : max(0, min(nk_all, kb0 + kper) - kb0);
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  auto compute2 = [&](int abuf, int bbuf) {
    const T* as = As[abuf];
    const T* bs = Bs[bbuf];
#pragma unroll
    for (int x = 0; x < NKK; ++x) {
      typename MF::frag fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *(const typename MF::frag*)&as[(wm0 + i * 16 + lr) * LDK + koff[x]];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[j] = *(const typename MF::frag*)&bs[(wn0 + j * 16 + lr) * LDK + koff[x]];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = MF::mma(fb[j], fa[i], acc[i][j]);
    }
  };
  auto compute = [&](int buf) { compute2(buf, buf); };
  // one K step: prefetch kt+2 into the set that held kt, compute kt, stage kt+1
  // PF == 2: two register sets (prefetch distance 2); PF == 1: one set,
  // loads of step k+1 issued while step k is computed.
  auto step = [&](int kt, auto set) {
    constexpr int S = decltype(set)::value;
    if constexpr (PF == 2) {
      using Sn = std::integral_constant<int, S ^ 1>;
      if (kt + 2 < nk) load_tile(kt + 2, set);
      compute(kt & 1);
      if (kt + 1 < nk) store_lds((kt + 1) & 1, Sn{});
    } else {
      if (kt + 1 < nk) load_tile(kt + 1, S0{});
      compute(kt & 1);
      if (kt + 1 < nk) store_lds((kt + 1) & 1, S0{});
    }
    __syncthreads();
  };
  if constexpr (SK != 2) {
    if constexpr (DMA && SA == 3) {
      // A(0), B(0), A(1)
      if (nk > 0) {
        dma_a(0, 0);
        dma_b(0, 0);
      }
      if (nk > 1) dma_a(1, 1);
    } else if constexpr (DMA) {
      if (nk > 0) dma_tile(0, 0);
    } else {
      load_tile(0, S0{});
      if constexpr (PF == 2) {
        if (nk > 1) load_tile(1, S1{});
      }
    }
  }
  // Source rows of the residual / gathered table rows, resolved before the
  // main loop so the epilogue's loads do not wait on the index loads.
  // Rows of this lane in the epilogue: NPASS rows of the row-major
  // epilogue, or TM fragment rows of the direct one.
  constexpr int RPP = NT / (BN / 8);
  constexpr int NROW = kShuffle ? BM / RPP : TM;
  int rrow[NROW];
#pragma unroll
  for (int i = 0; i < NROW; ++i) {
    const int m = kShuffle ? m0 + i * RPP + tid / (BN / 8)
                           : m0 + (wave / WAVES_N) * WM + i * 16 + (lane & 15);
    rrow[i] = 0;
    if (m < M) {
      if (p.epi == EPI_RESID_F32) rrow[i] = p.res_rows ? p.res_rows[m] : m;
      else if (p.epi == EPI_GATHER_ADD_F32) rrow[i] = p.g_rows[m];
    }
  }
  // Row scales of a fused RMSNorm of the A rows, one thread per tile row:
  // their loads wait together with the first tile's. With SA = 3 the value
  // waits in a register until the operand stages are free.
  float rs_reg = 1.f;
  if (p.rs.ss && tid < BM) {
    const int m = m0 + tid;
    float sc = 1.f;
    if (m < M) {
      // slots in batches of eight loads in flight (indexes clamped in bounds)
      const float* ss = p.rs.ss + (p.a_rows ? p.a_rows[m] : m);
      float t = 0.f;
      for (int q0 = 0; q0 < p.rs.np; q0 += 8) {
        float x[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) x[q] = ss[(size_t)min(q0 + q, p.rs.np - 1) * p.rs.ld];
#pragma unroll
        for (int q = 0; q < 8; ++q) t += q0 + q < p.rs.np ? x[q] : 0.f;
      }
      sc = 1.f / sqrtf(t / (float)p.rs.n + p.rs.eps);
    }
    if constexpr (SA == 2) rs_lds[tid] = sc;
    else rs_reg = sc;
  }
  if constexpr (DMA && SA == 3) {
    // at step kt's top only A(kt + 1) may still be in flight (copies retire
    // in issue order); after the barrier B(kt + 1) and A(kt + 2) go into the
    // stages step kt - 1 used
    int ac = 0, bc = 0;
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) dma_wait_but<AI>();
      else dma_wait_all();
      __syncthreads();
      if constexpr (PH) {
        if (kt == 0) clk1 = __builtin_amdgcn_s_memrealtime();
      }
      if (kt + 1 < nk) dma_b(kt + 1, bc ^ 1);
      if (kt + 2 < nk) dma_a(kt + 2, ac == 0 ? 2 : ac - 1);
      compute2(ac, bc);
      ac = ac == 2 ? 0 : ac + 1;
      bc ^= 1;
    }
    __syncthreads();  // operand LDS before the epilogue reuses it
    // past the output tile; the epilogue's barrier publishes them
    if (p.rs.ss && tid < BM) rs_lds[tid] = rs_reg;
  } else if constexpr (DMA) {
    // one barrier per K step: it publishes step kt's tile (every wave has
    // waited for its own copies) and frees the other buffer, into which the
    // copies of step kt + 1 go while step kt is computed
    for (int kt = 0; kt < nk; ++kt) {
      dma_wait_all();
      __syncthreads();
      if constexpr (PH) {
        if (kt == 0) clk1 = __builtin_amdgcn_s_memrealtime();
      }
      if (kt + 1 < nk) dma_tile(kt + 1, (kt + 1) & 1);
      compute(kt & 1);
    }
    __syncthreads();  // operand LDS (and rs_lds) before the epilogue reuses it
  } else {
    if constexpr (SK != 2) store_lds(0, S0{});
    __syncthreads();
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      step(kt, S0{});
      step(kt + 1, S1{});
    }
    if (kt < nk) step(kt, S0{});
  }

  if constexpr (SK != 0) {
    // split tiles: [tile][split][thread][TM*TN f32x4], each thread's
    // accumulators contiguous
    const size_t tile_id = (size_t)blockIdx.z * G + bid;
    const int S = SK == 1 ? nsplit : p.sk_splits;
    float* part = p.sk_part + tile_id * S * (size_t)(BM * BN);
    if constexpr (SK == 1) {
      f32x4* mine = (f32x4*)(part + (size_t)blockIdx.y * (BM * BN)) + tid * (TM * TN);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mine[i * TN + j] = acc[i][j];
      return;
    } else {
      for (int sp = 0; sp < S; ++sp) {
        const f32x4* src = (const f32x4*)(part + (size_t)sp * (BM * BN)) + tid * (TM * TN);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] += src[i * TN + j];
      }
    }
  }

  if constexpr (PH) {
    // a read of the last products' results waits for them to land
    float d;
    asm volatile("v_mov_b32 %0, %1" : "=v"(d) : "v"(acc[TM - 1][TN - 1][3]));
    asm volatile("" ::"v"(d));
    clk2 = __builtin_amdgcn_s_memrealtime();
  }
  if constexpr (kShuffle) {
    if (p.nt)
      epilogue_rowmajor<T, BM, BN, WM, WN, NW, true>(p, acc, (float*)smem, rs_lds, rrow, m0, n0,
                                                     M, wm0, wn0, lane, tid);
    else
      epilogue_rowmajor<T, BM, BN, WM, WN, NW, false>(p, acc, (float*)smem, rs_lds, rrow, m0, n0,
                                                      M, wm0, wn0, lane, tid);
    if constexpr (PH) {
      const unsigned long long clk3 = __builtin_amdgcn_s_memrealtime();
      if (tid == 0) {
        unsigned long long* o = p.clk + ((size_t)blockIdx.z * gridDim.x + blockIdx.x) * 4;
        o[0] = clk0;
        o[1] = clk1;
        o[2] = clk2;
        o[3] = clk3;
      }
    }
    return;
  }
  // Direct epilogue (tiles whose fp32 output does not fit the LDS block):
  // lane holds C[m][n .. n+3] of each 16x16 block.
  // Row scale of a fused RMSNorm of the A rows (1 without one).
  float rsc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) rsc[i] = p.rs.ss ? rs_lds[wm0 + i * 16 + lr] : 1.f;

  if (p.epi == EPI_ROWNORM) {
    // y = rsc * acc; with a gain, RMSNorm over the row's N columns, which
    // this tile spans: partial sums per wave, then across the WAVES_N waves
    // of a row through LDS (free after the main loop's last barrier).
    float scale[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) scale[i] = rsc[i];
    if (p.gain) {
      float* red = (float*)&As[0][0];
      float ssr[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        ssr[i] = 0.f;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = n0 + wn0 + j * 16 + (lane >> 4) * 4;
          if (n < p.N) {
            const f32x4 v = acc[i][j];
            ssr[i] += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
          }
        }
        ssr[i] = group_sum4(ssr[i]) * rsc[i] * rsc[i];
      }
      if (lane < 16) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
          red[(wm0 + i * 16 + lr) * WAVES_N + wave % WAVES_N] = ssr[i];
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES_N; ++w) t += red[(wm0 + i * 16 + lr) * WAVES_N + w];
        scale[i] = rsc[i] / sqrtf(t / (float)p.N + p.eps);
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wm0 + i * 16 + lr;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn0 + j * 16 + (lane >> 4) * 4;
        if (n >= p.N) continue;
        f32x4 v = acc[i][j] * scale[i];
        if (p.gain) v *= *(const f32x4*)(p.gain + n);
        const size_t off = (size_t)m * p.ldc + n;
        if (p.out_kind == K_F16)
          *(f16x4*)((f16*)p.C + off) = f16x4{(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
        else if (p.out_kind == K_BF16)
          store4<bf16>((bf16*)p.C + off, v[0], v[1], v[2], v[3]);
        else
          store4<float>((float*)p.C + off, v[0], v[1], v[2], v[3]);
      }
    }
    return;
  }

  // The other epilogues: one unrolled pass per kind, with all loads of a
  // pass (residual rows, table rows) issued before their first use.
  auto outs = [&](auto&& f) {  // f(i, j, m, n) over this lane's valid outputs
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wm0 + i * 16 + lr;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn0 + j * 16 + (lane >> 4) * 4;
        if (m < M && n < p.N) f(i, j, m, n);
      }
    }
  };
  auto coff = [&](int m, int n) {
    return (size_t)blockIdx.z * p.sC + (size_t)m * p.ldc + n;
  };
  switch (p.epi) {
    case EPI_STORE:
      outs([&](int i, int j, int m, int n) {
        const f32x4 v = acc[i][j] * (rsc[i] * p.alpha);
        store4<T>((T*)p.C + coff(m, n), v[0], v[1], v[2], v[3]);
      });
      break;
    case EPI_STORE_F32:
      outs([&](int i, int j, int m, int n) {
        const f32x4 v = add_time_enc(acc[i][j] * (rsc[i] * p.alpha), p, m, n);
        store4<float>((float*)p.C + coff(m, n), v[0], v[1], v[2], v[3]);
      });
      break;
    case EPI_GELU:
      outs([&](int i, int j, int m, int n) {
        const f32x4 v = acc[i][j] * rsc[i];
        store4<T>((T*)p.C + coff(m, n), gelu_t<T>(v[0]), gelu_t<T>(v[1]), gelu_t<T>(v[2]),
                  gelu_t<T>(v[3]));
      });
      break;
    case EPI_RESID_F32: {
      // one 16-row block at a time: its residual loads all in flight, then
      // its results (registers for TN loads, not TM x TN)
      float ssp[TM];  // partial sums of squares of the results
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        ssp[i] = 0.f;
        const int m = m0 + wm0 + i * 16 + lr;
        f32x4 r[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = n0 + wn0 + j * 16 + (lane >> 4) * 4;
          r[j] = f32x4{};
          if (m < M && n < p.N) r[j] = *(const f32x4*)(p.res.row(rrow[i]) + n);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = n0 + wn0 + j * 16 + (lane >> 4) * 4;
          if (m >= M || n >= p.N) continue;
          const f32x4 v = acc[i][j] * rsc[i] + r[j];
          store4<float>((float*)p.C + coff(m, n), v[0], v[1], v[2], v[3]);
          if (p.cast_out)
            store4<T>((T*)p.cast_out + (size_t)m * p.ld_cast + n, v[0], v[1], v[2], v[3]);
          ssp[i] += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
        }
      }
      if (p.ss_out) {
        // one slot per (row, strip of WN columns); strips start below N
        const int slots = (p.N + WN - 1) / WN;
        const int slot = (n0 + wn0) / WN;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const float t = group_sum4(ssp[i]);
          const int m = m0 + wm0 + i * 16 + lr;
          if (lane < 16 && m < M && slot < slots) p.ss_out[(size_t)slot * p.ss_ld + m] = t;
        }
      }
    } break;
    case EPI_GATHER_ADD_F32: {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = m0 + wm0 + i * 16 + lr;
        f32x4 r[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = n0 + wn0 + j * 16 + (lane >> 4) * 4;
          r[j] = f32x4{};
          if (m < M && n < p.N) r[j] = load4<T>((const T*)p.table + (size_t)rrow[i] * p.ld_table + n);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = n0 + wn0 + j * 16 + (lane >> 4) * 4;
          if (m >= M || n >= p.N) continue;
          const f32x4 v = acc[i][j] * rsc[i] + r[j];
          store4<float>((float*)p.C + coff(m, n), v[0], v[1], v[2], v[3]);
        }
      }
    } break;
    case EPI_GELU_BWD:
      outs([&](int i, int j, int m, int n) {
        const f32x4 a = load4<T>((const T*)p.table + (size_t)m * p.ld_table + n);
        const f32x4 v = acc[i][j] * rsc[i];
        f32x4 dg, g;
        gelu_bwd4<T>(v, a, dg, g);
        store4<T>((T*)p.C + coff(m, n), dg[0], dg[1], dg[2], dg[3]);
        store4<T>((T*)p.cast_out + (size_t)m * p.ld_cast + n, g[0], g[1], g[2], g[3]);
      });
      break;
  }
}

// Splits of K for a launch of `tiles` workgroups. Only launches that leave
// most CUs idle with a long chain of K steps per workgroup gain from the
// second pass (measured: products with K <= 512, or with 400 or more tiles,
// got slower split): then enough splits to approach one workgroup per CU,
// at least 4 K steps per split, within the scratch capacity; 1 without
// scratch.
static int k_splits(const GemmParams& p, long long tiles, int BM, int BN, int BK) {
  if (!p.sk_part || tiles <= 0 || tiles >= 128) return 1;
  const int nk = (p.K + BK - 1) / BK;
  if (nk < 16) return 1;
  // very long contractions (weight gradients over the rows) may split
  // further, down to 4 K steps per split, until 256 workgroups
  const long long cap = p.K >= 4096 ? 64 : 8;
  long long sp = std::min<long long>({cap, 256 / tiles, nk / 4});
  while (sp > 1 && tiles * sp * BM * BN > p.sk_part_cap) --sp;
  return (int)std::max<long long>(sp, 1);
}

template <typename T, int BM, int BN, int WM, int WN, int NW, int PF = 1, int SA = 2>
static hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  const int tiles = ((p.M_cap + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  if (tiles == 0 || p.batch == 0) return hipSuccess;
  constexpr int BK = 128 / (int)sizeof(T);
  const int splits = k_splits(p, (long long)tiles * p.batch, BM, BN, BK);
  timing_begin(p.name, s);
  if (splits == 1) {
    hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, NW, PF, 0, SA>), dim3(tiles, 1, p.batch),
                       dim3(64 * NW), 0, s, p);
  } else {
    GemmParams q = p;
    q.sk_splits = splits;
    hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, NW, PF, 1>), dim3(tiles, splits, p.batch),
                       dim3(64 * NW), 0, s, q);
    hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, NW, PF, 2>), dim3(tiles, 1, p.batch),
                       dim3(64 * NW), 0, s, q);
  }
  timing_end(s);
  return hipGetLastError();
}

// Phase diagnostics (gemm_phases_enable): the stamp buffer of this thread's
// device and the records taken so far.
struct GemmPhaseState {
  unsigned long long* buf = nullptr;
  int cap = 0;
  std::vector<double> rec;
};
static thread_local GemmPhaseState t_gph;

hipError_t gemm_phases_enable(int max_wg) {
  if (t_gph.buf) {
    hipError_t e = hipFree(t_gph.buf);
    t_gph.buf = nullptr;
    t_gph.cap = 0;
    if (e != hipSuccess) return e;
  }
  t_gph.rec.clear();
  if (max_wg <= 0) return hipSuccess;
  hipError_t e = hipMalloc(&t_gph.buf, (size_t)max_wg * 4 * sizeof(unsigned long long));
  if (e != hipSuccess) {
    t_gph.buf = nullptr;
    return e;
  }
  t_gph.cap = max_wg;
  return hipSuccess;
}

int gemm_phases_read(double* out, int cap) {
  const int n = (int)(t_gph.rec.size() / kGemmPhaseFields);
  if (out)
    for (int i = 0; i < std::min(n, cap) * kGemmPhaseFields; ++i) out[i] = t_gph.rec[i];
  return n;
}

// One instrumented launch of the 128 x 128 LDS-staged tile: stamps, then the
// host reduction (clock ticks are 10 ns). Record: workgroups with rows, M
// bound, N, K, summed wait for the first operands, K loop and epilogue (us),
// launch span and longest workgroup (us).
static hipError_t launch_gemm_phases(const GemmParams& p, int tiles, hipStream_t s) {
  const int nwg = tiles * p.batch;
  GemmParams q = p;
  q.clk = t_gph.buf;
  hipError_t e = hipMemsetAsync(q.clk, 0, (size_t)nwg * 4 * sizeof(unsigned long long), s);
  if (e != hipSuccess) return e;
  timing_begin(p.name, s);
  hipLaunchKernelGGL((gemm_kernel<bf16, 128, 128, 32, 64, 8, 0, 0, 3, true>), dim3(tiles, 1, p.batch),
                     dim3(512), 0, s, q);
  timing_end(s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  std::vector<unsigned long long> h((size_t)nwg * 4);
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
  if ((e = hipMemcpy(h.data(), q.clk, h.size() * sizeof(h[0]), hipMemcpyDeviceToHost)) != hipSuccess)
    return e;
  double wg = 0, first = 0, loop = 0, epi = 0, longest = 0;
  unsigned long long t0 = ~0ull, t1 = 0;
  for (int i = 0; i < nwg; ++i) {
    const unsigned long long* c = &h[(size_t)i * 4];
    if (c[0] == 0) continue;  // a workgroup past the row count
    wg += 1;
    first += (double)(c[1] - c[0]);
    loop += (double)(c[2] - c[1]);
    epi += (double)(c[3] - c[2]);
    longest = std::max(longest, (double)(c[3] - c[0]));
    t0 = std::min(t0, c[0]);
    t1 = std::max(t1, c[3]);
  }
  const double us = 0.01;
  const double rec[kGemmPhaseFields] = {wg, (double)p.M_cap, (double)p.N, (double)p.K,
                                        first * us, loop * us, epi * us,
                                        wg > 0 ? (double)(t1 - t0) * us : 0.0, longest * us};
  t_gph.rec.insert(t_gph.rec.end(), rec, rec + kGemmPhaseFields);
  return hipSuccess;
}

static long long ntiles(const GemmParams& p, int bm, int bn) {
  return (long long)((p.M_cap + bm - 1) / bm) * ((p.N + bn - 1) / bn) * p.batch;
}

// Tile choice: 128x128 with eight waves (32x64 each) when that gives the
// GPU (256 CUs) enough workgroups; 64x64 tiles for the small products
// (readout layer, last pyramid layers) that would otherwise occupy a few CUs.
// A row-normalising epilogue needs one tile across all N columns.
enum TileCfg { T64x64, T128x64, T64x128, T128x128, T128x256, F128x64, F128x128, T_NONE };

static TileCfg select_tile(const GemmParams& p, bool is_bf16) {
  if (p.epi == EPI_ROWNORM && p.gain) {
    if (!is_bf16) return p.N <= 64 ? F128x64 : p.N <= 128 ? F128x128 : T_NONE;
    if (p.N <= 64) return ntiles(p, 128, 64) < 256 ? T64x64 : T128x64;
    // 64-row tiles spread the rows over more CUs where that takes no more
    // rounds of the GPU: 128 x 128 tiles run two per CU (512 at once), the
    // 64 x 128 ones three (LDS: 768 at once). Each round costs about the
    // same (the K loop's latency), so 400 large tiles (one round) beat 800
    // small ones (two).
    if (p.N <= 128) {
      const long long r128 = (ntiles(p, 128, 128) + 511) / 512;
      const long long r64 = (ntiles(p, 64, 128) + 767) / 768;
      return r64 <= r128 ? T64x128 : T128x128;
    }
    if (p.N <= 256) return T128x256;
    return T_NONE;
  }
  if (is_bf16) {
    // long contractions over few output tiles (weight gradients, K = rows):
    // the large tile, with K split across the GPU; below 16 large tiles the
    // small one, whose split sums stay short for the reduce pass (one
    // workgroup per output tile)
    if (p.sk_part && p.K >= 4096 && p.batch == 1 && ntiles(p, 128, 128) >= 16 &&
        ntiles(p, 128, 128) < 128)
      return T128x128;
    if (ntiles(p, 128, 128) < 256) return T64x64;
    if (p.N <= 64) return T128x64;
    return T128x128;
  }
  return p.N <= 64 ? F128x64 : F128x128;
}

// Tiles with the row-major epilogue write one slot per tile column; the
// 128x256 tile (direct epilogue) one per 64-column wave strip.
int gemm_ss_slots(const GemmParams& p, bool is_bf16) {
  int w = 128;
  switch (select_tile(p, is_bf16)) {
    case T64x64: case T128x64: case F128x64: w = 64; break;
    case T128x256: w = 64; break;
    default: break;
  }
  return (p.N + w - 1) / w;
}

// bf16 operands whose K is a whole number of 64-wide steps and whose rows
// are 16-byte multiples are staged by LDS DMA (PF = 0); the others through
// registers.
static bool dma_ok(const GemmParams& p) { return p.K % 64 == 0 && p.lda % 8 == 0 && p.ldb % 8 == 0; }

hipError_t gemm(const GemmParams& p, bool is_bf16, hipStream_t s) {
  if (p.M_cap <= 0 || p.N <= 0) return hipSuccess;
  const bool dma = is_bf16 && dma_ok(p);
  switch (select_tile(p, is_bf16)) {
    case T64x64:
      return dma ? launch_gemm<bf16, 64, 64, 32, 32, 4, 0>(p, s) : launch_gemm<bf16, 64, 64, 32, 32, 4, 2>(p, s);
    case T128x64:
      return dma ? launch_gemm<bf16, 128, 64, 64, 32, 4, 0>(p, s) : launch_gemm<bf16, 128, 64, 64, 32, 4>(p, s);
    case T64x128:
      return dma ? launch_gemm<bf16, 64, 128, 32, 64, 4, 0>(p, s) : launch_gemm<bf16, 64, 128, 32, 64, 4>(p, s);
    case T128x128:
      // three A stages (A copies two K steps ahead): measured on the c3
      // forward, 1.7 % per step over two stages (W1 and W_o 3 %, W2 1 %)
      if (dma && t_gph.buf && p.batch >= 1 && ntiles(p, 128, 128) <= t_gph.cap &&
          k_splits(p, ntiles(p, 128, 128), 128, 128, 64) == 1)
        return launch_gemm_phases(p, (int)(ntiles(p, 128, 128) / std::max(p.batch, 1)), s);
      return dma ? launch_gemm<bf16, 128, 128, 32, 64, 8, 0, 3>(p, s)
                 : launch_gemm<bf16, 128, 128, 32, 64, 8>(p, s);
    case T128x256:
      return dma ? launch_gemm<bf16, 128, 256, 64, 64, 8, 0>(p, s) : launch_gemm<bf16, 128, 256, 64, 64, 8>(p, s);
    case F128x64: return launch_gemm<float, 128, 64, 64, 32, 4>(p, s);
    case F128x128: return launch_gemm<float, 128, 128, 64, 64, 4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace llatte
