// Backward of the latent attention core ([LLaTTE] Appendix A.3, absorbed
// MLA: attention on the latent C, which is both key and value), bf16
// operands on the matrix cores, fp32 accumulation.
//
// Per user and head, over the keys j a query row sees (the forward's masks):
//   p_j = exp(scale * q . C_j - lse),  D = d_out . out,
//   ds_j = p_j (d_out . C_j - D),
//   d_q = scale * sum_j ds_j C_j,
//   d_C_j = sum over rows and heads of (p_j d_out + scale * ds_j q).
// The softmax is recomputed from the forward's log-sum-exp, so neither P nor
// dS is stored. Two kernels:
//   d_q  one block per (64 query rows, user, head), looping over 64-key
//        tiles. It also computes D and writes d_out as two bf16 parts (see
//        split_bf16) to the workspace, for the second kernel.
//   d_C  one block per (128 keys, user, head group), looping over the heads
//        of its group and the 32-row query blocks that see its keys.
// Both keep the operand that stays fixed in registers (the wave's query
// rows; the wave's keys) and stage only row-major tiles of the other side
// through LDS, double-buffered with one barrier per step. Every product
// whose contraction runs over the staged tile's rows (dS C for d_q; P^T
// d_out and dS^T q for d_C) reads its transposed operand with the gfx950
// transpose load, and takes P / dS straight from the score accumulators:
// both operands use the same permutation of the contraction index (lane
// group g holds k = 4g..4g+3 and 16+4g..16+4g+3 of each 32-wide step),
// which is the accumulator layout of a 16x16 block pair.
//
// Precision: the d_C sums are dominated, for the first keys of a long
// history, by terms about sqrt(K) times the typical size, so bf16 rounding
// of P, d_out or dS alone moves them by a few percent of the gradient's
// RMS. Each of the three enters its products as a high bf16 part plus the
// bf16 rounding remainder; only the negligible remainder x remainder terms
// are dropped. dP = d_out . C takes both parts of d_out as well, so that
// dP - D does not cancel into the rounding of d_out.
//
// LDS: tile rows are R + 16 bf16 (R/2 + 8 four-byte banks, 8 modulo 64), so
// that the 16-byte operand reads (16 rows x 4 chunks), the transpose reads
// (8 rows x 4 eight-byte chunks per 32 lanes) and the 16-byte staging writes
// each touch every bank of a cycle at most once.
#include <type_traits>

#include "backward.hpp"

namespace llatte {

namespace {

constexpr int kQRows = 64;   // d_q: query rows per block (16 per wave)
constexpr int kKeys = 64;    // d_q: keys per staged tile
constexpr int kCKeys = 128;  // d_C: keys per block (32 per wave)
constexpr int kCRows = 32;   // d_C: query rows per staged tile
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 bwd_hx4;
typedef __attribute__((address_space(3))) bwd_hx4 bwd_lds_hx4;
typedef __attribute__((address_space(3))) f16 bwd_lds_f16;

__device__ __forceinline__ f32x4 mfma_bf(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposed 4x16 read of 16-bit data: within each 16-lane group, lane i
// receives column i of the 4 x 16 block whose rows the group's lanes address
// (four lanes per row, 8 bytes each). p points into LDS.
__device__ __forceinline__ bf16x4 lds_tr(const bf16* p) {
  auto q = (bwd_lds_hx4*)((bwd_lds_f16*)(f16*)p);
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(q));
}

// 2^x with the hardware instruction alone (no range scaling): arguments
// here are x = s - lse <= ~0, and probabilities below 2^-126 flush to 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// A user's query rows in the forward's order: history rows t < n (key
// position K - n + t), then the candidates (position K - 1).
struct UserRows {
  int K, n, total, kv0, hq0;
  __device__ int global_row(int t, int u, int nc, int n_cand) const {
    return t < n ? nc + hq0 + t : u * n_cand + (t - n);
  }
  __device__ int pos(int t) const { return t < n ? K - n + t : K - 1; }
};

__device__ __forceinline__ UserRows user_rows(const AttnBwdParams& p, int u) {
  UserRows r;
  r.kv0 = p.kv_off[u];
  r.K = p.kv_off[u + 1] - r.kv0;
  r.hq0 = p.hq_off[u];
  r.n = p.hq_off[u + 1] - r.hq0;
  r.total = r.n + p.n_cand;
  return r;
}

// x as two bf16 parts: hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void split_bf16(f32x4 a, f32x4 b, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float v = i < 4 ? a[i] : b[i - 4];
    hi[i] = to_bf16(v);
    lo[i] = to_bf16(v - from_bf16(hi[i]));
  }
}

}  // namespace

// d_q for query rows [t0, t0 + 64) of one user and head (t0 from the
// heaviest block down: blockIdx.y = 0 is the user's last row block).
// Lane (lr, lg) of wave w owns query row t0 + 16w + lr and the r-chunks
// 32 ks + 8 lg of its q and d_out; S and dP of a 64-key tile come out as
// 16x16 blocks with keys on the accumulator's row index, which is the
// layout the dS operand of the d_q product needs.
template <int R>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(AttnBwdParams p) {
  constexpr int NKS = R / 32, NRB = R / 16, LD = R + 16;
  constexpr int NLD = kKeys * R / 8 / 256;   // 16-byte staging loads per thread
  __shared__ __attribute__((aligned(16))) bf16 Cs[2][kKeys * LD];
  const int u = blockIdx.x / p.h, hh = blockIdx.x % p.h, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const UserRows ur = user_rows(p, u);
  const int t0 = (gridDim.y - 1 - blockIdx.y) * kQRows;
  // with two head groups the d_C kernel adds into d_C: the head-0 blocks
  // clear the user's keys [t0, t0 + 64) first (the grid covers max_len rows)
  if (p.dc_accumulate && hh == 0) {
    for (int e = tid; e < kQRows * R / 4; e += 256) {
      const int key = t0 + e / (R / 4);
      if (key < ur.K) *(f32x4*)(p.dc + (size_t)(ur.kv0 + key) * R + (e % (R / 4)) * 4) = f32x4{};
    }
  }
  if (t0 >= ur.total) return;
  const int nc = p.B * p.n_cand, h = p.h;

  // the last row of the block has the largest key position
  const int last = min(ur.total, t0 + kQRows) - 1;
  const int ntiles = ur.pos(last) / kKeys + 1;
  const bf16* cg = (const bf16*)p.c + (size_t)ur.kv0 * R;
  bf16x8 stage[NLD];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int e = tid + 256 * i, key = e / (R / 8), c = (e % (R / 8)) * 8;
      const int k = kt * kKeys + key;
      stage[i] = k < ur.K ? *(const bf16x8*)(cg + (size_t)k * R + c) : bf16x8{};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int e = tid + 256 * i, key = e / (R / 8), c = (e % (R / 8)) * 8;
      *(bf16x8*)&Cs[buf][key * LD + c] = stage[i];
    }
  };
  // the first key tile's loads go out before the row prologue's, so the two
  // latencies overlap
  gload(0);

  const int t0w = t0 + wave * 16;  // the wave's first row
  const int t = t0w + lr;
  const bool valid = t < ur.total;
  const size_t rowoff = valid ? ((size_t)ur.global_row(t, u, nc, p.n_cand) * h + hh) * R : 0;
  bf16x8 qf[NKS], gh[NKS], gl[NKS];
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const size_t o = rowoff + ks * 32 + lg * 8;
    f32x4 g0{}, g1{}, o0{}, o1{};
    qf[ks] = bf16x8{};
    if (valid) {
      qf[ks] = *(const bf16x8*)((const bf16*)p.q + o);
      g0 = *(const f32x4*)(p.dout + o);
      g1 = *(const f32x4*)(p.dout + o + 4);
      o0 = *(const f32x4*)(p.out + o);
      o1 = *(const f32x4*)(p.out + o + 4);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) dpart = fmaf(g0[i], o0[i], fmaf(g1[i], o1[i], dpart));
    split_bf16(g0, g1, gh[ks], gl[ks]);
    if (valid) {
      *(bf16x8*)(p.ws_ghi + o) = gh[ks];
      *(bf16x8*)(p.ws_glo + o) = gl[ks];
    }
  }
  const float D = group_sum4(dpart);
  float lse2 = 0.f;
  int pos = -1;
  if (valid) {
    const size_t ri = rowoff / R;
    lse2 = p.lse[ri] * kLog2e;
    pos = ur.pos(t);
    if (lg == 0) p.ws_d[ri] = D;
  }
  const float sl2 = p.scale * kLog2e;

  // transpose-read offsets: rows 4 lg + (lr >> 2) (+16), column block rb
  const int trow = 4 * lg + (lr >> 2), tcol = (lr & 3) * 4;

  f32x4 dq[NRB];
#pragma unroll
  for (int b = 0; b < NRB; ++b) dq[b] = f32x4{};

  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ntiles) gload(kt + 1);
    const bf16* cs = Cs[buf];
    // S and dP: lane holds keys nb*16 + 4 lg + e of its row
    f32x4 s[4], dp[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) s[nb] = dp[nb] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const bf16x8 a = *(const bf16x8*)&cs[(nb * 16 + lr) * LD + ks * 32 + lg * 8];
        s[nb] = mfma_bf(a, qf[ks], s[nb]);
        dp[nb] = mfma_bf(a, gh[ks], dp[nb]);
        dp[nb] = mfma_bf(a, gl[ks], dp[nb]);
      }
    // dS = P (dP - D) on allowed keys, as the B operand of step kk: keys
    // kk*32 + 4 lg + e (block 2kk) and kk*32 + 16 + 4 lg + e (block 2kk+1)
    bf16x8 dsh[2], dsl[2];
    const int k0 = kt * kKeys;
    auto make_ds = [&](auto unmasked) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = k0 + nb * 16 + lg * 4 + e;
          const bool ok = decltype(unmasked)::value || key <= pos;
          const float pr = ok ? exp2_hw(s[nb][e] * sl2 - lse2) : 0.f;
          const float ds = pr * (dp[nb][e] - D);
          const bf16 hi = to_bf16(ds);
          dsh[nb >> 1][(nb & 1) * 4 + e] = hi;
          dsl[nb >> 1][(nb & 1) * 4 + e] = to_bf16(ds - from_bf16(hi));
        }
    };
    // the wave's 16 rows all valid and all seeing the whole tile (positions
    // grow with the row): no mask (a wave-uniform branch)
    if (t0w + 16 <= ur.total && ur.pos(t0w) >= k0 + kKeys - 1) make_ds(std::true_type{});
    else make_ds(std::false_type{});
    // d_q += dS C: A = C^T rows rb*16.. (transpose loads), keys in the same order
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const bf16x8 a = cat8(lds_tr(cs + (kk * 32 + trow) * LD + rb * 16 + tcol),
                              lds_tr(cs + (kk * 32 + 16 + trow) * LD + rb * 16 + tcol));
        dq[rb] = mfma_bf(a, dsh[kk], dq[rb]);
        dq[rb] = mfma_bf(a, dsl[kk], dq[rb]);
      }
    if (kt + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }
  if (valid) {
    if (p.dq_bf16) {
      bf16* dst = p.dq_bf16 + rowoff;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const f32x4 v = dq[rb] * p.scale;
        *(bf16x4*)(dst + rb * 16 + lg * 4) = bf16x4{to_bf16(v[0]), to_bf16(v[1]), to_bf16(v[2]), to_bf16(v[3])};
      }
    } else {
      float* dst = p.dq + rowoff;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) *(f32x4*)(dst + rb * 16 + lg * 4) = dq[rb] * p.scale;
    }
  }
}

// d_C for keys [k0, k0 + 128) of one user, over the heads of one group and
// every 32-row query block that sees them. Wave w owns keys k0 + 32w + 16kb
// + lr (kb = 0, 1) and keeps their C rows in registers as the B operand of
// S^T and dP^T; the staged tiles are the block's q, d_out high and d_out low
// rows (row-major), read directly for S^T / dP^T and transposed for the d_C
// products. blockIdx.y = 0 holds the first keys, which the most rows see.
template <int R>
__global__ __launch_bounds__(256, 2) void attn_bwd_dc_kernel(AttnBwdParams p) {
  constexpr int NKS = R / 32, NRB = R / 16, LD = R + 16;
  constexpr int TILE = kCRows * LD;
  constexpr int NLD = 3 * kCRows * R / 8 / 256;
  __shared__ __attribute__((aligned(16))) bf16 Ts[2][3 * TILE];
  __shared__ __attribute__((aligned(16))) float s_lse2[2][kCRows], s_D[2][kCRows];
  const int ngroups = p.dc_accumulate ? 2 : 1;
  const int u = blockIdx.x / ngroups, grp = blockIdx.x % ngroups, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const UserRows ur = user_rows(p, u);
  const int k0 = blockIdx.y * kCKeys;
  if (k0 >= ur.K) return;
  const int nc = p.B * p.n_cand, h = p.h;
  const int hpg = h / ngroups, h0 = grp * hpg;

  const int kw = k0 + wave * 32;
  bf16x8 cf[2][NKS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kw + kb * 16 + lr;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      cf[kb][ks] = key < ur.K
                       ? *(const bf16x8*)((const bf16*)p.c + (size_t)(ur.kv0 + key) * R + ks * 32 + lg * 8)
                       : bf16x8{};
  }
  f32x4 dc[2][NRB];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) dc[kb][rb] = f32x4{};

  // history rows at key positions below k0 see none of these keys
  const int t_first = max(0, k0 - (ur.K - ur.n)) / kCRows * kCRows;
  const int nrb = ur.total > t_first ? (ur.total - t_first + kCRows - 1) / kCRows : 0;
  const int nit = hpg * nrb;

  bf16x8 stage[NLD];
  float meta = 0.f;
  // staging piece i of a thread: tile i / (pieces per tile) (q, d_out high,
  // d_out low), row rr, column c; its offset from the block's first row is
  // fixed across the loop
  constexpr int PPT = kCRows * R / 8;  // 16-byte pieces per tile (a multiple of 256)
  int soff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int w = (tid + 256 * i) % PPT;
    soff[i] = (w / (R / 8)) * h * R + (w % (R / 8)) * 8;
  }
  auto tile_src = [&](int i) -> const bf16* {
    const int tile = 256 * i / PPT;
    return tile == 0 ? (const bf16*)p.q : tile == 1 ? p.ws_ghi : p.ws_glo;
  };
  auto gload = [&](int it) {
    const int hh = h0 + it / nrb, t0 = t_first + (it % nrb) * kCRows;
    if (t0 + kCRows <= ur.n) {
      // 32 history rows: consecutive global rows from nc + hq0 + t0
      const size_t base = ((size_t)(nc + ur.hq0 + t0) * h + hh) * R;
#pragma unroll
      for (int i = 0; i < NLD; ++i) stage[i] = *(const bf16x8*)(tile_src(i) + base + soff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int w = (tid + 256 * i) % PPT;
        const int rr = w / (R / 8), c = (w % (R / 8)) * 8, t = t0 + rr;
        bf16x8 v{};
        if (t < ur.total) {
          const size_t o = ((size_t)ur.global_row(t, u, nc, p.n_cand) * h + hh) * R + c;
          v = *(const bf16x8*)(tile_src(i) + o);
        }
        stage[i] = v;
      }
    }
    if (tid < 2 * kCRows) {
      const int rr = tid % kCRows, t = t0 + rr;
      meta = 0.f;
      if (t < ur.total) {
        const size_t ri = (size_t)ur.global_row(t, u, nc, p.n_cand) * h + hh;
        meta = tid < kCRows ? p.lse[ri] * kLog2e : p.ws_d[ri];
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int e = tid + 256 * i, tile = e / (kCRows * R / 8), w = e % (kCRows * R / 8);
      const int rr = w / (R / 8), c = (w % (R / 8)) * 8;
      *(bf16x8*)&Ts[buf][tile * TILE + rr * LD + c] = stage[i];
    }
    if (tid < kCRows) s_lse2[buf][tid] = meta;
    else if (tid < 2 * kCRows) s_D[buf][tid - kCRows] = meta;
  };
  const float sl2 = p.scale * kLog2e;
  const int trow = 4 * lg + (lr >> 2), tcol = (lr & 3) * 4;

  if (nit > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int it = 0; it < nit; ++it) {
    const int buf = it & 1;
    const int t0 = t_first + (it % nrb) * kCRows;
    if (it + 1 < nit) gload(it + 1);
    const bf16* qs = Ts[buf];
    const bf16* ghs = Ts[buf] + TILE;
    const bf16* gls = Ts[buf] + 2 * TILE;
    // S^T and dP^T: lane holds key kb*16 + lr, rows nb*16 + 4 lg + e
    f32x4 s[2][2], dp[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) s[kb][nb] = dp[kb][nb] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int o = (nb * 16 + lr) * LD + ks * 32 + lg * 8;
        const bf16x8 aq = *(const bf16x8*)&qs[o];
        const bf16x8 ah = *(const bf16x8*)&ghs[o];
        const bf16x8 al = *(const bf16x8*)&gls[o];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[kb][nb] = mfma_bf(aq, cf[kb][ks], s[kb][nb]);
          dp[kb][nb] = mfma_bf(ah, cf[kb][ks], dp[kb][nb]);
          dp[kb][nb] = mfma_bf(al, cf[kb][ks], dp[kb][nb]);
        }
      }
    // P and scale * dS in two bf16 parts, rows 4 lg + e then 16 + 4 lg + e
    bf16x8 ph[2], pl[2], dh[2], dl[2];
    auto make_p = [&](auto unmasked) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const f32x4 lse4 = *(const f32x4*)&s_lse2[buf][nb * 16 + lg * 4];
        const f32x4 D4 = *(const f32x4*)&s_D[buf][nb * 16 + lg * 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = t0 + nb * 16 + lg * 4 + e;
          int pos = 0;
          if constexpr (!decltype(unmasked)::value) pos = t < ur.total ? ur.pos(t) : -1;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const int key = kw + kb * 16 + lr;
            const bool ok = decltype(unmasked)::value || key <= pos;
            const float pr = ok ? exp2_hw(s[kb][nb][e] * sl2 - lse4[e]) : 0.f;
            const float ds = p.scale * pr * (dp[kb][nb][e] - D4[e]);
            const bf16 a = to_bf16(pr), b = to_bf16(ds);
            ph[kb][nb * 4 + e] = a;
            pl[kb][nb * 4 + e] = to_bf16(pr - from_bf16(a));
            dh[kb][nb * 4 + e] = b;
            dl[kb][nb * 4 + e] = to_bf16(ds - from_bf16(b));
          }
        }
      }
    };
    // all 32 rows valid and seeing all of the wave's keys (the smallest
    // position is the first row's): no mask (a wave-uniform branch)
    if (t0 + kCRows <= ur.total && ur.pos(t0) >= kw + 31) make_p(std::true_type{});
    else make_p(std::false_type{});
    // d_C += P^T d_out + scale dS^T q: A = d_out^T / q^T rows rb*16..
    // (transpose loads over the tile's 32 rows), B = P^T / dS^T
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int o0 = trow * LD + rb * 16 + tcol, o1 = (16 + trow) * LD + rb * 16 + tcol;
      const bf16x8 agh = cat8(lds_tr(ghs + o0), lds_tr(ghs + o1));
      const bf16x8 agl = cat8(lds_tr(gls + o0), lds_tr(gls + o1));
      const bf16x8 aq = cat8(lds_tr(qs + o0), lds_tr(qs + o1));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        dc[kb][rb] = mfma_bf(agh, ph[kb], dc[kb][rb]);
        dc[kb][rb] = mfma_bf(agl, ph[kb], dc[kb][rb]);
        dc[kb][rb] = mfma_bf(agh, pl[kb], dc[kb][rb]);
        dc[kb][rb] = mfma_bf(aq, dh[kb], dc[kb][rb]);
        dc[kb][rb] = mfma_bf(aq, dl[kb], dc[kb][rb]);
      }
    }
    if (it + 1 < nit) lstore(buf ^ 1);
    __syncthreads();
  }
  // lane holds d_C[key kb*16 + lr][rb*16 + 4 lg .. + 3]
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kw + kb * 16 + lr;
    if (key >= ur.K) continue;
    float* dst = p.dc + (size_t)(ur.kv0 + key) * R + lg * 4;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      if (p.dc_accumulate) {
#pragma unroll
        for (int e = 0; e < 4; ++e) unsafeAtomicAdd(dst + rb * 16 + e, dc[kb][rb][e]);
      } else {
        *(f32x4*)(dst + rb * 16) = dc[kb][rb];
      }
    }
  }
}

size_t attention_backward_workspace(long long Mtot, int h, int r) {
  const size_t elems = (size_t)Mtot * h * r;
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  return 2 * up(elems * sizeof(bf16)) + up((size_t)Mtot * h * sizeof(float));
}

hipError_t attention_backward(AttnBwdParams p, int max_len, void* ws, hipStream_t s) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t ge = up((size_t)p.Mtot * p.h * p.r * sizeof(bf16));
  char* w = (char*)ws;
  p.ws_ghi = (bf16*)w;
  p.ws_glo = (bf16*)(w + ge);
  p.ws_d = (float*)(w + 2 * ge);
  // two head groups (deterministic: each d_C element gets exactly two
  // additions onto zero) when the heads split evenly
  p.dc_accumulate = p.h % 2 == 0;
  const int ngroups = p.dc_accumulate ? 2 : 1;
  const dim3 gq(p.B * p.h, (max_len + p.n_cand + kQRows - 1) / kQRows);
  const dim3 gc(p.B * ngroups, (max_len + kCKeys - 1) / kCKeys);
  timing_begin("attn_bwd_dq", s);
  if (p.r == 64) hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, gq, dim3(256), 0, s, p);
  else if (p.r == 128) hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, gq, dim3(256), 0, s, p);
  else return hipErrorInvalidValue;
  timing_end(s);
  hipError_t e = hipGetLastError();
  if (e) return e;
  timing_begin("attn_bwd_dc", s);
  if (p.r == 64) hipLaunchKernelGGL(attn_bwd_dc_kernel<64>, gc, dim3(256), 0, s, p);
  else hipLaunchKernelGGL(attn_bwd_dc_kernel<128>, gc, dim3(256), 0, s, p);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace llatte
