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
// dS is stored. Two kernels: one per (64-row query block, user, head) for
// d_q, looping over key tiles; one per (64-key tile, user) for d_C, looping
// over heads and the query blocks that see the tile. Each keeps its tiles in
// LDS as bf16 with 16-byte row padding (rows 16 bytes apart modulo the bank
// window), and stages the dS / P blocks through LDS to feed the next
// product.
#include "kernels.hpp"

namespace llatte {

namespace {

constexpr int kRows = 64;   // query rows per block, keys per tile

__device__ __forceinline__ f32x4 mfma_bf(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A user's query rows in the forward's order: history rows t < n (key
// position K - n + t), then the candidates (position K - 1).
struct UserRows {
  int K, n, total, kv0;
  __device__ int global_row(int t, int u, int nc, const int* hq_off, int n_cand) const {
    return t < n ? nc + hq_off[u] + t : u * n_cand + (t - n);
  }
  __device__ int pos(int t) const { return t < n ? K - n + t : K - 1; }
};

__device__ __forceinline__ UserRows user_rows(const AttnBwdParams& p, int u) {
  UserRows r;
  r.kv0 = p.kv_off[u];
  r.K = p.kv_off[u + 1] - r.kv0;
  r.n = p.hq_off[u + 1] - p.hq_off[u];
  r.total = r.n + p.n_cand;
  return r;
}

// d_out as two bf16 parts, hi = bf16(x) and lo = bf16(x - hi): dP = d_out . C
// from both parts keeps fp32-level accuracy, so that dP - D (D from the fp32
// d_out and out) does not cancel into the rounding of d_out.
__device__ __forceinline__ void split_bf16(const float* x, bf16x8& hi, bf16x8& lo) {
  const f32x4 a = *(const f32x4*)x, b = *(const f32x4*)(x + 4);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float v = i < 4 ? a[i] : b[i - 4];
    hi[i] = to_bf16(v);
    lo[i] = to_bf16(v - from_bf16(hi[i]));
  }
}

// Row `lr` of a padded [rows][LD] bf16 tile, 16-byte piece `c`
template <int LD>
__device__ __forceinline__ bf16x8 frag(const bf16* t, int row, int k0) {
  return *(const bf16x8*)(t + row * LD + k0);
}

}  // namespace

// d_q for query rows [t0, t0 + 64) of user blockIdx.y, head blockIdx.z.
template <int R>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(AttnBwdParams p) {
  constexpr int LDR = R + 8;       // padded row of an R-wide tile
  constexpr int LDK = kRows + 8;   // padded row of a 64-wide tile
  __shared__ __attribute__((aligned(16))) bf16 Qs[kRows * LDR];
  __shared__ __attribute__((aligned(16))) bf16 Gs[kRows * LDR];   // d_out, bf16 high part
  __shared__ __attribute__((aligned(16))) bf16 GLs[kRows * LDR];  // d_out - high part
  __shared__ __attribute__((aligned(16))) bf16 Cs[kRows * LDR];
  __shared__ __attribute__((aligned(16))) bf16 CTs[R * LDK];
  __shared__ __attribute__((aligned(16))) bf16 DSs[kRows * LDK];   // dS, bf16 high part
  __shared__ __attribute__((aligned(16))) bf16 DSLs[kRows * LDK];  // dS - high part
  __shared__ float s_lse[kRows], s_D[kRows];
  __shared__ int s_pos[kRows];
  const int u = blockIdx.y, hh = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const UserRows ur = user_rows(p, u);
  const int t0 = blockIdx.x * kRows;
  if (t0 >= ur.total) return;
  const int nc = p.B * p.n_cand, h = p.h;

  // rows: q (bf16), d_out (to bf16), lse, D = d_out . out, key position
  for (int e = tid; e < kRows * (R / 8); e += 256) {
    const int rr = e / (R / 8), c = (e % (R / 8)) * 8, t = t0 + rr;
    bf16x8 qv = {}, gv = {}, gl = {};
    if (t < ur.total) {
      const size_t g = ((size_t)ur.global_row(t, u, nc, p.hq_off, p.n_cand) * h + hh) * R + c;
      qv = *(const bf16x8*)((const bf16*)p.q + g);
      split_bf16(p.dout + g, gv, gl);
    }
    *(bf16x8*)&Qs[rr * LDR + c] = qv;
    *(bf16x8*)&Gs[rr * LDR + c] = gv;
    *(bf16x8*)&GLs[rr * LDR + c] = gl;
  }
  {  // four threads per row
    const int rr = tid >> 2, part = tid & 3, t = t0 + rr;
    float d = 0.f;
    size_t g = 0;
    if (t < ur.total) {
      g = (size_t)ur.global_row(t, u, nc, p.hq_off, p.n_cand) * h + hh;
      for (int k = part * (R / 4); k < (part + 1) * (R / 4); ++k)
        d = fmaf(p.dout[g * R + k], p.out[g * R + k], d);
    }
    d += __shfl_xor(d, 1, 64);
    d += __shfl_xor(d, 2, 64);
    if (part == 0) {
      s_D[rr] = d;
      s_lse[rr] = t < ur.total ? p.lse[g] : 0.f;
      s_pos[rr] = t < ur.total ? ur.pos(t) : -1;
    }
  }
  __syncthreads();
  const int last = min(ur.total, t0 + kRows) - 1;
  const int ntiles = ur.pos(last) / kRows + 1;  // positions grow with t

  const int myrow = wave * 16 + lr;  // this lane's query row within the block
  const float lse = s_lse[myrow], D = s_D[myrow];
  const int pos = s_pos[myrow];
  const float sl2 = p.scale * 1.4426950408889634f;
  f32x4 dq[R / 16];
#pragma unroll
  for (int b = 0; b < R / 16; ++b) dq[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * kRows;
    for (int e = tid; e < kRows * (R / 8); e += 256) {
      const int key = e / (R / 8), c = (e % (R / 8)) * 8;
      bf16x8 v = {};
      if (k0 + key < ur.K) v = *(const bf16x8*)((const bf16*)p.c + (size_t)(ur.kv0 + k0 + key) * R + c);
      *(bf16x8*)&Cs[key * LDR + c] = v;
#pragma unroll
      for (int i = 0; i < 8; ++i) CTs[(c + i) * LDK + key] = v[i];
    }
    __syncthreads();
    // S and dP for this wave's 16 rows x 64 keys: lane holds row lr, keys
    // nb*16 + 4*lg .. +3
    f32x4 s[4], dp[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      s[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < R / 32; ++ks) {
      const bf16x8 qa = frag<LDR>(Qs, wave * 16 + lr, ks * 32 + lg * 8);
      const bf16x8 ga = frag<LDR>(Gs, wave * 16 + lr, ks * 32 + lg * 8);
      const bf16x8 gla = frag<LDR>(GLs, wave * 16 + lr, ks * 32 + lg * 8);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const bf16x8 cb = frag<LDR>(Cs, nb * 16 + lr, ks * 32 + lg * 8);
        s[nb] = mfma_bf(cb, qa, s[nb]);
        dp[nb] = mfma_bf(cb, ga, dp[nb]);
        dp[nb] = mfma_bf(cb, gla, dp[nb]);
      }
    }
    // dS = P (dP - D), P = exp(scale s - lse) on allowed keys
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      bf16x4 o, ol;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = k0 + nb * 16 + lg * 4 + e;
        const bool ok = key <= pos && key < ur.K;
        const float pr = ok ? exp2f(s[nb][e] * sl2 - lse * 1.4426950408889634f) : 0.f;
        const float ds = pr * (dp[nb][e] - D);
        o[e] = to_bf16(ds);
        ol[e] = to_bf16(ds - from_bf16(o[e]));
      }
      *(bf16x4*)&DSs[myrow * LDK + nb * 16 + lg * 4] = o;
      *(bf16x4*)&DSLs[myrow * LDK + nb * 16 + lg * 4] = ol;
    }
    // d_q rows += dS C: A = dS rows (k = keys) in two bf16 parts (the dS of
    // a row sum to zero, so d_q is a small difference of large terms),
    // B = C^T rows (k = keys)
#pragma unroll
    for (int ks = 0; ks < kRows / 32; ++ks) {
      const bf16x8 da = frag<LDK>(DSs, wave * 16 + lr, ks * 32 + lg * 8);
      const bf16x8 dla = frag<LDK>(DSLs, wave * 16 + lr, ks * 32 + lg * 8);
#pragma unroll
      for (int rb = 0; rb < R / 16; ++rb) {
        const bf16x8 cb = frag<LDK>(CTs, rb * 16 + lr, ks * 32 + lg * 8);
        dq[rb] = mfma_bf(cb, da, dq[rb]);
        dq[rb] = mfma_bf(cb, dla, dq[rb]);
      }
    }
    __syncthreads();
  }
  const int t = t0 + myrow;
  if (t < ur.total) {
    float* dst = p.dq + ((size_t)ur.global_row(t, u, nc, p.hq_off, p.n_cand) * h + hh) * R;
#pragma unroll
    for (int rb = 0; rb < R / 16; ++rb)
      *(f32x4*)(dst + rb * 16 + lg * 4) = dq[rb] * p.scale;
  }
}

// d_C for keys [k0, k0 + 64) of user blockIdx.y, over every head and every
// query block (32 rows) that sees them. d_C_j sums many terms of both signs,
// so P, d_out and dS enter the products as two bf16 parts each (high part
// plus the rounding remainder); only the negligible lo x lo terms are left.
template <int R>
__global__ __launch_bounds__(256) void attn_bwd_dc_kernel(AttnBwdParams p) {
  constexpr int QB = 32;           // query rows per block
  constexpr int LDR = R + 8;
  constexpr int LDQ = QB + 8;
  __shared__ __attribute__((aligned(16))) bf16 Cs[kRows * LDR];
  __shared__ __attribute__((aligned(16))) bf16 Qs[QB * LDR];
  __shared__ __attribute__((aligned(16))) bf16 Gs[QB * LDR];
  __shared__ __attribute__((aligned(16))) bf16 GLs[QB * LDR];
  __shared__ __attribute__((aligned(16))) bf16 QTs[R * LDQ];
  __shared__ __attribute__((aligned(16))) bf16 GTs[R * LDQ];
  __shared__ __attribute__((aligned(16))) bf16 GLTs[R * LDQ];
  __shared__ __attribute__((aligned(16))) bf16 PTs[kRows * LDQ];
  __shared__ __attribute__((aligned(16))) bf16 PLTs[kRows * LDQ];
  __shared__ __attribute__((aligned(16))) bf16 DTs[kRows * LDQ];
  __shared__ __attribute__((aligned(16))) bf16 DLTs[kRows * LDQ];
  __shared__ float s_lse[QB], s_D[QB];
  __shared__ int s_pos[QB];
  const int u = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const UserRows ur = user_rows(p, u);
  const int k0 = blockIdx.x * kRows;
  if (k0 >= ur.K) return;
  const int nc = p.B * p.n_cand, h = p.h;
  for (int e = tid; e < kRows * (R / 8); e += 256) {
    const int key = e / (R / 8), c = (e % (R / 8)) * 8;
    bf16x8 v = {};
    if (k0 + key < ur.K) v = *(const bf16x8*)((const bf16*)p.c + (size_t)(ur.kv0 + k0 + key) * R + c);
    *(bf16x8*)&Cs[key * LDR + c] = v;
  }
  const int mykey = wave * 16 + lr;  // this lane's key within the tile
  const float sl2 = p.scale * 1.4426950408889634f;
  f32x4 dc[R / 16];
#pragma unroll
  for (int b = 0; b < R / 16; ++b) dc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // history rows at positions below k0 see none of these keys
  const int t_first = max(0, k0 - (ur.K - ur.n)) / QB * QB;

  for (int hh = 0; hh < h; ++hh) {
    for (int t0 = t_first; t0 < ur.total; t0 += QB) {
      __syncthreads();  // previous block's tiles are consumed
      for (int e = tid; e < QB * (R / 8); e += 256) {
        const int rr = e / (R / 8), c = (e % (R / 8)) * 8, t = t0 + rr;
        bf16x8 qv = {}, gv = {}, gl = {};
        if (t < ur.total) {
          const size_t g = ((size_t)ur.global_row(t, u, nc, p.hq_off, p.n_cand) * h + hh) * R + c;
          qv = *(const bf16x8*)((const bf16*)p.q + g);
          split_bf16(p.dout + g, gv, gl);
        }
        *(bf16x8*)&Qs[rr * LDR + c] = qv;
        *(bf16x8*)&Gs[rr * LDR + c] = gv;
        *(bf16x8*)&GLs[rr * LDR + c] = gl;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          QTs[(c + i) * LDQ + rr] = qv[i];
          GTs[(c + i) * LDQ + rr] = gv[i];
          GLTs[(c + i) * LDQ + rr] = gl[i];
        }
      }
      if (tid < QB * 4) {  // four threads per row
        const int rr = tid >> 2, part = tid & 3, t = t0 + rr;
        float d = 0.f;
        size_t g = 0;
        if (t < ur.total) {
          g = (size_t)ur.global_row(t, u, nc, p.hq_off, p.n_cand) * h + hh;
          for (int k = part * (R / 4); k < (part + 1) * (R / 4); ++k)
            d = fmaf(p.dout[g * R + k], p.out[g * R + k], d);
        }
        d += __shfl_xor(d, 1, 64);
        d += __shfl_xor(d, 2, 64);
        if (part == 0) {
          s_D[rr] = d;
          s_lse[rr] = t < ur.total ? p.lse[g] : 0.f;
          s_pos[rr] = t < ur.total ? ur.pos(t) : -1;
        }
      }
      __syncthreads();
      // S^T and dP^T for this wave's 16 keys x 32 rows: lane holds key lr,
      // rows nb*16 + 4*lg .. +3
      f32x4 s[2], dp[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        s[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int ks = 0; ks < R / 32; ++ks) {
        const bf16x8 ca = frag<LDR>(Cs, wave * 16 + lr, ks * 32 + lg * 8);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          s[nb] = mfma_bf(frag<LDR>(Qs, nb * 16 + lr, ks * 32 + lg * 8), ca, s[nb]);
          dp[nb] = mfma_bf(frag<LDR>(Gs, nb * 16 + lr, ks * 32 + lg * 8), ca, dp[nb]);
          dp[nb] = mfma_bf(frag<LDR>(GLs, nb * 16 + lr, ks * 32 + lg * 8), ca, dp[nb]);
        }
      }
      const int key = k0 + mykey;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        bf16x4 ph, pl, dh, dl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = nb * 16 + lg * 4 + e;
          const bool ok = key <= s_pos[rr] && key < ur.K;
          const float pr = ok ? exp2f(s[nb][e] * sl2 - s_lse[rr] * 1.4426950408889634f) : 0.f;
          const float ds = p.scale * pr * (dp[nb][e] - s_D[rr]);
          ph[e] = to_bf16(pr);
          pl[e] = to_bf16(pr - from_bf16(ph[e]));
          dh[e] = to_bf16(ds);
          dl[e] = to_bf16(ds - from_bf16(dh[e]));
        }
        const int o = mykey * LDQ + nb * 16 + lg * 4;
        *(bf16x4*)&PTs[o] = ph;
        *(bf16x4*)&PLTs[o] = pl;
        *(bf16x4*)&DTs[o] = dh;
        *(bf16x4*)&DLTs[o] = dl;
      }
      // d_C keys += P^T d_out + scale dS^T q (k = the block's 32 rows)
      {
        const int ko = lg * 8;
        const bf16x8 pa = frag<LDQ>(PTs, wave * 16 + lr, ko);
        const bf16x8 pla = frag<LDQ>(PLTs, wave * 16 + lr, ko);
        const bf16x8 da = frag<LDQ>(DTs, wave * 16 + lr, ko);
        const bf16x8 dla = frag<LDQ>(DLTs, wave * 16 + lr, ko);
#pragma unroll
        for (int rb = 0; rb < R / 16; ++rb) {
          const bf16x8 gb = frag<LDQ>(GTs, rb * 16 + lr, ko);
          const bf16x8 glb = frag<LDQ>(GLTs, rb * 16 + lr, ko);
          const bf16x8 qb = frag<LDQ>(QTs, rb * 16 + lr, ko);
          dc[rb] = mfma_bf(gb, pa, dc[rb]);
          dc[rb] = mfma_bf(glb, pa, dc[rb]);
          dc[rb] = mfma_bf(gb, pla, dc[rb]);
          dc[rb] = mfma_bf(qb, da, dc[rb]);
          dc[rb] = mfma_bf(qb, dla, dc[rb]);
        }
      }
    }
  }
  if (k0 + mykey < ur.K) {
    float* dst = p.dc + (size_t)(ur.kv0 + k0 + mykey) * R;
#pragma unroll
    for (int rb = 0; rb < R / 16; ++rb) *(f32x4*)(dst + rb * 16 + lg * 4) = dc[rb];
  }
}

hipError_t attention_backward(const AttnBwdParams& p, int max_len, hipStream_t s) {
  const dim3 gq((max_len + p.n_cand + kRows - 1) / kRows, p.B, p.h);
  const dim3 gc((max_len + kRows - 1) / kRows, p.B, 1);
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
