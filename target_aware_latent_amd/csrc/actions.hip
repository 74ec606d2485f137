// Action tokenization ([LLaTTE] Appendix A.2, Sequence Module item 1): the
// per-field embeddings of every action side by side, ready for MLP_act.
//
// One thread writes one 16-byte piece of a row of U = [E_type(type) |
// E_item(item) | E_surf(surface) | E_time(bucket(age)) | meta W_meta]. Field
// widths are multiples of the piece, so a piece never straddles two fields.
// The age of an action is its user's request time minus its timestamp
// (negative taken as 0), the time bucket floor(log2(1 + age)) clamped to the
// last table row; ids outside their table are clamped into it, so a bad id
// cannot read past a table. Each block also writes the ages of its rows,
// which the second product's epilogue turns into the timestamp encoding.
#include "kernels.hpp"

namespace llatte {

__device__ __forceinline__ int clampi(int v, int hi) { return min(max(v, 0), hi - 1); }

// Row -> user by binary search over the exclusive offsets (offsets[0] = 0,
// offsets[B] = n): the largest u with offsets[u] <= row. Any offsets give a
// user in [0, B), so the request-time read stays in bounds.
__device__ __forceinline__ int row_user(const int* offsets, int B, int row) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= row) lo = mid;
    else hi = mid;
  }
  return lo;
}

template <typename T>
__global__ __launch_bounds__(256) void action_concat_kernel(ActionConcat p) {
  constexpr int CE = 16 / sizeof(T);
  const int cpr = p.d_in / CE;
  // The block's rows: one lane per row finds the row's user and age (the
  // searches run side by side), shared through LDS.
  __shared__ int s_age[258];
  const long long g0 = (long long)blockIdx.x * 256;
  const long long total = (long long)p.n * cpr;
  const int r_first = (int)(g0 / cpr);
  const int r_last = (int)((min(g0 + 256, total) - 1) / cpr);
  if ((int)threadIdx.x <= r_last - r_first) {
    const int r = r_first + threadIdx.x;
    const int u = row_user(p.offsets, p.B, r);
    long long a = (long long)p.t_req[u] - (long long)p.tau[r];
    a = a < 0 ? 0 : (a > 0x7FFFFFFFLL ? 0x7FFFFFFFLL : a);
    s_age[threadIdx.x] = (int)a;
    p.age[r] = (int)a;
  }
  __syncthreads();
  const long long g = g0 + threadIdx.x;
  if (g >= total) return;
  const int row = (int)(g / cpr), c0 = (int)(g % cpr) * CE;
  const int o_item = p.d_type, o_surf = o_item + p.d_item, o_time = o_surf + p.d_surf;
  const int o_meta = o_time + p.d_time;
  const int age = s_age[row - r_first];
  T* dst = (T*)p.U + (size_t)row * p.d_in + c0;
  const T* src;
  if (c0 < o_item) {
    src = (const T*)p.E_type + (size_t)clampi(p.type_id[row], p.V_type) * p.d_type + c0;
  } else if (c0 < o_surf) {
    src = (const T*)p.E_item + (size_t)clampi(p.item_id[row], p.V_item) * p.d_item + (c0 - o_item);
  } else if (c0 < o_time) {
    src = (const T*)p.E_surf + (size_t)clampi(p.surf_id[row], p.V_surf) * p.d_surf + (c0 - o_surf);
  } else if (c0 < o_meta) {
    // floor(log2(1 + age)) = 31 - clz(1 + age); 1 + age fits in 32 bits unsigned
    const int b = 31 - __builtin_clz((unsigned)age + 1u);
    src = (const T*)p.E_time + (size_t)min(b, p.n_buckets - 1) * p.d_time + (c0 - o_time);
  } else {
    // meta W_meta for the CE output columns of this piece, fp32 accumulation
    const int j0 = c0 - o_meta;
    const T* m = (const T*)p.meta + (size_t)row * p.d_meta;
    float acc[CE];
#pragma unroll
    for (int e = 0; e < CE; ++e) acc[e] = 0.f;
    // meta row and W_meta rows in 16-byte pieces (widths are multiples)
    for (int k0 = 0; k0 < p.d_meta; k0 += CE) {
      const i32x4 mraw = *(const i32x4*)(m + k0);
      const T* mv = (const T*)&mraw;
#pragma unroll
      for (int kk = 0; kk < CE; ++kk) {
        const i32x4 wraw = *(const i32x4*)((const T*)p.W_meta + (size_t)(k0 + kk) * p.d_meta_emb + j0);
        const T* wv = (const T*)&wraw;
        const float mk = tof(mv[kk]);
#pragma unroll
        for (int e = 0; e < CE; ++e) acc[e] = fmaf(mk, tof(wv[e]), acc[e]);
      }
    }
    if constexpr (__is_same(T, bf16)) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = to_bf16(acc[e]);
      *(bf16x8*)dst = o;
    } else {
      *(f32x4*)dst = f32x4{acc[0], acc[1], acc[2], acc[3]};
    }
    return;
  }
  *(i32x4*)dst = *(const i32x4*)src;
}

hipError_t action_concat(const ActionConcat& p, bool is_bf16, hipStream_t s) {
  if (p.n <= 0) return hipSuccess;
  const int ce = is_bf16 ? 8 : 4;
  const long long threads = (long long)p.n * (p.d_in / ce);
  const unsigned grid = (unsigned)((threads + 255) / 256);
  timing_begin("action_concat", s);
  if (is_bf16)
    hipLaunchKernelGGL(action_concat_kernel<bf16>, dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(action_concat_kernel<float>, dim3(grid), dim3(256), 0, s, p);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace llatte
