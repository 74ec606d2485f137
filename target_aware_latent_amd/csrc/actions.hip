// Action tokenization ([LLaTTE] Appendix A.2, Sequence Module item 1): the
// per-field embeddings of every action side by side, ready for MLP_act.
//
// One thread writes one 16-byte piece of a row of U = [E_type(type) |
// E_item(item) | E_surf(surface) | E_time(bucket(age)) | meta W_meta]. Field
// widths are multiples of the piece, so a piece never straddles two fields.
// The age of an action is its user's request time minus its timestamp
// (negative taken as 0), the time bucket floor(log2(1 + age)) clamped to the
// last table row; ids outside their table are clamped into it, so a bad id
// cannot read past a table. The thread of a row's first piece also writes
// the row's age, which the second product's epilogue turns into the
// timestamp encoding.
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
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  if (g >= (long long)p.n * cpr) return;
  const int row = (int)(g / cpr), c0 = (int)(g % cpr) * CE;
  const int o_item = p.d_type, o_surf = o_item + p.d_item, o_time = o_surf + p.d_surf;
  const int o_meta = o_time + p.d_time;
  int age = 0;
  if (c0 == 0 || (c0 >= o_time && c0 < o_meta)) {
    const int u = row_user(p.offsets, p.B, row);
    long long a = (long long)p.t_req[u] - (long long)p.tau[row];
    a = a < 0 ? 0 : (a > 0x7FFFFFFFLL ? 0x7FFFFFFFLL : a);
    age = (int)a;
    if (c0 == 0) p.age[row] = age;
  }
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
    for (int k = 0; k < p.d_meta; ++k) {
      const float mk = tof(m[k]);
      const T* w = (const T*)p.W_meta + (size_t)k * p.d_meta_emb + j0;
#pragma unroll
      for (int e = 0; e < CE; ++e) acc[e] = fmaf(mk, tof(w[e]), acc[e]);
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
