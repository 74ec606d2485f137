// Shared device types and helpers for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llatte {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// float -> bf16 with the hardware conversion (round to nearest even).
__device__ __forceinline__ bf16 to_bf16(float f) { return (bf16)f; }
__device__ __forceinline__ float from_bf16(bf16 b) {
  return __builtin_bit_cast(float, ((uint32_t)__builtin_bit_cast(uint16_t, b)) << 16);
}

template <typename T> __device__ __forceinline__ T cvt(float f);
template <> __device__ __forceinline__ float cvt<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16 cvt<bf16>(float f) { return to_bf16(f); }
template <> __device__ __forceinline__ f16 cvt<f16>(float f) { return (f16)f; }
__device__ __forceinline__ float tof(float f) { return f; }
__device__ __forceinline__ float tof(bf16 b) { return from_bf16(b); }

// Sum / max over the 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Sum over the four lanes l, l^16, l^32, l^48 (one column, or one row, of
// an MFMA accumulator block across its four 16-lane groups). Each permlane
// swap gives a lane its own value and its partner's; the two lanes of a pair
// add the same two numbers, so all four lanes end with the same bits.
__device__ __forceinline__ float group_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Rows of a layer's row space: the first `nc` rows live at `c`, the rest at
// `h` (row i >= nc is h[(i - nc)]). For layers after the first both blocks
// sit in one buffer with h == c + nc * ld.
struct RowSrc {
  const float* c;
  const float* h;
  int nc;
  int ld;
  __device__ __forceinline__ const float* row(int i) const {
    return i < nc ? c + (size_t)i * ld : h + (size_t)(i - nc) * ld;
  }
};

// Device-side count with a host-side capacity: kernels are launched for the
// capacity and rows at or beyond *dev (when given) do no work.
__device__ __forceinline__ int dev_count(const int* dev, int cap) {
  return dev ? min(*dev, cap) : cap;
}

}  // namespace llatte
