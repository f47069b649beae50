// Shared device-side helpers for the gfx950 kernels: element types, MFMA fragment traits,
// wave-level reductions and rounding.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dm {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int WAVE = 64;

// --------------------------------------------------------------------------- MFMA fragments
// Every matrix operand fragment is 16 bytes per lane: EPL consecutive elements along the
// contraction axis.  For a 16x16 output tile, lane l supplies row (l % 16) of A and column
// (l % 16) of B, for the contraction indices [g*EPL, (g+1)*EPL) with g = l / 16; one
// "k-chunk" therefore spans 4*EPL contraction indices.  The result tile holds, in lane l and
// register i, element (row 4*(l/16) + i, column l % 16).
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  typedef bf16x8 frag;
  static constexpr int EPL = 8;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

// fp32: one 16-byte fragment = 4 floats; four 16x16x4 MFMAs, the j-th taking element j of
// every lane, so contraction index (g*4 + j) of A meets the same index of B.
template <> struct Mfma<float> {
  typedef f32x4 frag;
  static constexpr int EPL = 4;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
};

template <typename T> __device__ __forceinline__ typename Mfma<T>::frag load_frag(const T *p) {
  return *reinterpret_cast<const typename Mfma<T>::frag *>(p);
}

template <typename T> __device__ __forceinline__ typename Mfma<T>::frag zero_frag() {
  typename Mfma<T>::frag z;
#pragma unroll
  for (int i = 0; i < Mfma<T>::EPL; ++i) z[i] = T(0.0f);
  return z;
}

// --------------------------------------------------------------------------- conversions
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// Round to nearest even, written out on the bit pattern (finite inputs).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return __builtin_bit_cast(bf16, (uint16_t)(u >> 16));
}
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) {
  return __uint_as_float(((uint32_t)__builtin_bit_cast(uint16_t, x)) << 16);
}

// --------------------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace dm
