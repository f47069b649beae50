// Shared device-side helpers for the gfx950 kernels: element types, MFMA fragment traits,
// wave-level reductions and rounding.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "addr_words.h"

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

// FP8 E4M3 (OCP e4m3fn) codes, one byte per element.  One 16x16x128 MFMA per k-chunk: lane l
// supplies row (l % 16) of A and column (l % 16) of B for 32 contraction indices, 32 bytes per
// lane; A and B fragments are loaded with the same byte-to-index map, so the product is exact
// whatever order the hardware walks those 32 indices in.  Scale operands 0x7F are E8M0 2^0
// (unscaled); the per-token and per-channel scales are applied in the epilogue.
typedef uint8_t fp8;
typedef __attribute__((ext_vector_type(8))) int i32x8;
struct Mfma8 {
  typedef i32x8 frag;
  static constexpr int EPL = 32;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0x7F7F7F7F, 0, 0x7F7F7F7F);
  }
};

template <typename T> __device__ __forceinline__ typename Mfma<T>::frag load_frag(const T *p) {
  return *reinterpret_cast<const typename Mfma<T>::frag *>(p);
}

// Loads a fragment from a valid address and zeroes it when `ok` is false, without a branch
// around the load (so all loads of an unrolled sequence stay in flight together).
template <typename T> __device__ __forceinline__ typename Mfma<T>::frag load_frag_masked(const T *p, bool ok) {
  const i32x4 v = __builtin_bit_cast(i32x4, *reinterpret_cast<const typename Mfma<T>::frag *>(p));
  const int m = ok ? -1 : 0;
  return __builtin_bit_cast(typename Mfma<T>::frag, v & i32x4{m, m, m, m});
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
// Round to nearest even: one v_cvt_pk_bf16_f32 on gfx950.
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) {
  return __uint_as_float(((uint32_t)__builtin_bit_cast(uint16_t, x)) << 16);
}

// --------------------------------------------------------------------------- cross-lane
// Lane exchanges: DPP within 16-lane rows (no LDS crossbar), gfx950 permlane swaps across rows.
// A row is lanes 16r..16r+15.
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15-i within each row

// Reductions over lane pairs (l, l^16) and (l, l^32) with gfx950's v_permlane16/32_swap: given
// the same register twice, the two results hold v[l] and v[l^16] (resp. l^32) in some order, so
// their sum or max is the pair's, bitwise identical in both lanes; no LDS round trip.
__device__ __forceinline__ float sum_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
// Sum over the 4 lanes of a quad, the 16 lanes of a row, and the whole wave.
__device__ __forceinline__ float sum4(float v) {
  v += dpp<DPP_XOR1>(v);
  return v + dpp<DPP_XOR2>(v);
}
__device__ __forceinline__ float sum16(float v) {
  v = sum4(v);
  v += dpp<DPP_HALF_MIRROR>(v);
  return v + dpp<DPP_MIRROR>(v);
}
__device__ __forceinline__ float wave_sum(float v) { return sum_xor32(sum_xor16(sum16(v))); }
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<DPP_XOR1>(v));
  v = fmaxf(v, dpp<DPP_XOR2>(v));
  v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_MIRROR>(v));
  return max_xor32(max_xor16(v));
}

// silu(z) = z / (1 + e^-z), with the hardware exponential and reciprocal (about 1 ulp each).
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// ---------------------------------------------------------------- global -> LDS copies
// Workgroup barrier without a global-memory fence (a fence would wait for every outstanding
// load, prefetches included).  It waits for this wave's LDS reads first, so no wave can start a
// copy into a buffer another wave is still reading; the memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ unsigned lds_addr(const void *p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
// global -> LDS copy of 16 bytes per lane: lane l writes LDS bytes [lds + 16 l, lds + 16 l + 16)
// (lds is wave-uniform, in M0).  Written as asm so that the compiler does not treat later LDS
// reads of other buffers as waiting on it; the consumer waits for these copies explicitly
// (s_waitcnt vmcnt + barrier).  It has no output register: the data lands in LDS.
__device__ __forceinline__ void dma16(const void *g, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
// The same copy addressed as a wave-uniform 64-bit base (SGPRs) plus a 32-bit per-lane byte
// offset, so a stream of copies needs no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void dma16_sbase(const void *base, unsigned off, unsigned lds) {
  const unsigned long long b = (unsigned long long)(uintptr_t)base;
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)addr_lo(b));
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)addr_hi(b));
  const unsigned long long sb = addr_join(lo, hi);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(sb),
               "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
// wait until at most N of this wave's vector-memory operations are outstanding (they complete
// in issue order)
template <int N> __device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace dm

