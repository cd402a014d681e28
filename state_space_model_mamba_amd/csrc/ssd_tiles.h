// Global <-> LDS staging helpers shared by the SSD kernels.
#pragma once

#include "ssd_device.h"

namespace ssd {

template <typename T> struct Vec16 {
  static constexpr int N = 16 / static_cast<int>(sizeof(T));
};

__device__ __forceinline__ uint4 ld_global16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ uint4 zero_u4() { return uint4{0u, 0u, 0u, 0u}; }

// element e of a 16-byte vector holding T values
template <typename T> __device__ __forceinline__ T vraw(const uint4& v, int e);
template <> __device__ __forceinline__ bf16_t vraw<bf16_t>(const uint4& v, int e) {
  const uint32_t w = (&v.x)[e >> 1];
  return static_cast<bf16_t>((e & 1) ? (w >> 16) : (w & 0xffffu));
}
template <> __device__ __forceinline__ float vraw<float>(const uint4& v, int e) {
  return __uint_as_float((&v.x)[e]);
}

template <typename T> __device__ __forceinline__ float vget(const uint4& v, int e) {
  return Elem<T>::to_f(vraw<T>(v, e));
}

// Masked KW-fragment of a K-major operand: elements whose k index falls
// outside [lo, hi) read as zero.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag load_k_masked(const T* p, int k, int lo, int hi);
template <>
__device__ __forceinline__ Mma<bf16_t>::frag load_k_masked<bf16_t>(const bf16_t* p, int k, int lo, int hi) {
  u16x8_t v = *reinterpret_cast<const u16x8_t*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (k + e < lo || k + e >= hi) v[e] = 0;
  return __builtin_bit_cast(Mma<bf16_t>::frag, v);
}
template <>
__device__ __forceinline__ float load_k_masked<float>(const float* p, int k, int lo, int hi) {
  return (k < lo || k >= hi) ? 0.f : *p;
}

// Like tile_mma_kk, but only k in [lo, hi) contributes (A elements outside
// read as zero).
template <typename T>
__device__ __forceinline__ f32x4_t tile_mma_kk_range(f32x4_t acc, const T* a_base, int lda,
                                                     const T* b_base, int ldb, int lo, int hi) {
  constexpr int KS = Mma<T>::KSTEP, KW = Mma<T>::KW;
  const int l = lane_id();
  const int r16 = l & 15, kg = l >> 4;
  const T* ap = a_base + r16 * lda + kg * KW;
  const T* bp = b_base + r16 * ldb + kg * KW;
  const int kb = (lo / KS) * KS;
  for (int k = kb; k < hi; k += KS)
    acc = Mma<T>::mma(load_k_masked<T>(ap + k, k + kg * KW, lo, hi), Mma<T>::load_k(bp + k), acc);
  return acc;
}

__device__ __forceinline__ int clamp_seq(int s, int nseqs) {
  return s < 0 ? 0 : (s >= nseqs ? nseqs - 1 : s);
}

}  // namespace ssd
