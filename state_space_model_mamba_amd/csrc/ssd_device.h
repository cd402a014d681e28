// Device-side building blocks for the SSD backward kernels (gfx950 / CDNA4).
//
// * element conversion (bf16 <-> f32, round to nearest even)
// * 16x16 MFMA tiles with fp32 accumulation: bf16 inputs use
//   v_mfma_f32_16x16x32_bf16 (8 k-values per lane), fp32 inputs use
//   v_mfma_f32_16x16x4_f32 (1 k-value per lane); both accumulate into a
//   16x16 fp32 tile held as 4 values per lane:
//       acc[r] = Out[4 * (lane / 16) + r][lane % 16]
//   A-fragments hold A[m0 + lane % 16][k0 + KW * (lane / 16) + e] and
//   B-fragments hold B[k0 + KW * (lane / 16) + e][n0 + lane % 16].
// * "register-direct" products: an accumulator tile X (rows = k) used as the
//   B operand of a K = 16 contraction, Out[m][n] = sum_k A[m][k] X[k][n],
//   without a round trip through LDS.
// * wave-level scans and reductions in a fixed shuffle order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float to_f(bf16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ bf16_t from_f(float f) { return f32_to_bf16(f); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float f) { return f; }
};

template <typename T> struct Mma;

template <> struct Mma<bf16_t> {
  static constexpr int KW = 8;
  static constexpr int KSTEP = 32;
  typedef bf16x8_t frag;
  // KW consecutive elements (16-byte aligned)
  static __device__ __forceinline__ frag load_k(const bf16_t* p) {
    u16x8_t v = *reinterpret_cast<const u16x8_t*>(p);
    return __builtin_bit_cast(frag, v);
  }
  // KW elements at a stride
  static __device__ __forceinline__ frag load_strided(const bf16_t* p, int stride) {
    u16x8_t v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = p[e * stride];
    return __builtin_bit_cast(frag, v);
  }
  static __device__ __forceinline__ frag zero() { return __builtin_bit_cast(frag, u16x8_t{0, 0, 0, 0, 0, 0, 0, 0}); }
  static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // Out += A * X where X is an accumulator tile (k = its row index) and
  // a[r] = A[m = lane % 16][k = 4 * (lane / 16) + r].
  static __device__ __forceinline__ f32x4_t mma_regdirect(const float a[4], f32x4_t x, f32x4_t c) {
    u16x4_t av, bv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      av[r] = f32_to_bf16(a[r]);
      bv[r] = f32_to_bf16(x[r]);
    }
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, av),
                                                     __builtin_bit_cast(s16x4_t, bv), c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int KW = 1;
  static constexpr int KSTEP = 4;
  typedef float frag;
  static __device__ __forceinline__ frag load_k(const float* p) { return *p; }
  static __device__ __forceinline__ frag load_strided(const float* p, int) { return *p; }
  static __device__ __forceinline__ frag zero() { return 0.f; }
  static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mma_regdirect(const float a[4], f32x4_t x, f32x4_t c) {
#pragma unroll
    for (int r = 0; r < 4; ++r) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], x[r], c, 0, 0, 0);
    return c;
  }
};

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (WAVE - 1); }
__device__ __forceinline__ int wave_id() { return static_cast<int>(threadIdx.x) / WAVE; }

// 16x16 tile product over k in [k_begin, k_end) (multiples of KSTEP):
//   acc += A[m0.., k] * B[k, n0..]
// A is stored K-major: A(m, k) = a_base[m * lda + k]; B is stored K-major:
// B(k, n) = b_base[n * ldb + k].
template <typename T>
__device__ __forceinline__ f32x4_t tile_mma_kk(f32x4_t acc, const T* a_base, int lda,
                                               const T* b_base, int ldb, int k_begin, int k_end) {
  const int l = lane_id();
  const int r16 = l & 15, kg = l >> 4;
  const T* ap = a_base + r16 * lda + kg * Mma<T>::KW;
  const T* bp = b_base + r16 * ldb + kg * Mma<T>::KW;
  for (int k = k_begin; k < k_end; k += Mma<T>::KSTEP)
    acc = Mma<T>::mma(Mma<T>::load_k(ap + k), Mma<T>::load_k(bp + k), acc);
  return acc;
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// A zero the compiler cannot see through.  Adding it to an LDS base pointer
// inside a loop keeps the per-tile addresses derived from that base from
// being hoisted out of the loop and held live (which otherwise costs one
// register per address per tile across the whole loop).
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("; opaque zero" : "=s"(z) : "0"(0));
  return z;
}

// Sum over the 16 lanes that share lane / 16 (fixed butterfly order).
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1, WAVE);
  v += __shfl_xor(v, 2, WAVE);
  v += __shfl_xor(v, 4, WAVE);
  v += __shfl_xor(v, 8, WAVE);
  return v;
}

// Sum over the 4 lanes that share lane % 16 (fixed butterfly order).
__device__ __forceinline__ float sum_kgroups(float v) {
  v += __shfl_xor(v, 16, WAVE);
  v += __shfl_xor(v, 32, WAVE);
  return v;
}

// Sum over the whole wave (fixed butterfly order); every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// Remap a linear block id so that consecutive logical ids run on the same XCD
// (MI355X dispatches block i to XCD i % 8), which lets blocks that read the
// same data share that XCD's L2.  A bijection on [0, total).
__device__ __forceinline__ int64_t xcd_logical_block(int64_t id, int64_t total) {
  constexpr int64_t NXCD = 8;
  const int64_t xcd = id % NXCD, slot = id / NXCD;
  const int64_t q = total / NXCD, r = total % NXCD;
  const int64_t before = xcd * q + (xcd < r ? xcd : r);
  return before + slot;
}

}  // namespace ssd
