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
// * wave-level reductions in registers (DPP row operations and the gfx950
//   row swaps), each in one fixed order.
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

// round to nearest even (the hardware v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Two floats -> two bf16 (round to nearest even) in one 32-bit word, low
// half first: one v_cvt_pk_bf16_f32 (a 4-wide vector conversion compiles to
// single conversions plus permutes).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float to_f(bf16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ bf16_t from_f(float f) { return f32_to_bf16(f); }
  // exp of the decay factors: the hardware exp2 path (about 1 ulp), ample next
  // to bf16 operands
  static __device__ __forceinline__ float exp(float x) { return __expf(x); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float f) { return f; }
  static __device__ __forceinline__ float exp(float x) { return expf(x); }
};

// gfx950 LDS transpose read (ds_read_b64_tr_b16) of 16-bit elements.  Each
// lane passes the address of 4 consecutive elements (8-byte aligned); within
// every group of 16 lanes, lane i of the group receives element i % 4 of the
// chunks addressed by lanes i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12 of its
// group.  So when lane j of the wave addresses row j / 4, columns
// 4 (j % 4) .. 4 (j % 4) + 3 of a row-major 16 x 16 block, lane i receives
// column i % 16 of rows 4 (i / 16) .. 4 (i / 16) + 3.
__device__ __forceinline__ s16x4_t lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(const_cast<void*>(p)));
}

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
  // Register-direct products: Out += A * X where X is an accumulator tile
  // (k = its row index), with rd-fragments holding 4 k-values per lane:
  //   A: a[r] = A[m = lane % 16][k = 4 * (lane / 16) + r]
  //   X: the tile's own 4 values per lane.
  typedef s16x4_t rfrag;
  static __device__ __forceinline__ rfrag rfrag_from_acc(f32x4_t x) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(rfrag, u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])});
  }
  // 4 values at p, p + stride, p + 2 stride, p + 3 stride
  static __device__ __forceinline__ rfrag rfrag_load(const bf16_t* p, int stride) {
    u16x4_t v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = p[r * stride];
    return __builtin_bit_cast(rfrag, v);
  }
  static __device__ __forceinline__ f32x4_t mma_rd(rfrag a, rfrag x, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, x, c, 0, 0, 0);
  }
  static __device__ __forceinline__ rfrag rfrag_zero() { return rfrag{0, 0, 0, 0}; }
  // rd-fragment of a row-major 16 x 16 block M (LDS, rows = k):
  // lane gets M[4 * (lane / 16) + r][lane % 16], r = 0..3
  static __device__ __forceinline__ rfrag rfrag_load_kn(const bf16_t* blk, int ld) {
    const int l = static_cast<int>(threadIdx.x) & 63;
    return lds_read_tr16(blk + (l >> 2) * ld + 4 * (l & 3));
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
  typedef f32x4_t rfrag;
  static __device__ __forceinline__ rfrag rfrag_from_acc(f32x4_t x) { return x; }
  static __device__ __forceinline__ rfrag rfrag_load(const float* p, int stride) {
    return f32x4_t{p[0], p[stride], p[2 * stride], p[3 * stride]};
  }
  static __device__ __forceinline__ rfrag rfrag_zero() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }
  static __device__ __forceinline__ rfrag rfrag_load_kn(const float* blk, int ld) {
    const int l = static_cast<int>(threadIdx.x) & 63;
    return rfrag_load(blk + 4 * (l >> 4) * ld + (l & 15), ld);
  }
  static __device__ __forceinline__ f32x4_t mma_rd(rfrag a, rfrag x, f32x4_t c) {
#pragma unroll
    for (int r = 0; r < 4; ++r) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], x[r], c, 0, 0, 0);
    return c;
  }
};

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (WAVE - 1); }
__device__ __forceinline__ int wave_id() { return static_cast<int>(threadIdx.x) / WAVE; }
// the same as a scalar (wave-uniform) value: tile indices derived from it
// stay in scalar registers
__device__ __forceinline__ int wave_id_s() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / WAVE);
}

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

// A zero in a vector register: an address offset by it makes the load a
// vector memory load (counted by vmcnt) rather than a scalar one, whose
// completion every later LDS wait would also have to cover.
__device__ __forceinline__ int vgpr_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// A zero the compiler cannot see through.  Adding it to an LDS base pointer
// inside a loop keeps the per-tile addresses derived from that base from
// being hoisted out of the loop and held live (which otherwise costs one
// register per address per tile across the whole loop).
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("; opaque zero" : "=s"(z) : "0"(0));
  return z;
}

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a row (the lanes sharing lane / 16), in registers
// (DPP quad permutes, then row rotations by 4 and 8).  Every lane receives a
// sum of the same 16 values; the association differs between the quads of a
// row, so callers read the result from one fixed lane (lane % 16 == 0).
__device__ __forceinline__ float sum16(float v) {
  v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_move<0x124>(v);  // row_ror:4
  v += dpp_move<0x128>(v);  // row_ror:8
  return v;
}

// Sum over the 4 lanes that share lane % 16 (one per row), with the gfx950
// row swaps; all four lanes receive identical bits.
// v_permlane16_swap / v_permlane32_swap exchange lanes between their two
// register operands (odd rows of the first with even rows of the second, and
// the upper half of the first with the lower half of the second); both
// operands are outputs, so they are issued here with both bound read-write.
// The s_nop padding covers the VALU-write -> permlane-read hazard.
__device__ __forceinline__ void permlane16_swap(unsigned& a, unsigned& b) {
  asm volatile("s_nop 2\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 2" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane32_swap(unsigned& a, unsigned& b) {
  asm volatile("s_nop 2\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 2" : "+v"(a), "+v"(b));
}

// Sum over the 4 lanes that share lane % 16 (one per row); all four lanes
// receive identical bits.
__device__ __forceinline__ float sum_kgroups(float v) {
  unsigned a = __builtin_bit_cast(unsigned, v), b = a;
  permlane16_swap(a, b);   // a = (r0, r0, r2, r2), b = (r1, r1, r3, r3)
  const float y = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
  unsigned c = __builtin_bit_cast(unsigned, y), d = c;
  permlane32_swap(c, d);   // c = (lo, lo), d = (hi, hi)
  return __builtin_bit_cast(float, c) + __builtin_bit_cast(float, d);
}

// The values of the 4 lanes that share lane % 16 (one per row, row = lane /
// 16), gathered into each of those lanes: out[q] = v of row q.
__device__ __forceinline__ void gather_kgroups(float v, float (&out)[4]) {
  unsigned a = __builtin_bit_cast(unsigned, v), b = a;
  permlane16_swap(a, b);   // a = (r0, r0, r2, r2), b = (r1, r1, r3, r3)
  unsigned a0 = a, a2 = a, b1 = b, b3 = b;
  permlane32_swap(a0, a2);  // a0 = r0, a2 = r2 in every row
  permlane32_swap(b1, b3);  // b1 = r1, b3 = r3 in every row
  out[0] = __builtin_bit_cast(float, a0);
  out[1] = __builtin_bit_cast(float, b1);
  out[2] = __builtin_bit_cast(float, a2);
  out[3] = __builtin_bit_cast(float, b3);
}

// Sum over the whole wave; lane 0's result is the one to use.
__device__ __forceinline__ float wave_sum(float v) { return sum_kgroups(sum16(v)); }

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
