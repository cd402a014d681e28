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

// 16-byte load at a 32-bit byte offset from a wave-uniform base: the 64-bit
// base stays in scalar registers and the offset in one vector register (the
// scalar-base form of the global load), so no 64-bit address arithmetic runs
// per lane.
__device__ __forceinline__ uint4 ld_global16_at(const void* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(static_cast<const char*>(base) + off);
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

// 4 consecutive elements (8-byte aligned for bf16, 16-byte for fp32) as floats,
// and the reverse with round-to-nearest-even
template <typename T> __device__ __forceinline__ f32x4_t load4f(const T* p);
template <> __device__ __forceinline__ f32x4_t load4f<bf16_t>(const bf16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return f32x4_t{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                 __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
}
template <> __device__ __forceinline__ f32x4_t load4f<float>(const float* p) {
  return *reinterpret_cast<const f32x4_t*>(p);
}
template <typename T> __device__ __forceinline__ void store4f(T* p, f32x4_t v);
template <> __device__ __forceinline__ void store4f<bf16_t>(bf16_t* p, f32x4_t v) {
  *reinterpret_cast<uint2*>(p) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
template <> __device__ __forceinline__ void store4f<float>(float* p, f32x4_t v) {
  *reinterpret_cast<f32x4_t*>(p) = v;
}

// ---------------------------------------------------------------------------
// Block-wide staging of a ROWS x COLS tile from global memory (rows given by
// a functor returning the row's first element, or nullptr for a zero row)
// into LDS.  All of a thread's 16-byte loads are issued before any LDS store,
// so a stage costs one memory latency instead of one per loop trip.
// ---------------------------------------------------------------------------
template <typename TIN, int ROWS, int COLS, int NTHR>
struct RowStage {
  static constexpr int VEC = Vec16<TIN>::N;
  static constexpr int CV = COLS / VEC;                 // vectors per row
  static constexpr int NV = ROWS * CV;
  static constexpr int IT = (NV + NTHR - 1) / NTHR;     // vectors per thread
  static_assert(COLS % VEC == 0, "row length must be a multiple of 16 bytes");
  uint4 buf[IT];

  template <typename RowPtr>
  __device__ __forceinline__ void load(RowPtr rowptr) {
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int v = static_cast<int>(threadIdx.x) + k * NTHR;
      buf[k] = zero_u4();
      if (NV % NTHR == 0 || v < NV) {
        const TIN* p = rowptr(v / CV);
        if (p) buf[k] = ld_global16(p + (v % CV) * VEC);
      }
    }
  }
  // Requests at fixed per-lane byte offsets from a wave-uniform base, for
  // rows at a fixed byte pitch from it (one head's rows after another's:
  // only the base moves, so a request takes no 64-bit address arithmetic per
  // lane).  Rows at or past nrows are not read (their pieces are zero).
  struct Offs {
    uint32_t off[IT];
    uint32_t ok;   // bit k: piece k is read
  };
  static __device__ __forceinline__ Offs offsets(uint32_t row_bytes, int nrows) {
    Offs o;
    o.ok = 0;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int v = static_cast<int>(threadIdx.x) + k * NTHR;
      const int r = v / CV;
      o.off[k] = static_cast<uint32_t>(r) * row_bytes + static_cast<uint32_t>((v % CV) * 16);
      if ((NV % NTHR == 0 || v < NV) && r < nrows) o.ok |= 1u << k;
    }
    return o;
  }
  __device__ __forceinline__ void load_at(const TIN* base, const Offs& o) {
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      buf[k] = zero_u4();
      if ((o.ok >> k) & 1u) buf[k] = ld_global16_at(base, o.off[k]);
    }
  }
  // The same with the row count given per request (offsets taken for all
  // ROWS rows): rows at or past nrows are not read.
  __device__ __forceinline__ void load_at(const TIN* base, const Offs& o, int nrows) {
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int v = static_cast<int>(threadIdx.x) + k * NTHR;
      buf[k] = zero_u4();
      if ((o.ok >> k) & 1u && v / CV < nrows) buf[k] = ld_global16_at(base, o.off[k]);
    }
  }
  // fp32 rows requested now (16-byte loads, F4 per piece of TIN) and rounded
  // to TIN later by convert_f32, so that the requests stay in flight meanwhile
  static constexpr int F4 = VEC / 4;
  template <typename RowPtr>
  __device__ __forceinline__ void load_f32_raw(RowPtr rowptr, uint4 (&raw)[IT][F4]) const {
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int v = static_cast<int>(threadIdx.x) + k * NTHR;
#pragma unroll
      for (int f = 0; f < F4; ++f) raw[k][f] = zero_u4();
      if (NV % NTHR == 0 || v < NV) {
        const float* p = rowptr(v / CV);
        if (p) {
#pragma unroll
          for (int f = 0; f < F4; ++f) raw[k][f] = ld_global16(p + (v % CV) * VEC + 4 * f);
        }
      }
    }
  }
  __device__ __forceinline__ void convert_f32(const uint4 (&raw)[IT][F4]) {
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      TIN o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] = Elem<TIN>::from_f(__uint_as_float((&raw[k][e / 4].x)[e % 4]));
      buf[k] = *reinterpret_cast<const uint4*>(o);
    }
  }
  // The same rows read from fp32 memory and rounded to TIN (to nearest even):
  // each 16-byte piece takes 16 / sizeof(TIN) floats.  The conversion waits
  // for the loads, so this is for rarely taken paths.
  template <typename RowPtr>
  __device__ __forceinline__ void load_from_f32(RowPtr rowptr) {
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int v = static_cast<int>(threadIdx.x) + k * NTHR;
      buf[k] = zero_u4();
      if (NV % NTHR == 0 || v < NV) {
        const float* p = rowptr(v / CV);
        if (p) {
          TIN o[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) o[e] = Elem<TIN>::from_f(p[(v % CV) * VEC + e]);
          buf[k] = *reinterpret_cast<const uint4*>(o);
        }
      }
    }
  }
  // row-major into LDS (same element type): lds[r * ld + c]
  __device__ __forceinline__ void store(TIN* lds, int ld) const {
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int v = static_cast<int>(threadIdx.x) + k * NTHR;
      if (NV % NTHR == 0 || v < NV) *reinterpret_cast<uint4*>(lds + (v / CV) * ld + (v % CV) * VEC) = buf[k];
    }
  }
  // row-major with conversion: lds[r * ld + c] = TOUT(x)
  template <typename TOUT>
  __device__ __forceinline__ void store_convert(TOUT* lds, int ld) const {
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int v = static_cast<int>(threadIdx.x) + k * NTHR;
      if (NV % NTHR == 0 || v < NV) {
        const int r = v / CV, c0 = (v % CV) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) lds[r * ld + c0 + e] = Elem<TOUT>::from_f(vget<TIN>(buf[k], e));
      }
    }
  }
  // row-major with conversion from fp32, 4 elements per store:
  // lds[r * ld + c] = TOUT(x)  (ld and the row starts keep 4-element groups
  // 8-byte aligned for bf16 and 16-byte aligned for fp32)
  template <typename TOUT>
  __device__ __forceinline__ void store_rows_f32(TOUT* lds, int ld) const {
    static_assert(sizeof(TIN) == 4 && VEC == 4, "fp32 rows");
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int v = static_cast<int>(threadIdx.x) + k * NTHR;
      if (NV % NTHR == 0 || v < NV) {
        const f32x4_t f = __builtin_bit_cast(f32x4_t, buf[k]);
        store4f<TOUT>(lds + (v / CV) * ld + (v % CV) * VEC, f);
      }
    }
  }
  // transposed with conversion: lds[c * ld + r] = TOUT(x)
  template <typename TOUT>
  __device__ __forceinline__ void store_transposed(TOUT* lds, int ld) const {
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int v = static_cast<int>(threadIdx.x) + k * NTHR;
      if (NV % NTHR == 0 || v < NV) {
        const int r = v / CV, c0 = (v % CV) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) lds[(c0 + e) * ld + r] = Elem<TOUT>::from_f(vget<TIN>(buf[k], e));
      }
    }
  }
};

// MFMA fragments of an operand stored with k as the row index ("kn" layout:
// X[k][m], m contiguous; X points at column m0), k in [k0, k0 + KSTEP):
//   bf16: lane (kg, r16) gets X[k0 + 8 kg + e][r16], e = 0..7, with two LDS
//         transpose reads (lane j of each 16-lane group addresses row
//         k0 + 8 kg + j / 4 (+ 4), columns 4 (j % 4) .. + 3)
//   fp32: lane (kg, r16) gets X[k0 + kg][r16]
// ld must keep rows 8-byte aligned (a multiple of 4 elements).
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag load_kn(const T* X, int ld, int k0);
template <>
__device__ __forceinline__ Mma<bf16_t>::frag load_kn<bf16_t>(const bf16_t* X, int ld, int k0) {
  const int l = lane_id();
  const bf16_t* p = X + (k0 + 8 * (l >> 4) + ((l & 15) >> 2)) * ld + 4 * (l & 3);
  const s16x4_t lo = lds_read_tr16(p);
  const s16x4_t hi = lds_read_tr16(p + 4 * ld);
  return __builtin_bit_cast(Mma<bf16_t>::frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
template <>
__device__ __forceinline__ float load_kn<float>(const float* X, int ld, int k0) {
  const int l = lane_id();
  return X[(k0 + (l >> 4)) * ld + (l & 15)];
}

// 16x16 tile product with both operands in the kn layout:
//   acc[m][n] += sum_k A[k][m] B[k][n],  k in [k_begin, k_end) (multiples of KSTEP)
template <typename T>
__device__ __forceinline__ f32x4_t tile_mma_kn(f32x4_t acc, const T* a, int lda, const T* b, int ldb,
                                               int k_begin, int k_end) {
  for (int k = k_begin; k < k_end; k += Mma<T>::KSTEP)
    acc = Mma<T>::mma(load_kn<T>(a, lda, k), load_kn<T>(b, ldb, k), acc);
  return acc;
}

// 16x16 tile product with A stored K-major (A(m, k) = a_base[m * lda + k])
// and B in the kn layout (B(k, n) = b[k * ldb + n]).
template <typename T>
__device__ __forceinline__ f32x4_t tile_mma_kk_kn(f32x4_t acc, const T* a_base, int lda, const T* b, int ldb,
                                                  int k_begin, int k_end) {
  const int l = lane_id();
  const T* ap = a_base + (l & 15) * lda + (l >> 4) * Mma<T>::KW;
  for (int k = k_begin; k < k_end; k += Mma<T>::KSTEP)
    acc = Mma<T>::mma(Mma<T>::load_k(ap + k), load_kn<T>(b, ldb, k), acc);
  return acc;
}

// Like tile_mma_kn, but only k in [lo, hi) contributes (A elements outside
// read as zero).
template <typename T>
__device__ __forceinline__ f32x4_t tile_mma_kn_range(f32x4_t acc, const T* a, int lda, const T* b, int ldb,
                                                     int lo, int hi) {
  constexpr int KS = Mma<T>::KSTEP, KW = Mma<T>::KW;
  const int kg = lane_id() >> 4;
  for (int k = (lo / KS) * KS; k < hi; k += KS) {
    typename Mma<T>::frag fa = load_kn<T>(a, lda, k);
    if constexpr (KW == 1) {
      if (k + kg < lo || k + kg >= hi) fa = 0.f;
    } else {
      u16x8_t v = __builtin_bit_cast(u16x8_t, fa);
#pragma unroll
      for (int e = 0; e < KW; ++e)
        if (k + KW * kg + e < lo || k + KW * kg + e >= hi) v[e] = 0;
      fa = __builtin_bit_cast(typename Mma<T>::frag, v);
    }
    acc = Mma<T>::mma(fa, load_kn<T>(b, ldb, k), acc);
  }
  return acc;
}

// Row pitch (elements) of a row-major LDS tile of `cols` 16-bit columns read
// with load_kn: rows land 32 or 96 bytes apart modulo 128, so the four rows
// of a transpose read hit distinct banks.  Four-byte elements get 16 bytes.
template <typename T>
constexpr int kn_pitch(int cols) {
  return sizeof(T) == 2 ? ((cols * 2) % 128 == 32 || (cols * 2) % 128 == 96 ? cols : cols + 16) : cols + 4;
}

// A row-major LDS tile of COLS columns read with the transpose reads.
// 128-byte rows of 16-bit elements are stored unpadded, their 32-byte
// segments XOR-swizzled by (row mod 4): the four rows of one transpose read
// then cover all banks once.  Other widths are padded (kn_pitch).
template <typename T, int COLS>
struct KnTile {
  static constexpr bool SWZ = sizeof(T) == 2 && COLS * 2 == 128;
  static constexpr int LD = SWZ ? COLS : kn_pitch<T>(COLS);
  // element offset of (row, col); 8 consecutive columns from a multiple of 8
  // stay contiguous
  static __device__ __forceinline__ int at(int row, int col) {
    if constexpr (SWZ)
      return row * LD + ((((col >> 4) ^ (row & 3))) << 4) + (col & 15);
    else
      return row * LD + col;
  }
  // MFMA fragment of the 16 columns from m0 (a multiple of 16), k rows from k0
  // (the load_kn layout)
  static __device__ __forceinline__ typename Mma<T>::frag frag(const T* base, int m0, int k0) {
    const int l = lane_id();
    if constexpr (sizeof(T) == 2) {
      const int row = k0 + 8 * (l >> 4) + ((l & 15) >> 2);
      const int col = m0 + 4 * (l & 3);
      const s16x4_t lo = lds_read_tr16(base + at(row, col));
      const s16x4_t hi = lds_read_tr16(base + at(row + 4, col));
      return __builtin_bit_cast(typename Mma<T>::frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      return base[at(k0 + (l >> 4), m0 + (l & 15))];
    }
  }
};

// A fragment (k values k0 + KW (lane / 16) + e) with the k values outside
// [lo, hi) zeroed.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag mask_k(typename Mma<T>::frag f, int k0, int lo, int hi) {
  constexpr int KW = Mma<T>::KW;
  const int kg = lane_id() >> 4;
  if constexpr (KW == 1) {
    return (k0 + kg < lo || k0 + kg >= hi) ? 0.f : f;
  } else {
    u16x8_t v = __builtin_bit_cast(u16x8_t, f);
#pragma unroll
    for (int e = 0; e < KW; ++e)
      if (k0 + KW * kg + e < lo || k0 + KW * kg + e >= hi) v[e] = 0;
    return __builtin_bit_cast(typename Mma<T>::frag, v);
  }
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

// The causal 16x16 tiles (I >= J) of a Q x Q matrix, T = Q/16 tiles per side,
// split over W = T/2 waves: wave p owns the column pair {p, T-1-p} (T+1 causal
// tiles, so every wave costs the same).  Its tiles k = 0 .. T are ordered
//   k <  T-1-p : column p,      row tiles T-1 down to p+1
//   k <  T-1   : column T-1-p,  row tiles T-1 down to T-p
//   k == T-1   : diagonal tile (p, p)
//   k == T     : diagonal tile (T-1-p, T-1-p)
// so the off-diagonal tiles are exactly k < T-1 (known once unrolled), and
// each column is walked bottom-up with its diagonal tile after the rest.
// `second` tells which column of the pair (slot 0 or 1) a tile belongs to.
template <int T16, int W>
struct CausalSplit {
  static_assert(T16 % 2 == 0 && T16 / 2 == W, "one column pair per wave");
  static constexpr int NOWN = T16 + 1;   // causal tiles per wave
  static constexpr int NCOL = 2;         // owned column tiles per wave
  static constexpr int NOFF = T16 - 1;   // off-diagonal tiles per wave
  // column tile of owned slot a
  static __device__ __forceinline__ int col(int w, int a) { return a ? T16 - 1 - w : w; }
  static __device__ __forceinline__ void tile(int w, int k, int& I, int& J, bool& second) {
    const int p = w;
    if (k == T16 - 1) {
      I = J = p;
      second = false;
    } else if (k == T16) {
      I = J = T16 - 1 - p;
      second = true;
    } else if (k < T16 - 1 - p) {
      J = p;
      I = T16 - 1 - k;
      second = false;
    } else {
      J = T16 - 1 - p;
      I = T16 - 1 - (k - (T16 - 1 - p));
      second = true;
    }
  }
};

// Waves of the blocks that own the causal tiles of a Q x Q chunk product:
// one column pair {p, T-1-p} per wave (8 waves, two per SIMD, at Q = 256).
// The dCB/CB kernel and the head kernel use the same split, so a wave of one
// owns exactly the tiles of the same wave of the other.
template <int Q>
constexpr int causal_waves() {
  return Q / 32;
}

__device__ __forceinline__ int clamp_seq(int s, int nseqs) {
  return s < 0 ? 0 : (s >= nseqs ? nseqs - 1 : s);
}

}  // namespace ssd
