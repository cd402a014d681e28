// The intra-chunk dCB of one (batch, group, chunk), the product that the
// chunk_scan_bwd_dC and chunk_state_bwd_db rows of the kernel table on the
// page "Deterministic bwd kernel for mamba2" both need, and the chunk's C B^T
// tiles for the head kernel.  The head sum runs inside one block in ascending
// head order (fp32 accumulators), so there are no per-head slots and no
// atomics.
//
// k_dcb, per (batch, group, chunk):
//   CB  = C B^T over the causal tiles (head independent; fp32, for the head kernel)
//   dCB = sum_h W_h o (dy_h x_h^T),  W_h[i,j] = exp(Acs_i - Acs_j) dt_j  (j <= i, same segment)
//   written as a Q x Q tile and as its transpose (zeros above the diagonal).
#include "ssd_problem.h"
#include "ssd_tiles.h"

namespace ssd {

// ----------------------------------------------------------------------------
// k_dcb
// ----------------------------------------------------------------------------
template <typename T, int Q, int P>
struct DcbCfg {
  static constexpr int T16 = Q / 16;
  static constexpr int W = causal_waves<Q>();   // the head kernel's split (8 waves at Q = 256)
  using Split = CausalSplit<T16, W>;
  static constexpr int NTHR = W * WAVE;
  static constexpr int VEC = Vec16<T>::N;
  static constexpr int LDP = P + VEC;
  static constexpr int NOWN = Split::NOWN;
  static constexpr int NS = sizeof(T) == 2 ? 32 : 16;   // dstate slab of the CB product
  static constexpr int NSL = 4;                         // slabs in flight
  static constexpr int LDN = NS + VEC;
  static_assert(LDN <= LDP, "C/B slabs reuse the x/dy rows' LDS");
  static constexpr int NV = Q * P / VEC;                 // vectors of x (or dy) per head
  static constexpr int NVT = (NV + NTHR - 1) / NTHR;     // per thread
  static constexpr size_t LDS = size_t(2) * Q * LDP * sizeof(T) + size_t(4) * Q * 4;
};

// One head's contribution to the owned dCB tiles: dcb[k] += W o (dy x^T) on
// tile k.  UNI: the chunk has a single segment (the off-diagonal decays are
// factored through the per-row table er); the two versions keep the unrolled
// tile sequence free of branches.
template <typename T, int Q, int P, bool UNI, int NOWN>
__device__ __forceinline__ void dcb_tiles(f32x4_t (&dcb)[NOWN], const T* xk, const T* dyk,
                                          const float* acs, const float* dtv, const float* erv, const int* lov,
                                          int wz) {
  using Cf = DcbCfg<T, Q, P>;
  constexpr int LDP = Cf::LDP;
  const int l = lane_id(), r16 = l & 15, kg = l >> 4;
#pragma clang loop unroll(full)
  for (int k = 0; k < Cf::NOWN; ++k) {
    int I, J;
    bool second;
    Cf::Split::tile(wz, k, I, J, second);
    const f32x4_t m = tile_mma_kk<T>(zero4(), dyk + 16 * I * LDP, LDP, xk + 16 * J * LDP, LDP, 0, P);
    const int j = 16 * J + r16;
    const float aj = acs[j], dtj = dtv[j];
    f32x4_t e4;   // exp(Acs_i - Acs_j) where (i, j) is causal and in one segment, else 0
    if (UNI && k < Cf::Split::NOFF) {
      const float ec = Elem<T>::exp(acs[16 * I] - aj);
      const f32x4_t er = *reinterpret_cast<const f32x4_t*>(erv + 16 * I + 4 * kg);
#pragma unroll
      for (int r = 0; r < 4; ++r) e4[r] = er[r] * ec;
    } else {
      const int loj = lov[j];
      const f32x4_t acs4 = *reinterpret_cast<const f32x4_t*>(acs + 16 * I + 4 * kg);
      const int4 lo4 = *reinterpret_cast<const int4*>(lov + 16 * I + 4 * kg);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * kg + r;
        const int loi = r == 0 ? lo4.x : (r == 1 ? lo4.y : (r == 2 ? lo4.z : lo4.w));
        const bool ok = (j <= i) & (loi == loj);
        // exp of a non-positive argument only; masked entries use a zero argument
        const float e = Elem<T>::exp(ok ? acs4[r] - aj : 0.f);
        e4[r] = ok ? e : 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) dcb[k][r] += (e4[r] * dtj) * m[r];
    // keep the scheduler from hoisting every tile's fragment loads at once
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <typename T, int Q, int P>
__global__ __launch_bounds__((DcbCfg<T, Q, P>::NTHR)) void k_dcb(Problem pb) {
  using Cf = DcbCfg<T, Q, P>;
  constexpr int T16 = Cf::T16, NTHR = Cf::NTHR, VEC = Cf::VEC, LDP = Cf::LDP;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* s_xk = reinterpret_cast<T*>(smem);
  T* s_dyk = s_xk + Q * LDP;
  float* s_acs = reinterpret_cast<float*>(s_dyk + Q * LDP);
  float* s_dt = s_acs + Q;
  float* s_er = s_dt + Q;
  int* s_lo = reinterpret_cast<int*>(s_er + Q);

  const int64_t total = static_cast<int64_t>(pb.B) * pb.G * pb.nc;
  const int64_t lb = xcd_logical_block(blockIdx.x, total);
  const int c = static_cast<int>(lb % pb.nc);
  const int64_t bg = lb / pb.nc;
  const int g = static_cast<int>(bg % pb.G), b = static_cast<int>(bg / pb.G);
  const int tid = threadIdx.x, w = wave_id_s(), l = lane_id(), r16 = l & 15, kg = l >> 4;
  const int64_t bc = static_cast<int64_t>(b) * pb.nc + c;
  const T* xg = static_cast<const T*>(pb.x);
  const T* dyg = static_cast<const T*>(pb.dy);

  const int64_t bgc = (static_cast<int64_t>(b) * pb.G + g) * pb.nc + c;
  for (int i = tid; i < Q; i += NTHR) s_lo[i] = seg_lo(pb.segpos[bc * Q + i]);

  // ---- CB = C B^T over the owned causal tiles.  It is the same for every
  // head of the group, so it is formed once here and stored for the head
  // kernel in fp32, in that kernel's (wave, tile) order and lane layout.
  {
    constexpr int NS = Cf::NS, NSL = Cf::NSL, LDN = Cf::LDN;
    T* s_ck = s_xk;   // the x / dy rows are not staged yet
    T* s_bk = s_ck + Q * LDN;
    const T* Bg = static_cast<const T*>(pb.Bm);
    const T* Cg = static_cast<const T*>(pb.Cm);
    auto bc_row = [&](const T* base, int n0) {
      return [=](int i) -> const T* {
        const int t = c * Q + i;
        return t < pb.L ? base + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + n0 : nullptr;
      };
    };
    RowStage<T, Q, NS, NTHR> st_c[NSL], st_b[NSL];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      if (sl * NS < pb.N) {
        st_c[sl].load(bc_row(Cg, sl * NS));
        st_b[sl].load(bc_row(Bg, sl * NS));
      }
    }
    f32x4_t cbt[Cf::NOWN];
#pragma unroll
    for (int k = 0; k < Cf::NOWN; ++k) cbt[k] = zero4();
    for (int nb = 0; nb < pb.N; nb += NSL * NS) {
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) {
        const int n0 = nb + sl * NS;
        if (n0 < pb.N) {
          __syncthreads();
          st_c[sl].store(s_ck, LDN);
          st_b[sl].store(s_bk, LDN);
          __syncthreads();
          if (n0 + NSL * NS < pb.N) {
            st_c[sl].load(bc_row(Cg, n0 + NSL * NS));
            st_b[sl].load(bc_row(Bg, n0 + NSL * NS));
          }
          const int z = opaque_zero();
          const int wz = w + z;
#pragma clang loop unroll(full)
          for (int k = 0; k < Cf::NOWN; ++k) {
            int I, J;
            bool second;
            Cf::Split::tile(wz, k, I, J, second);
            cbt[k] = tile_mma_kk<T>(cbt[k], s_ck + z + 16 * I * LDN, LDN, s_bk + z + 16 * J * LDN, LDN, 0, NS);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    float* dst = pb.cbt + (bgc * Cf::W + w) * Cf::NOWN * 256 + l * 4;
#pragma unroll
    for (int k = 0; k < Cf::NOWN; ++k) *reinterpret_cast<f32x4_t*>(dst + k * 256) = cbt[k];
  }

  f32x4_t dcb[Cf::NOWN];
#pragma unroll
  for (int k = 0; k < Cf::NOWN; ++k) dcb[k] = zero4();

  auto head_row = [&](const T* base, int h) {
    return [=](int i) -> const T* {
      const int t = c * Q + i;
      return t < pb.L ? base + ((static_cast<int64_t>(b) * pb.L + t) * pb.H + h) * P : nullptr;
    };
  };
  // each head's x / dy rows and Acs / dt are loaded into registers while the
  // previous head's tiles are multiplied
  static_assert(NTHR >= Q, "one thread per chunk position");
  RowStage<T, Q, P, NTHR> st_x, st_dy;
  float acs_n = 0.f, dt_n = 0.f;
  auto load_head = [&](int hh) {
    const int h = g * pb.hpg + hh;
    const int64_t bhc = (static_cast<int64_t>(b) * pb.H + h) * pb.nc + c;
    st_x.load(head_row(xg, h));
    st_dy.load(head_row(dyg, h));
    if (tid < Q) {
      acs_n = pb.acs[bhc * Q + tid];
      dt_n = pb.dtc[bhc * Q + tid];
    }
  };
  // A chunk without sequence starts after position 0 has one segment and a
  // non-increasing Acs: there the decay of an off-diagonal tile is
  // er_i * exp(Acs_{16I} - Acs_j) with er_i = exp(Acs_i - Acs_{16 floor(i/16)}),
  // both factors <= 1.
  const bool uniform = __builtin_amdgcn_readfirstlane(seg_lo(pb.segpos[bc * Q + Q - 1])) == 0;
  __syncthreads();   // (keeps the first head's loads out of the CB phase's registers)
  load_head(0);

  for (int hh = 0; hh < pb.hpg; ++hh) {
    __syncthreads();
    st_x.store(s_xk, LDP);
    st_dy.store(s_dyk, LDP);
    {
      const float acs_tile0 = __shfl(acs_n, l & ~15, WAVE);
      if (tid < Q) {
        s_acs[tid] = acs_n;
        s_dt[tid] = dt_n;
        s_er[tid] = uniform ? Elem<T>::exp(acs_n - acs_tile0) : 0.f;
      }
    }
    __syncthreads();
    if (hh + 1 < pb.hpg) load_head(hh + 1);

    const int z = opaque_zero();
    const int wz = w + z;
    const T* xk = s_xk + z;
    const T* dyk = s_dyk + z;
    const float* acs = s_acs + z;
    const float* dtv = s_dt + z;
    const float* erv = s_er + z;
    const int* lov = s_lo + z;
    if (uniform)
      dcb_tiles<T, Q, P, true, Cf::NOWN>(dcb, xk, dyk, acs, dtv, erv, lov, wz);
    else
      dcb_tiles<T, Q, P, false, Cf::NOWN>(dcb, xk, dyk, acs, dtv, erv, lov, wz);
  }

  // write dCB (row-major) and dCB^T, the owned columns in full (zeros above the diagonal)
  T* dcb_out = static_cast<T*>(pb.dcb) + bgc * Q * Q;
  T* dcbt_out = static_cast<T*>(pb.dcbt) + bgc * Q * Q;
#pragma clang loop unroll(full)
  for (int k = 0; k < Cf::NOWN; ++k) {
    int I, J;
    bool second;
    Cf::Split::tile(w, k, I, J, second);
    const int j = 16 * J + r16;
    T tv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      tv[r] = Elem<T>::from_f(dcb[k][r]);
      dcb_out[static_cast<int64_t>(16 * I + 4 * kg + r) * Q + j] = tv[r];
      dcbt_out[static_cast<int64_t>(j) * Q + 16 * I + 4 * kg + r] = tv[r];
    }
  }
  // zeros above the diagonal of the owned columns
  for (int a = 0; a < Cf::Split::NCOL; ++a) {
    const int J = Cf::Split::col(w, a);
    const int j = 16 * J + r16;
    for (int I = 0; I < J; ++I)
      for (int r = 0; r < 4; ++r) {
        dcb_out[static_cast<int64_t>(16 * I + 4 * kg + r) * Q + j] = Elem<T>::from_f(0.f);
        dcbt_out[static_cast<int64_t>(j) * Q + 16 * I + 4 * kg + r] = Elem<T>::from_f(0.f);
      }
  }
}

template <typename K>
static hipError_t allow_lds(K kernel, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(bytes));
}

template <typename T, int Q, int P>
static hipError_t launch_dcb_t(const Problem& pb, hipStream_t s) {
  using C1 = DcbCfg<T, Q, P>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = allow_lds(&k_dcb<T, Q, P>, C1::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t b1 = static_cast<int64_t>(pb.B) * pb.G * pb.nc;
  hipLaunchKernelGGL((k_dcb<T, Q, P>), dim3(static_cast<unsigned>(b1)), dim3(C1::NTHR), C1::LDS, s, pb);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_dcb_any(const Problem& pb, hipStream_t s) {
#define SSD_DCB_CASE(QQ, PP) \
  if (pb.Q == QQ && pb.P == PP) return launch_dcb_t<T, QQ, PP>(pb, s);
  if constexpr (sizeof(T) == 2) {
    SSD_BF16_SHAPES(SSD_DCB_CASE)
  } else {
    SSD_F32_SHAPES(SSD_DCB_CASE)
  }
#undef SSD_DCB_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_dcb(const Problem& pb, bool io_bf16, hipStream_t s) {
  return io_bf16 ? launch_dcb_any<bf16_t>(pb, s) : launch_dcb_any<float>(pb, s);
}

// LDS bytes of k_dcb for a compiled shape; ~0 when not compiled.
size_t dcb_lds_bytes(int Q, int P, bool bf16) {
#define SSD_DCB_LDS_B(QQ, PP) \
  if (bf16 && Q == QQ && P == PP) return DcbCfg<bf16_t, QQ, PP>::LDS;
#define SSD_DCB_LDS_F(QQ, PP) \
  if (!bf16 && Q == QQ && P == PP) return DcbCfg<float, QQ, PP>::LDS;
  SSD_BF16_SHAPES(SSD_DCB_LDS_B)
  SSD_F32_SHAPES(SSD_DCB_LDS_F)
#undef SSD_DCB_LDS_B
#undef SSD_DCB_LDS_F
  return ~size_t(0);
}

}  // namespace ssd
