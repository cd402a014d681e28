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
// On a grid too small for the GPU the group's heads are cut into nslice
// slices of consecutive heads, one block each: every block sums its slice in
// ascending head order into fp32 tiles parked in a workspace slot, and
// k_dcb_out adds the slots in slice order and writes the two tiles.
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
  // dCB output staging: RB rows of LDR elements in the x / dy rows' LDS
  static constexpr int LDR = Q + VEC;
  static constexpr int RB_FIT = (2 * Q * LDP / LDR) / 16 * 16;
  static constexpr int RB = RB_FIT >= Q ? Q : (RB_FIT >= 128 ? 128 : (RB_FIT >= 64 ? 64 : (RB_FIT >= 32 ? 32 : 16)));
  static_assert(RB >= 16 && Q % RB == 0 && size_t(RB) * LDR <= size_t(2) * Q * LDP, "dCB staging rows");
};

// Row operands of one causal tile of one head, requested one tile ahead so
// that their latency hides behind the previous tile's arithmetic.
template <typename T, int P>
struct DcbTileIn {
  static constexpr int MK = P / Mma<T>::KSTEP;   // k-steps of dy x^T
  typename Mma<T>::frag ma[MK];                   // dy rows of tile I
  f32x4_t rowv;   // UNI off-diagonal: er of rows I; otherwise Acs of rows I
  int4 lo4;       // segment starts of rows I (not UNI off-diagonal)
  float acs_i0;   // Acs at row 16 I (UNI off-diagonal)
};

template <typename T, int Q, int P, bool UNI, bool DIAG>
__device__ __forceinline__ void dcb_tile_load(DcbTileIn<T, P>& in, int I, const T* dyk, const float* acs,
                                              const float* erv, const int* lov) {
  constexpr int LDP = DcbCfg<T, Q, P>::LDP, KW = Mma<T>::KW, KS = Mma<T>::KSTEP;
  const int l = lane_id(), r16 = l & 15, kg = l >> 4;
  const T* ap = dyk + (16 * I + r16) * LDP + kg * KW;
#pragma unroll
  for (int s = 0; s < DcbTileIn<T, P>::MK; ++s) in.ma[s] = Mma<T>::load_k(ap + s * KS);
  if constexpr (UNI && !DIAG) {
    in.acs_i0 = acs[16 * I];
    in.rowv = *reinterpret_cast<const f32x4_t*>(erv + 16 * I + 4 * kg);
  } else {
    in.rowv = *reinterpret_cast<const f32x4_t*>(acs + 16 * I + 4 * kg);
    in.lo4 = *reinterpret_cast<const int4*>(lov + 16 * I + 4 * kg);
  }
}

// Column operands of the column tile being walked: the x rows (B operand of
// dy x^T) and this lane's column's Acs, dt and segment start.
template <typename T, int P>
struct DcbColumn {
  typename Mma<T>::frag mb[P / Mma<T>::KSTEP];
  float aj, dtj;
  int loj;
};

template <typename T, int Q, int P>
__device__ __forceinline__ void dcb_column_load(DcbColumn<T, P>& cl, int J, const T* xk, const float* acs,
                                                const float* dtv, const int* lov) {
  constexpr int LDP = DcbCfg<T, Q, P>::LDP, KW = Mma<T>::KW, KS = Mma<T>::KSTEP;
  const int l = lane_id(), r16 = l & 15, kg = l >> 4;
  const T* bp = xk + (16 * J + r16) * LDP + kg * KW;
#pragma unroll
  for (int s = 0; s < P / KS; ++s) cl.mb[s] = Mma<T>::load_k(bp + s * KS);
  const int j = 16 * J + r16;
  cl.aj = acs[j];
  cl.dtj = dtv[j];
  cl.loj = lov[j];
}

// One head's contribution to the owned dCB tiles: dcb[k] += W o (dy x^T) on
// tile k.  UNI: the chunk has a single segment (the off-diagonal decays are
// factored through the per-row table er); the two versions keep the unrolled
// tile sequence free of branches on it.  The wave walks its first column's
// off-diagonal tiles, then its second column's, then the two diagonal tiles;
// the column operands are reloaded where the column changes (a wave-uniform
// branch at a wave-dependent tile, taken once).
template <typename T, int Q, int P, bool UNI, int NOWN>
__device__ __forceinline__ void dcb_tiles(f32x4_t (&dcb)[NOWN], const T* xk, const T* dyk,
                                          const float* acs, const float* dtv, const float* erv, const int* lov,
                                          int wz) {
  using Cf = DcbCfg<T, Q, P>;
  using Split = typename Cf::Split;
  using In = DcbTileIn<T, P>;
  const int l = lane_id(), r16 = l & 15, kg = l >> 4;
  const int n0 = Cf::T16 - 1 - wz;   // off-diagonal tiles of the first column
  In cur;
  DcbColumn<T, P> col;
  {
    int I, J;
    bool second;
    Split::tile(wz, 0, I, J, second);
    dcb_tile_load<T, Q, P, UNI, Split::NOFF == 0>(cur, I, dyk, acs, erv, lov);
    dcb_column_load<T, Q, P>(col, J, xk, acs, dtv, lov);
  }
#pragma clang loop unroll(full)
  for (int k = 0; k < Cf::NOWN; ++k) {
    int I, J;
    bool second;
    Split::tile(wz, k, I, J, second);
    In nxt;
    if (k + 1 < Cf::NOWN) {
      int In_, Jn;
      bool sn;
      Split::tile(wz, k + 1, In_, Jn, sn);
      if (k + 1 >= Split::NOFF)
        dcb_tile_load<T, Q, P, UNI, true>(nxt, In_, dyk, acs, erv, lov);
      else
        dcb_tile_load<T, Q, P, UNI, false>(nxt, In_, dyk, acs, erv, lov);
    }
    f32x4_t m = zero4();
#pragma unroll
    for (int s = 0; s < In::MK; ++s) m = Mma<T>::mma(cur.ma[s], col.mb[s], m);
    const int j = 16 * J + r16;
    const float aj = col.aj, dtj = col.dtj;
    f32x4_t e4;   // exp(Acs_i - Acs_j) dt_j where (i, j) is causal and in one segment, else 0
    if (UNI && k < Split::NOFF) {
      const float ec = Elem<T>::exp(cur.acs_i0 - aj) * dtj;
#pragma unroll
      for (int r = 0; r < 4; ++r) e4[r] = cur.rowv[r] * ec;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * kg + r;
        const int loi = r == 0 ? cur.lo4.x : (r == 1 ? cur.lo4.y : (r == 2 ? cur.lo4.z : cur.lo4.w));
        const bool ok = (j <= i) & (loi == col.loj);
        // exp of a non-positive argument only; masked entries use a zero argument
        const float e = Elem<T>::exp(ok ? cur.rowv[r] - aj : 0.f);
        e4[r] = ok ? e * dtj : 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) dcb[k][r] += e4[r] * m[r];
    // the tile's sums are complete here: keeps them from being sunk past the
    // column branches below (which would hold every tile's products live)
    asm volatile("" : "+v"(dcb[k]));
    if (k + 1 < Cf::NOWN) {
      cur = nxt;
      // column of tile k + 1
      if (k + 1 >= Split::NOFF) {
        dcb_column_load<T, Q, P>(col, k + 1 == Split::NOFF ? wz : Cf::T16 - 1 - wz, xk, acs, dtv, lov);
      } else if (k >= Cf::T16 / 2 - 1 && k + 1 == n0) {
        dcb_column_load<T, Q, P>(col, Cf::T16 - 1 - wz, xk, acs, dtv, lov);
      }
    }
  }
}

// dCB of one (batch, group, chunk) (the wave's causal tiles, fp32) -> dcb
// (row-major) and dcbt (its transpose), in full (zeros above the diagonal),
// RB rows at a time through the block's LDS (the x / dy rows' region): the
// block is cleared, each wave writes its tiles into it, and the rows leave
// with 16-byte stores.  Starts with a barrier (the LDS may still be in use).
template <typename T, int Q, int P>
__device__ __forceinline__ void dcb_write(const Problem& pb, int64_t bgc, const f32x4_t (&dcb)[DcbCfg<T, Q, P>::NOWN],
                                          char* smem) {
  using Cf = DcbCfg<T, Q, P>;
  constexpr int NTHR = Cf::NTHR, VEC = Cf::VEC;
  const int tid = threadIdx.x, w = wave_id_s(), l = lane_id(), r16 = l & 15, kg = l >> 4;
  T* s_xk = reinterpret_cast<T*>(smem);
  constexpr int RB = Cf::RB, LDR = Cf::LDR, CPR = Q / VEC;   // 16-byte chunks per row
  T* s_out = s_xk;
  T* dcb_out = static_cast<T*>(pb.dcb) + bgc * Q * Q;
  T* dcbt_out = static_cast<T*>(pb.dcbt) + bgc * Q * Q;
#pragma unroll 1
  for (int pass = 0; pass < 2 * (Q / RB); ++pass) {
    const bool trans = pass >= Q / RB;
    const int r0 = (trans ? pass - Q / RB : pass) * RB;   // first output row of the pass
    __syncthreads();   // the x / dy rows (first pass) or the previous pass's rows are read
    for (int v = tid; v < RB * CPR; v += NTHR)
      *reinterpret_cast<uint4*>(s_out + (v / CPR) * LDR + (v % CPR) * VEC) = zero_u4();
    __syncthreads();
#pragma clang loop unroll(full)
    for (int k = 0; k < Cf::NOWN; ++k) {
      int I, J;
      bool second;
      Cf::Split::tile(w, k, I, J, second);
      if (!trans && 16 * I >= r0 && 16 * I < r0 + RB) {
        // rows 16 I + 4 kg + r of dCB, column 16 J + r16
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s_out[(16 * I + 4 * kg + r - r0) * LDR + 16 * J + r16] = Elem<T>::from_f(dcb[k][r]);
      }
      if (trans && 16 * J >= r0 && 16 * J < r0 + RB) {
        // row 16 J + r16 of dCB^T, columns 16 I + 4 kg .. + 3
        T* dst = s_out + (16 * J + r16 - r0) * LDR + 16 * I + 4 * kg;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[r] = Elem<T>::from_f(dcb[k][r]);
      }
    }
    __syncthreads();
    T* gout = (trans ? dcbt_out : dcb_out) + static_cast<int64_t>(r0) * Q;
    for (int v = tid; v < RB * CPR; v += NTHR)
      *reinterpret_cast<uint4*>(gout + static_cast<int64_t>(v / CPR) * Q + (v % CPR) * VEC) =
          *reinterpret_cast<const uint4*>(s_out + (v / CPR) * LDR + (v % CPR) * VEC);
  }
}

template <typename T, int Q, int P>
__global__ __launch_bounds__((DcbCfg<T, Q, P>::NTHR)) void k_dcb(Problem pb) {
  using Cf = DcbCfg<T, Q, P>;
  constexpr int NTHR = Cf::NTHR, LDP = Cf::LDP;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* s_xk = reinterpret_cast<T*>(smem);
  T* s_dyk = s_xk + Q * LDP;
  float* s_acs = reinterpret_cast<float*>(s_dyk + Q * LDP);
  float* s_dt = s_acs + Q;
  float* s_er = s_dt + Q;
  int* s_lo = reinterpret_cast<int*>(s_er + Q);

  // logical blocks: the slices of one (batch, group, chunk) are consecutive
  const int S = pb.nslice;
  const int64_t total = static_cast<int64_t>(pb.B) * pb.G * pb.nc * S;
  const int64_t lbs = xcd_logical_block(blockIdx.x, total);
  const int sl = static_cast<int>(lbs % S);
  const int64_t lb = lbs / S;
  const int c = static_cast<int>(lb % pb.nc);
  const int64_t bg = lb / pb.nc;
  const int g = static_cast<int>(bg % pb.G), b = static_cast<int>(bg / pb.G);
  const int tid = threadIdx.x, w = wave_id_s(), l = lane_id();
  const int64_t bc = static_cast<int64_t>(b) * pb.nc + c;
  const T* xg = static_cast<const T*>(pb.x);
  const T* dyg = static_cast<const T*>(pb.dy);
  // this block's heads of the group: [hh_lo, hh_hi) (empty for a trailing slice)
  const int hps = (pb.hpg + S - 1) / S;
  const int hh_lo = sl * hps, hh_hi = min(pb.hpg, hh_lo + hps);

  const int64_t bgc = (static_cast<int64_t>(b) * pb.G + g) * pb.nc + c;
  for (int i = tid; i < Q; i += NTHR) s_lo[i] = seg_lo(pb.segpos[bc * Q + i]);

  // ---- CB = C B^T over the owned causal tiles.  It is the same for every
  // head of the group, so it is formed once here (by the first slice) and
  // stored for the head kernel in fp32, in that kernel's (wave, tile) order
  // and lane layout.
  if (sl == 0) {   // (uniform)
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

  // each head's x / dy rows and Acs / dt are loaded into registers while the
  // previous head's tiles are multiplied
  static_assert(NTHR >= Q, "one thread per chunk position");
  RowStage<T, Q, P, NTHR> st_x, st_dy;
  float acs_n = 0.f, dt_n = 0.f;
  // per-lane offsets of the head rows: fixed for the block, only the base
  // moves from head to head
  const auto off_h = RowStage<T, Q, P, NTHR>::offsets(static_cast<uint32_t>(pb.H * P * sizeof(T)), pb.L - c * Q);
  const int64_t row0 = (static_cast<int64_t>(b) * pb.L + static_cast<int64_t>(c) * Q) * pb.H * P;
  auto load_head = [&](int hh) {
    const int h = g * pb.hpg + hh;
    const int64_t bhc = (static_cast<int64_t>(b) * pb.H + h) * pb.nc + c;
    st_x.load_at(xg + row0 + h * P, off_h);
    st_dy.load_at(dyg + row0 + h * P, off_h);
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
  if (hh_lo < hh_hi) load_head(hh_lo);

  for (int hh = hh_lo; hh < hh_hi; ++hh) {
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
    if (hh + 1 < hh_hi) load_head(hh + 1);

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

  if (S == 1) {
    dcb_write<T, Q, P>(pb, bgc, dcb, smem);
  } else {   // this slice's sums -> its slot, in the CB tiles' (wave, tile) order and lane layout
    float* dst = pb.dcbp + ((bgc * S + sl) * Cf::W + w) * Cf::NOWN * 256 + l * 4;
#pragma unroll
    for (int k = 0; k < Cf::NOWN; ++k) *reinterpret_cast<f32x4_t*>(dst + k * 256) = dcb[k];
  }
}

// The slices' dCB tiles of one (batch, group, chunk), added in slice order,
// -> dcb and dcbt (the grid: one block per (batch, group, chunk)).
template <typename T, int Q, int P>
__global__ __launch_bounds__((DcbCfg<T, Q, P>::NTHR)) void k_dcb_out(Problem pb) {
  using Cf = DcbCfg<T, Q, P>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int64_t total = static_cast<int64_t>(pb.B) * pb.G * pb.nc;
  const int64_t bgc = xcd_logical_block(blockIdx.x, total);   // (batch, group, chunk), row-major
  const int S = pb.nslice, w = wave_id_s(), l = lane_id();
  f32x4_t dcb[Cf::NOWN];
  const float* src = pb.dcbp + (bgc * S * Cf::W + w) * Cf::NOWN * 256 + l * 4;
#pragma unroll
  for (int k = 0; k < Cf::NOWN; ++k) dcb[k] = *reinterpret_cast<const f32x4_t*>(src + k * 256);
  for (int s = 1; s < S; ++s) {
    const float* q = src + static_cast<int64_t>(s) * Cf::W * Cf::NOWN * 256;
#pragma unroll
    for (int k = 0; k < Cf::NOWN; ++k) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(q + k * 256);
#pragma unroll
      for (int r = 0; r < 4; ++r) dcb[k][r] += v[r];
    }
  }
  dcb_write<T, Q, P>(pb, bgc, dcb, smem);
}

template <typename T, int Q, int P>
static hipError_t launch_dcb_t(const Problem& pb, hipStream_t s) {
  using C1 = DcbCfg<T, Q, P>;
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&k_dcb<T, Q, P>), C1::LDS);
  if (e == hipSuccess && pb.nslice > 1)
    e = ensure_dynamic_lds(reinterpret_cast<const void*>(&k_dcb_out<T, Q, P>), C1::LDS);
  if (e != hipSuccess) return e;
  const int64_t b1 = static_cast<int64_t>(pb.B) * pb.G * pb.nc;
  hipLaunchKernelGGL((k_dcb<T, Q, P>), dim3(static_cast<unsigned>(b1 * pb.nslice)), dim3(C1::NTHR), C1::LDS, s, pb);
  e = hipGetLastError();
  if (e != hipSuccess || pb.nslice == 1) return e;
  hipLaunchKernelGGL((k_dcb_out<T, Q, P>), dim3(static_cast<unsigned>(b1)), dim3(C1::NTHR), C1::LDS, s, pb);
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
