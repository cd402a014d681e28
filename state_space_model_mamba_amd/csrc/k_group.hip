// Group kernels: dB and dC of one (batch, group, chunk) -- the
// chunk_scan_bwd_dC and chunk_state_bwd_db rows of the kernel table on the
// page "Deterministic bwd kernel for mamba2", plus the intra-chunk dCB
// product that both need.  The head sum of every term runs inside one block
// in ascending head order (fp32 accumulators), so there are no per-head
// slots and no atomics.
//
// k_dcb, per (batch, group, chunk):
//   CB  = C B^T over the causal tiles (head independent; fp32, for the head kernel)
//   dCB = sum_h W_h o (dy_h x_h^T),  W_h[i,j] = exp(Acs_i - Acs_j) dt_j  (j <= i, same segment)
//   written as a Q x Q tile and as its transpose (zeros above the diagonal).
// k_dbdc, per (batch, group, chunk, dstate tile):
//   dC = dCB B + sum_h exp(Acs_i) dy_h,i E_h,seg(i)
//   dB = dCB^T C + sum_h w_h,j x_h,j dS_h,     w_j = exp(Acs_end - Acs_j) dt_j (last segment)
//   E is the state entering a row's segment: Hin for a segment that continues
//   the previous chunk's sequence, the sequence's initial state otherwise.
// k_dbdc also leaves, per head, the partials (over its dstate tile) of
//   offd_i = exp(Acs_i) dy_i . (E C_i)   and   endd = <dS, E_end>
// (the off-diagonal and chunk-end ddA_cumsum terms) in slots owned by
// (batch, head, chunk, tile).
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

// ----------------------------------------------------------------------------
// k_dbdc
// ----------------------------------------------------------------------------
template <typename T, int Q, int P, int NTG>
struct DbdcCfg {
  static constexpr int T16 = Q / 16;
  static constexpr int W = T16 / 2;
  using Split = CausalSplit<T16, W>;
  static constexpr int NROW = Split::NCOL;       // owned row tiles per wave
  static constexpr int NTHR = W * WAVE;
  static constexpr int NCT = NTG / 16;
  static constexpr int VEC = Vec16<T>::N;
  static constexpr int KSL = 32;                 // K slab of the dCB products
  static constexpr int LDK = KSL + VEC;
  static constexpr int LDP = P + VEC;
  static constexpr size_t R_SLAB = (size_t(Q) + NTG) * LDK * sizeof(T);
  static constexpr size_t R_HEAD = (size_t(Q) + NTG) * LDP * sizeof(T);
  static constexpr size_t R1 = ((R_SLAB > R_HEAD ? R_SLAB : R_HEAD) + 15) / 16 * 16;
  static constexpr int LDC = NTG + VEC;
  static constexpr size_t RC = size_t(Q) * LDC * sizeof(T);   // C rows of the chunk (dstate tile)
  // vectors: acs, eA/w (2 Q floats), seg (Q ints), segstart (Q + 1 ints), red (W + 8 floats)
  static constexpr size_t LDS =
      R1 + RC + size_t(2) * Q * 4 + size_t(Q) * 4 + size_t(Q + 1) * 4 + size_t(W + 8) * 4;
};

template <typename T, int Q, int P, int NTG>
__global__ __launch_bounds__((DbdcCfg<T, Q, P, NTG>::NTHR)) void k_dbdc(Problem pb) {
  using Cf = DbdcCfg<T, Q, P, NTG>;
  constexpr int T16 = Cf::T16, W = Cf::W, NTHR = Cf::NTHR, NCT = Cf::NCT, VEC = Cf::VEC;
  constexpr int KSL = Cf::KSL, LDK = Cf::LDK, LDP = Cf::LDP;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* s_a = reinterpret_cast<T*>(smem);          // slab phase: [Q][LDK] rows of dCB or dCB^T
  T* s_b = s_a + Q * LDK;                       //             [NTG][LDK] B^T or C^T slab
  T* s_rows = reinterpret_cast<T*>(smem);       // head phase: [Q][LDP] dy or x rows
  T* s_nt = s_rows + Q * LDP;                   //             [NTG][LDP] E^T or dS^T
  T* s_cm = reinterpret_cast<T*>(smem + Cf::R1);   // [Q][LDC] C rows for the offd row dots
  float* s_acs = reinterpret_cast<float*>(smem + Cf::R1 + Cf::RC);
  float* s_v = s_acs + Q;                       // exp(Acs_i) or w_j
  int* s_seg = reinterpret_cast<int*>(s_v + Q);
  int* s_segstart = s_seg + Q;
  float* s_red = reinterpret_cast<float*>(s_segstart + Q + 1);

  const int ntiles = pb.ntg;
  const int64_t total = static_cast<int64_t>(pb.B) * pb.G * pb.nc * ntiles;
  const int64_t lb = xcd_logical_block(blockIdx.x, total);
  const int ntile = static_cast<int>(lb % ntiles);
  int64_t rest = lb / ntiles;
  const int c = static_cast<int>(rest % pb.nc);
  rest /= pb.nc;
  const int g = static_cast<int>(rest % pb.G), b = static_cast<int>(rest / pb.G);
  const int n0 = ntile * NTG;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r16 = l & 15, kg = l >> 4;
  const int64_t bc = static_cast<int64_t>(b) * pb.nc + c;
  const int64_t bgc = (static_cast<int64_t>(b) * pb.G + g) * pb.nc + c;
  const T* xg = static_cast<const T*>(pb.x);
  const T* dyg = static_cast<const T*>(pb.dy);
  const T* Bg = static_cast<const T*>(pb.Bm);
  const T* Cg = static_cast<const T*>(pb.Cm);
  const T* dcb_in = static_cast<const T*>(pb.dcb) + bgc * Q * Q;
  const T* dcbt_in = static_cast<const T*>(pb.dcbt) + bgc * Q * Q;
  constexpr int NROW = Cf::NROW;
  int own[NROW];
#pragma unroll
  for (int a = 0; a < NROW; ++a) own[a] = Cf::Split::col(w, a);

  const int nstart = pb.cinfo[bc * CINFO + 0];
  const int seqbase = pb.cinfo[bc * CINFO + 3];
  for (int i = tid; i < Q; i += NTHR) s_seg[i] = pb.segpos[bc * Q + i];
  if (tid == 0) s_segstart[0] = 0;
  __syncthreads();
  const int start0 = seg_rank(s_seg[0]);
  const int nseg = nstart + 1 - start0;
  const int lolast = seg_lo(s_seg[Q - 1]);
  for (int i = tid; i < Q; i += NTHR)
    if (i > 0 && seg_lo(s_seg[i]) == i) s_segstart[seg_rank(s_seg[i]) - start0] = i;
  if (tid == 0) s_segstart[nseg] = Q;

  auto bc_row = [&](const T* base, int k0) {
    return [=](int kk) -> const T* {
      const int t = c * Q + k0 + kk;
      return t < pb.L ? base + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + n0 : nullptr;
    };
  };
  // K-slab product: acc[a][nt] += rows own[a] of `rowsrc` (Q x Q, row-major)
  // times rows k0.. of the chunk's `colsrc` tile (B or C), slab by slab, the
  // next slab loaded into registers while the current one is multiplied
  auto slab_product = [&](f32x4_t (&acc)[NROW][NCT], const T* rowsrc, const T* colsrc, bool lower) {
    RowStage<T, Q, KSL, NTHR> st_a;
    RowStage<T, KSL, NTG, NTHR> st_b;
    auto a_row = [=](int k0) {
      return [=](int i) -> const T* { return rowsrc + static_cast<int64_t>(i) * Q + k0; };
    };
    st_a.load(a_row(0));
    st_b.load(bc_row(colsrc, 0));
    for (int k0 = 0; k0 < Q; k0 += KSL) {
      __syncthreads();
      st_a.store(s_a, LDK);
      st_b.template store_transposed<T>(s_b, LDK);
      __syncthreads();
      if (k0 + KSL < Q) {
        st_a.load(a_row(k0 + KSL));
        st_b.load(bc_row(colsrc, k0 + KSL));
      }
#pragma unroll
      for (int a = 0; a < NROW; ++a) {
        const int R = own[a];
        // dCB rows R hold columns <= 16R+15; dCB^T rows R hold columns >= 16R
        const bool live = lower ? (k0 <= 16 * R + 15) : (k0 + KSL > 16 * R);
        if (!live) continue;
#pragma unroll
        for (int nt = 0; nt < NCT; ++nt)
          acc[a][nt] = tile_mma_kk<T>(acc[a][nt], s_a + 16 * R * LDK, LDK, s_b + 16 * nt * LDK, LDK, 0, KSL);
      }
    }
  };
  auto head_row = [&](const T* base, int h) {
    return [=](int i) -> const T* {
      const int t = c * Q + i;
      return t < pb.L ? base + ((static_cast<int64_t>(b) * pb.L + t) * pb.H + h) * P : nullptr;
    };
  };
  auto state_row = [&](const float* base) {
    return [=](int p) -> const float* { return base + static_cast<int64_t>(p) * pb.N + n0; };
  };

  f32x4_t acc[NROW][NCT];

  // ------------------------------------------------------------------ dC
#pragma unroll
  for (int a = 0; a < NROW; ++a)
#pragma unroll
    for (int nt = 0; nt < NCT; ++nt) acc[a][nt] = zero4();
  slab_product(acc, dcb_in, Bg, true);
  // C rows of the chunk (this dstate tile), for the offd row dots
  {
    RowStage<T, Q, NTG, NTHR> st_cm;
    st_cm.load(bc_row(Cg, 0));
    st_cm.store(s_cm, Cf::LDC);
  }
  for (int hh = 0; hh < pb.hpg; ++hh) {
    const int h = g * pb.hpg + hh;
    const int64_t bhc = (static_cast<int64_t>(b) * pb.H + h) * pb.nc + c;
    __syncthreads();
    for (int i = tid; i < Q; i += NTHR) s_v[i] = Elem<T>::exp(pb.acs[bhc * Q + i]);
    {
      RowStage<T, Q, P, NTHR> st_dy;
      st_dy.load(head_row(dyg, h));
      st_dy.store(s_rows, LDP);
    }
    float offp[NROW][4];
#pragma unroll
    for (int a = 0; a < NROW; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) offp[a][r] = 0.f;
    float endp = 0.f;
    for (int m = 0; m < nseg; ++m) {
      const int lo = s_segstart[m], hi = s_segstart[m + 1];
      const int rank = seg_rank(s_seg[lo]);
      const float* esrc = nullptr;
      if (rank == 0) {
        esrc = pb.hin + bhc * P * pb.N;
      } else if (pb.h0) {
        const int s = clamp_seq(seqbase + rank - 1, pb.nseqs);
        esrc = pb.h0 + (static_cast<int64_t>(s) * pb.H + h) * P * pb.N;
      }
      const bool want_end = (hi == Q) && (nstart == 0 || rank > 0);
      if (m > 0) __syncthreads();  // previous pass finished reading the E tile
      if (esrc) {
        RowStage<float, P, NTG, NTHR> st_e;
        st_e.load(state_row(esrc));
        if (want_end) {
          RowStage<float, P, NTG, NTHR> st_s;
          st_s.load(state_row(pb.dstate + bhc * P * pb.N));
#pragma unroll
          for (int k = 0; k < st_e.IT; ++k)
#pragma unroll
            for (int e = 0; e < st_e.VEC; ++e) endp += vget<float>(st_s.buf[k], e) * vget<float>(st_e.buf[k], e);
        }
        st_e.template store_transposed<T>(s_nt, LDP);
      }
      __syncthreads();
      if (!esrc) continue;
#pragma unroll
      for (int a = 0; a < NROW; ++a) {
        const int I = own[a];
        if (16 * I + 15 < lo || 16 * I >= hi) continue;
#pragma unroll
        for (int nt = 0; nt < NCT; ++nt) {
          const f32x4_t y = tile_mma_kk<T>(zero4(), s_rows + 16 * I * LDP, LDP, s_nt + 16 * nt * LDP, LDP, 0, P);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * I + 4 * kg + r;
            if (i >= lo && i < hi) {
              const float yv = y[r] * s_v[i];
              acc[a][nt][r] += yv;
              offp[a][r] += yv * Elem<T>::to_f(s_cm[i * Cf::LDC + 16 * nt + r16]);
            }
          }
        }
      }
    }
    const int64_t offd_base = (bhc * pb.ntg + ntile) * Q;
#pragma unroll
    for (int a = 0; a < NROW; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = sum16(offp[a][r]);
        if (r16 == 0) pb.offd[offd_base + 16 * own[a] + 4 * kg + r] = v;
      }
    const float ev = wave_sum(endp);
    if (l == 0) s_red[w] = ev;
    __syncthreads();
    if (tid == 0) {
      float s = 0.f;
      for (int k = 0; k < W; ++k) s += s_red[k];
      pb.endd[bhc * pb.ntg + ntile] = s;
    }
  }
#pragma unroll
  for (int a = 0; a < NROW; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = c * Q + 16 * own[a] + 4 * kg + r;
      if (t >= pb.L) continue;
      T* dst = static_cast<T*>(pb.dC) + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + n0;
#pragma unroll
      for (int nt = 0; nt < NCT; ++nt) dst[16 * nt + r16] = Elem<T>::from_f(acc[a][nt][r]);
    }

  // ------------------------------------------------------------------ dB
#pragma unroll
  for (int a = 0; a < NROW; ++a)
#pragma unroll
    for (int nt = 0; nt < NCT; ++nt) acc[a][nt] = zero4();
  slab_product(acc, dcbt_in, Cg, false);
  for (int hh = 0; hh < pb.hpg; ++hh) {
    const int h = g * pb.hpg + hh;
    const int64_t bhc = (static_cast<int64_t>(b) * pb.H + h) * pb.nc + c;
    __syncthreads();
    const float acs_end = pb.acs[bhc * Q + Q - 1];
    for (int i = tid; i < Q; i += NTHR)
      s_v[i] = (i >= lolast) ? Elem<T>::exp(acs_end - pb.acs[bhc * Q + i]) * pb.dtc[bhc * Q + i] : 0.f;
    {
      RowStage<T, Q, P, NTHR> st_x;
      RowStage<float, P, NTG, NTHR> st_s;
      st_x.load(head_row(xg, h));
      st_s.load(state_row(pb.dstate + bhc * P * pb.N));
      st_x.store(s_rows, LDP);
      st_s.template store_transposed<T>(s_nt, LDP);
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < NROW; ++a) {
      const int J = own[a];
      if (16 * J + 15 < lolast) continue;
#pragma unroll
      for (int nt = 0; nt < NCT; ++nt) {
        const f32x4_t u = tile_mma_kk<T>(zero4(), s_rows + 16 * J * LDP, LDP, s_nt + 16 * nt * LDP, LDP, 0, P);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[a][nt][r] += s_v[16 * J + 4 * kg + r] * u[r];
      }
    }
  }
#pragma unroll
  for (int a = 0; a < NROW; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = c * Q + 16 * own[a] + 4 * kg + r;
      if (t >= pb.L) continue;
      T* dst = static_cast<T*>(pb.dB) + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + n0;
#pragma unroll
      for (int nt = 0; nt < NCT; ++nt) dst[16 * nt + r16] = Elem<T>::from_f(acc[a][nt][r]);
    }
}

// dstate tile width of k_dbdc
int group_ntile(int N, bool io_bf16) {
  (void)io_bf16;
  if (N % 128 == 0) return 128;
  if (N % 64 == 0) return 64;
  if (N % 32 == 0) return 32;
  return 16;
}

template <typename K>
static hipError_t allow_lds(K kernel, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(bytes));
}

template <typename T, int Q, int P, int NTG>
static hipError_t launch_group_t(const Problem& pb, int part, hipStream_t s) {
  using C1 = DcbCfg<T, Q, P>;
  using C2 = DbdcCfg<T, Q, P, NTG>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = allow_lds(&k_dcb<T, Q, P>, C1::LDS);
    if (e == hipSuccess) e = allow_lds(&k_dbdc<T, Q, P, NTG>, C2::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t b1 = static_cast<int64_t>(pb.B) * pb.G * pb.nc;
  if (part == 0)
    hipLaunchKernelGGL((k_dcb<T, Q, P>), dim3(static_cast<unsigned>(b1)), dim3(C1::NTHR), C1::LDS, s, pb);
  else
    hipLaunchKernelGGL((k_dbdc<T, Q, P, NTG>), dim3(static_cast<unsigned>(b1 * pb.ntg)), dim3(C2::NTHR),
                       C2::LDS, s, pb);
  return hipGetLastError();
}

template <typename T, int Q, int P>
static hipError_t launch_group_qp(const Problem& pb, int part, hipStream_t s) {
  const int w = pb.N / pb.ntg;
  if (w == 128) return launch_group_t<T, Q, P, 128>(pb, part, s);
  if (w == 64) return launch_group_t<T, Q, P, 64>(pb, part, s);
  if (w == 32) return launch_group_t<T, Q, P, 32>(pb, part, s);
  if (w == 16) return launch_group_t<T, Q, P, 16>(pb, part, s);
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_group_any(const Problem& pb, int part, hipStream_t s) {
#define SSD_GROUP_CASE(QQ, PP) \
  if (pb.Q == QQ && pb.P == PP) return launch_group_qp<T, QQ, PP>(pb, part, s);
  if constexpr (sizeof(T) == 2) {
    SSD_BF16_SHAPES(SSD_GROUP_CASE)
  } else {
    SSD_F32_SHAPES(SSD_GROUP_CASE)
  }
#undef SSD_GROUP_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_dcb(const Problem& pb, bool io_bf16, hipStream_t s) {
  return io_bf16 ? launch_group_any<bf16_t>(pb, 0, s) : launch_group_any<float>(pb, 0, s);
}

hipError_t launch_dbdc(const Problem& pb, bool io_bf16, hipStream_t s) {
  return io_bf16 ? launch_group_any<bf16_t>(pb, 1, s) : launch_group_any<float>(pb, 1, s);
}

// LDS bytes of the larger group kernel for a compiled shape; ~0 when not compiled.
size_t group_lds_bytes(int Q, int P, int NTG, bool bf16) {
  size_t r = ~size_t(0);
#define SSD_GROUP_LDS(TT, QQ, PP)                                                             \
  if (Q == QQ && P == PP) {                                                                   \
    const size_t a = DcbCfg<TT, QQ, PP>::LDS;                                                 \
    size_t bb = ~size_t(0);                                                                   \
    if (NTG == 128) bb = DbdcCfg<TT, QQ, PP, 128>::LDS;                                       \
    if (NTG == 64) bb = DbdcCfg<TT, QQ, PP, 64>::LDS;                                         \
    if (NTG == 32) bb = DbdcCfg<TT, QQ, PP, 32>::LDS;                                         \
    if (NTG == 16) bb = DbdcCfg<TT, QQ, PP, 16>::LDS;                                         \
    r = a > bb ? a : bb;                                                                      \
  }
#define SSD_GROUP_LDS_B(QQ, PP) if (bf16) { SSD_GROUP_LDS(bf16_t, QQ, PP) }
#define SSD_GROUP_LDS_F(QQ, PP) if (!bf16) { SSD_GROUP_LDS(float, QQ, PP) }
  SSD_BF16_SHAPES(SSD_GROUP_LDS_B)
  SSD_F32_SHAPES(SSD_GROUP_LDS_F)
#undef SSD_GROUP_LDS_B
#undef SSD_GROUP_LDS_F
#undef SSD_GROUP_LDS
  return r;
}

}  // namespace ssd
