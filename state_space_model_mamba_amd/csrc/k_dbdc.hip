// dC and dB of one (batch, group, chunk, dstate tile) -- the chunk_scan_bwd_dC
// and chunk_state_bwd_db rows of the kernel table on the page "Deterministic
// bwd kernel for mamba2".  The head sum of every term runs inside one block
// in ascending head order (fp32 accumulators): no per-head slots, no atomics.
//
// k_dc:
//   dC_i  = sum_j dCB[i,j] B_j  +  sum_h exp(Acs_h,i) dy_h,i E_h,seg(i)
//   offd_h,i = exp(Acs_h,i) dy_h,i . (E_h,seg(i) C_i)   (this tile's part, per head)
//   endd_h   = <dS_h, E_h,end>                        (this tile's part, per head)
// k_db:
//   dB_j  = sum_i dCB[i,j] C_i  +  sum_h w_h,j x_h,j dS_h,   w_j = exp(Acs_end - Acs_j) dt_j
//                                                           (last segment only)
// E is the state entering a row's segment: Hin for a segment that continues
// the previous chunk's sequence, the sequence's initial state otherwise.
// offd and endd are the off-diagonal and chunk-end ddA_cumsum terms; they go
// to slots owned by (batch, head, chunk, tile), summed later in tile order.
// On a grid too small for the GPU the group's heads are cut into nslice_bd
// slices of consecutive heads, one block each (the first also takes the dCB
// product): each block parks its fp32 rows in a workspace slot and k_bd_out
// adds the slots in slice order.
//
// Every operand whose contraction index is its row index (B, C, E, dS) is
// staged row-major with 16-byte (or 8-byte) stores and read as MFMA
// fragments with the LDS transpose reads; the next head's rows are loaded
// into registers while the current head is multiplied.
#include <type_traits>

#include "ssd_problem.h"
#include "ssd_tiles.h"

namespace ssd {

// The owned row tiles that a K slab of the dCB product touches vary with the
// wave and the slab (causally dead slabs): the slab's body is instantiated per
// combination of live tiles and chosen by one wave-uniform branch, so its
// fragment reads and products stay one straight-line sequence (a branch per
// product made every product wait for all LDS reads in flight).
template <typename F>
__device__ __forceinline__ void with_live(bool live0, bool live1, F&& f) {
  if (live0 && live1)
    f(std::true_type{}, std::true_type{});
  else if (live0)
    f(std::true_type{}, std::false_type{});
  else if (live1)
    f(std::false_type{}, std::true_type{});
}

template <typename T, int Q, int P, int NTG>
struct DbdcCfg {
  static constexpr int T16 = Q / 16;
  static constexpr int W = causal_waves<Q>();
  using Split = CausalSplit<T16, W>;
  static constexpr int NROW = Split::NCOL;       // owned row tiles per wave: {p, T-1-p}
  static constexpr int NTHR = W * WAVE;
  static_assert(NTHR >= Q, "one thread per chunk position");
  static constexpr int NCT = NTG / 16;
  static constexpr int VEC = Vec16<T>::N;
  // K slab of the dCB products: 64 positions where that takes no more LDS
  // than the head phase (P >= 64), else 32
  static constexpr int KSL = P >= 64 ? 64 : 32;
  static constexpr int LDA = KSL + VEC;          // dCB slab rows [i][k]
  static constexpr int LDK = kn_pitch<T>(NTG);   // B / C rows [k][n]
  static constexpr int LDP = P + VEC;            // dy / x rows [i][p]
  static constexpr int LDE = kn_pitch<T>(NTG);   // E / dS rows [p][n]
  static constexpr size_t R_SLAB = (size_t(Q) * LDA + size_t(KSL) * LDK) * sizeof(T);
  static constexpr size_t R_HEAD = (size_t(Q) * LDP + size_t(P) * LDE) * sizeof(T);
  static constexpr size_t R_C = size_t(Q) * LDK * sizeof(T);
  static constexpr size_t R1 = ((R_SLAB > R_HEAD ? R_SLAB : R_HEAD) + 15) / 16 * 16;
  // k_dc keeps the chunk's C rows (this tile) in LDS behind R1
  static constexpr size_t R2 = R1 + (R_C + 15) / 16 * 16;
  // vectors: v (Q floats), seg (Q ints), segstart (Q + 1 ints), red (W + 8 floats)
  static constexpr size_t VEC_BYTES = size_t(Q) * 4 * 2 + size_t(Q + 1) * 4 + size_t(W + 8) * 4;
  static constexpr size_t LDS = R2 + VEC_BYTES;      // k_dc
  static constexpr size_t LDS_DB = R1 + VEC_BYTES;   // k_db
};

// Block coordinates and the chunk's segment list, shared by both kernels.
struct DbdcBlock {
  int b, g, c, ntile, n0;
  int sl, hh_lo, hh_hi;   // head slice and its heads of the group, [hh_lo, hh_hi)
  int64_t bc, bgc;
  int nstart, seqbase, start0, nseg, lolast;
};

template <int Q, int NTHR>
__device__ __forceinline__ DbdcBlock dbdc_block(const Problem& pb, int* s_seg, int* s_segstart) {
  DbdcBlock k;
  const int tid = threadIdx.x;
  const int S = pb.nslice_bd;
  const int64_t total = static_cast<int64_t>(pb.B) * pb.G * pb.nc * pb.ntg * S;
  const int64_t lbs = xcd_logical_block(blockIdx.x, total);   // the slices of one tile are consecutive
  k.sl = static_cast<int>(lbs % S);
  const int64_t lb = lbs / S;
  const int hps = (pb.hpg + S - 1) / S;
  k.hh_lo = k.sl * hps;
  k.hh_hi = min(pb.hpg, k.hh_lo + hps);
  k.ntile = static_cast<int>(lb % pb.ntg);
  int64_t rest = lb / pb.ntg;
  k.c = static_cast<int>(rest % pb.nc);
  rest /= pb.nc;
  k.g = static_cast<int>(rest % pb.G);
  k.b = static_cast<int>(rest / pb.G);
  k.bc = static_cast<int64_t>(k.b) * pb.nc + k.c;
  k.bgc = (static_cast<int64_t>(k.b) * pb.G + k.g) * pb.nc + k.c;
  k.nstart = pb.cinfo[k.bc * CINFO + 0];
  k.seqbase = pb.cinfo[k.bc * CINFO + 3];
  if (tid < Q) s_seg[tid] = pb.segpos[k.bc * Q + tid];
  if (tid == 0) s_segstart[0] = 0;
  __syncthreads();
  k.start0 = seg_rank(s_seg[0]);
  k.nseg = k.nstart + 1 - k.start0;
  k.lolast = seg_lo(s_seg[Q - 1]);
  if (tid < Q && tid > 0 && seg_lo(s_seg[tid]) == tid) s_segstart[seg_rank(s_seg[tid]) - k.start0] = tid;
  if (tid == 0) s_segstart[k.nseg] = Q;
  __syncthreads();
  return k;
}

// acc[a][nt] += rows own[a] of `rowsrc` (a Q x Q matrix, row-major) times the
// chunk's rows of `colsrc` (B or C, this dstate tile), K slab by K slab; the
// next slab is loaded into registers while the current one is multiplied.
// lower: rowsrc rows R hold columns <= 16R+15 (dCB); else columns >= 16R (dCB^T).
template <typename T, int Q, int P, int NTG>
__device__ __forceinline__ void dcb_slab_product(const Problem& pb, const DbdcBlock& k,
                                                 f32x4_t (&acc)[2][NTG / 16], const int (&own)[2],
                                                 const T* rowsrc, const T* colsrc, bool lower, T* s_a, T* s_k) {
  using Cf = DbdcCfg<T, Q, P, NTG>;
  constexpr int KSL = Cf::KSL, NTHR = Cf::NTHR;
  RowStage<T, Q, KSL, NTHR> st_a;
  RowStage<T, KSL, NTG, NTHR> st_k;
  auto a_row = [=](int k0) {
    return [=](int i) -> const T* { return rowsrc + static_cast<int64_t>(i) * Q + k0; };
  };
  auto k_row = [=, &pb](int k0) {
    return [=, &pb](int kk) -> const T* {
      const int t = k.c * Q + k0 + kk;
      return t < pb.L ? colsrc + ((static_cast<int64_t>(k.b) * pb.L + t) * pb.G + k.g) * pb.N + k.n0 : nullptr;
    };
  };
  st_a.load(a_row(0));
  st_k.load(k_row(0));
  for (int k0 = 0; k0 < Q; k0 += KSL) {
    __syncthreads();
    st_a.store(s_a, Cf::LDA);
    st_k.store(s_k, Cf::LDK);
    __syncthreads();
    if (k0 + KSL < Q) {
      st_a.load(a_row(k0 + KSL));
      st_k.load(k_row(k0 + KSL));
    }
    constexpr int KS = KSL / Mma<T>::KSTEP;
    const int l = lane_id();
    bool live[2];   // the row tile has causally live columns in this slab
#pragma unroll
    for (int a = 0; a < 2; ++a) live[a] = lower ? (k0 <= 16 * own[a] + 15) : (k0 + KSL > 16 * own[a]);
    // both owned row tiles take each column fragment from one LDS read
    with_live(live[0], live[1], [&](auto L0, auto L1) {
      constexpr bool LV[2] = {decltype(L0)::value, decltype(L1)::value};
      typename Mma<T>::frag af[2][KS];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        if (LV[a])
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            af[a][ks] = Mma<T>::load_k(s_a + (16 * own[a] + (l & 15)) * Cf::LDA + (l >> 4) * Mma<T>::KW +
                                       ks * Mma<T>::KSTEP);
#pragma unroll
      for (int nt = 0; nt < NTG / 16; ++nt) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const typename Mma<T>::frag bf = load_kn<T>(s_k + 16 * nt, Cf::LDK, ks * Mma<T>::KSTEP);
#pragma unroll
          for (int a = 0; a < 2; ++a)
            if (LV[a]) acc[a][nt] = Mma<T>::mma(af[a][ks], bf, acc[a][nt]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  }
}

// The block's rows: to dC / dB (out) when it has all of the group's heads,
// else as fp32 to its slice's slot (part: [(b, g, c, tile)][slice][Q][NTG]).
template <typename T, int Q, int NTG>
__device__ __forceinline__ void write_rows(const Problem& pb, const DbdcBlock& k, void* out, float* part,
                                           const f32x4_t (&acc)[2][NTG / 16], const int (&own)[2]) {
  const int l = lane_id(), r16 = l & 15, kg = l >> 4;
  if (pb.nslice_bd > 1) {   // (uniform)
    float* dst = part + ((k.bgc * pb.ntg + k.ntile) * pb.nslice_bd + k.sl) * Q * NTG;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int nt = 0; nt < NTG / 16; ++nt) dst[(16 * own[a] + 4 * kg + r) * NTG + 16 * nt + r16] = acc[a][nt][r];
    return;
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = k.c * Q + 16 * own[a] + 4 * kg + r;
      if (t >= pb.L) continue;
      T* dst = static_cast<T*>(out) + ((static_cast<int64_t>(k.b) * pb.L + t) * pb.G + k.g) * pb.N + k.n0;
#pragma unroll
      for (int nt = 0; nt < NTG / 16; ++nt) dst[16 * nt + r16] = Elem<T>::from_f(acc[a][nt][r]);
    }
}

// ----------------------------------------------------------------------------
// k_dc
// ----------------------------------------------------------------------------
// SEQ: the input has sequence boundaries (seq_idx), so chunks can hold
// several segments; without them every chunk is one segment and the kernel
// keeps no registers for a second segment's early requests.
template <typename T, int Q, int P, int NTG, bool SEQ>
__global__ __launch_bounds__((DbdcCfg<T, Q, P, NTG>::NTHR)) void k_dc(Problem pb) {
  using Cf = DbdcCfg<T, Q, P, NTG>;
  constexpr int W = Cf::W, NTHR = Cf::NTHR, NCT = Cf::NCT, LDP = Cf::LDP, LDE = Cf::LDE, LDK = Cf::LDK;
  constexpr int KP = P / Mma<T>::KSTEP;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* s_a = reinterpret_cast<T*>(smem);      // slab phase: dCB rows [Q][LDA]
  T* s_k = s_a + Q * Cf::LDA;               //             B rows [KSL][LDK]
  T* s_rows = reinterpret_cast<T*>(smem);   // head phase: dy rows [Q][LDP]
  T* s_e = s_rows + Q * LDP;                //             E rows [P][LDE]
  T* s_c = reinterpret_cast<T*>(smem + Cf::R1);   // C rows [Q][LDK] of the chunk
  float* s_v = reinterpret_cast<float*>(smem + Cf::R2);
  int* s_seg = reinterpret_cast<int*>(s_v + Q);
  int* s_segstart = s_seg + Q;
  float* s_red = reinterpret_cast<float*>(s_segstart + Q + 1);

  const int tid = threadIdx.x, w = wave_id_s(), l = lane_id(), r16 = l & 15, kg = l >> 4;
  DbdcBlock k = dbdc_block<Q, NTHR>(pb, s_seg, s_segstart);
  k.n0 = k.ntile * NTG;
  const T* dyg = static_cast<const T*>(pb.dy);
  const T* Bg = static_cast<const T*>(pb.Bm);
  const T* Cg = static_cast<const T*>(pb.Cm);
  int own[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) own[a] = Cf::Split::col(w, a);

  f32x4_t acc[2][NCT];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nt = 0; nt < NCT; ++nt) acc[a][nt] = zero4();
  if (k.sl == 0)   // (uniform) the dCB part, once per tile
    dcb_slab_product<T, Q, P, NTG>(pb, k, acc, own, static_cast<const T*>(pb.dcb) + k.bgc * Q * Q, Bg, true, s_a,
                                   s_k);

  // the chunk's C rows (this tile), for the offd row dots (visible to all
  // waves after the first barrier of the head loop)
  {
    RowStage<T, Q, NTG, NTHR> st_cm;
    st_cm.load([&](int i) -> const T* {
      const int t = k.c * Q + i;
      return t < pb.L ? Cg + ((static_cast<int64_t>(k.b) * pb.L + t) * pb.G + k.g) * pb.N + k.n0 : nullptr;
    });
    st_cm.store(s_c, LDK);
  }

  // entering state of segment m of head h: Hin (I/O dtype) for a segment
  // that continues the chunk's sequence, h0[s] (fp32) for one that starts
  // sequence s, none (zero) when h0 is not given
  struct ERows {
    const void* p;
    bool h0;
  };
  auto e_src = [&](int h, int m) -> ERows {
    const int64_t bhc = (static_cast<int64_t>(k.b) * pb.H + h) * pb.nc + k.c;
    const int rank = __builtin_amdgcn_readfirstlane(seg_rank(s_seg[s_segstart[m]]));
    if (rank == 0) return {static_cast<const T*>(pb.hin) + bhc * P * pb.N, false};
    if (!pb.h0) return {nullptr, true};
    const int s = clamp_seq(k.seqbase + rank - 1, pb.nseqs);
    return {pb.h0 + (static_cast<int64_t>(s) * pb.H + h) * P * pb.N, true};
  };
  auto state_row = [&](const auto* base) {
    return [=, &pb](int p) { return base + static_cast<int64_t>(p) * pb.N + k.n0; };
  };
  auto zero_row = [](int) -> const T* { return nullptr; };
  // per-lane offsets of the head rows (dy) and of the state rows (E, dS) of this
  // tile: fixed for the block, only the base moves from head to head
  const auto off_dy = RowStage<T, Q, P, NTHR>::offsets(static_cast<uint32_t>(pb.H * P * sizeof(T)), pb.L - k.c * Q);
  const auto off_st = RowStage<T, P, NTG, NTHR>::offsets(static_cast<uint32_t>(pb.N * sizeof(T)), P);
  const T* dy_c = dyg + (static_cast<int64_t>(k.b) * pb.L + static_cast<int64_t>(k.c) * Q) * pb.H * P;
  auto load_e = [&](RowStage<T, P, NTG, NTHR>& st, ERows e) {
    if (!e.p)
      st.load(zero_row);
    else if (!e.h0)
      st.load_at(static_cast<const T*>(e.p) + k.n0, off_st);
    else
      st.load_from_f32(state_row(static_cast<const float*>(e.p)));
  };
  // the last segment's <dS, E> feeds endd unless it starts a sequence without a
  // given initial state (E = 0)
  const bool single = k.nseg == 1;

  // next head's rows: dy, segment 0's E, and (single segment) dS
  RowStage<T, Q, P, NTHR> st_dy;
  RowStage<T, P, NTG, NTHR> st_e, st_s;
  float acs_n = 0.f;
  auto load_head = [&](int hh) {
    const int h = k.g * pb.hpg + hh;
    const int64_t bhc = (static_cast<int64_t>(k.b) * pb.H + h) * pb.nc + k.c;
    st_dy.load_at(dy_c + h * P, off_dy);
    load_e(st_e, e_src(h, 0));
    if (single) st_s.load_at(static_cast<const T*>(pb.dstate) + bhc * P * pb.N + k.n0, off_st);
    if (tid < Q) acs_n = pb.acs[bhc * Q + tid];
  };
  // prefetch the next head where its registers fit; a chunk's further segments
  // (a sequence starts inside it) take their E and the chunk-end dS into
  // registers of their own, so the prefetched head's stay untouched
  constexpr bool PF = RowStage<T, Q, P, NTHR>::IT + 2 * RowStage<T, P, NTG, NTHR>::IT <= 16;
  const bool pf = PF;
  RowStage<T, P, NTG, NTHR> st_e2, st_s2;
  // a second segment's entering state when it is a given initial state (fp32),
  // requested before the first segment's products and rounded when staged
  // (where its registers fit: at most four 16-byte pieces per thread)
  using StE = RowStage<T, P, NTG, NTHR>;
  constexpr bool E2PF = SEQ && StE::IT * StE::F4 <= 4;
  uint4 e2raw[StE::IT][StE::F4];
  if (pf && k.hh_lo < k.hh_hi) load_head(k.hh_lo);

  for (int hh = k.hh_lo; hh < k.hh_hi; ++hh) {
    const int h = k.g * pb.hpg + hh;
    const int64_t bhc = (static_cast<int64_t>(k.b) * pb.H + h) * pb.nc + k.c;
    float endp = 0.f;
    if (!pf) load_head(hh);
    __syncthreads();
    st_dy.store(s_rows, LDP);
    st_e.store(s_e, LDE);
    if (single && e_src(h, 0).p) {
#pragma unroll
      for (int kk = 0; kk < st_e.IT; ++kk)
#pragma unroll
        for (int e = 0; e < st_e.VEC; ++e) endp += vget<T>(st_s.buf[kk], e) * vget<T>(st_e.buf[kk], e);
    }
    if (tid < Q) s_v[tid] = Elem<T>::exp(acs_n);
    __syncthreads();
    if (pf && hh + 1 < k.hh_hi) load_head(hh + 1);
    // A chunk in which a sequence starts: the second segment's E (the
    // sequence's initial state) and, when that segment ends the chunk, the
    // chunk-end dS are requested now, so that the first segment's products
    // cover their latency; later segments load theirs when they come.
    bool e2_early = false, s2_early = false;
    if (SEQ && k.nseg > 1) {   // (uniform)
      const ERows e1 = e_src(h, 1);
      if constexpr (E2PF) {
        if (e1.p && e1.h0) {
          st_e2.load_f32_raw(state_row(static_cast<const float*>(e1.p)), e2raw);
          e2_early = true;
        }
      }
      if (s_segstart[2] == Q && e1.p) {
        st_s2.load_at(static_cast<const T*>(pb.dstate) + bhc * P * pb.N + k.n0, off_st);
        s2_early = true;
      }
    }

    float offp[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) offp[a][r] = 0.f;
    for (int m = 0; m < k.nseg; ++m) {
      const int lo = s_segstart[m], hi = s_segstart[m + 1];
      const ERows esrc = e_src(h, m);
      if (m > 0) {
        // further segments (a sequence starts inside the chunk): stage their E here
        __syncthreads();
        bool staged = false;
        if constexpr (E2PF) {
          if (m == 1 && e2_early) {
            st_e2.convert_f32(e2raw);
            staged = true;
          }
        }
        if (!staged) load_e(st_e2, esrc);
        if (hi == Q && esrc.p) {
          if (!(m == 1 && s2_early)) st_s2.load_at(static_cast<const T*>(pb.dstate) + bhc * P * pb.N + k.n0, off_st);
#pragma unroll
          for (int kk = 0; kk < st_e2.IT; ++kk)
#pragma unroll
            for (int e = 0; e < st_e2.VEC; ++e) endp += vget<T>(st_s2.buf[kk], e) * vget<T>(st_e2.buf[kk], e);
        }
        st_e2.store(s_e, LDE);
        __syncthreads();
      }
      if (!esrc.p) continue;
      // both owned row tiles take each E fragment from one LDS read
      bool live[2];
      typename Mma<T>::frag af[2][KP];   // dy rows of tile I over p
      f32x4_t sv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int I = own[a];
        live[a] = !(16 * I + 15 < lo || 16 * I >= hi);
#pragma unroll
        for (int ks = 0; ks < KP; ++ks)
          af[a][ks] = Mma<T>::load_k(s_rows + (16 * I + r16) * LDP + kg * Mma<T>::KW + ks * Mma<T>::KSTEP);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * I + 4 * kg + r;
          sv[a][r] = (i >= lo && i < hi) ? s_v[i] : 0.f;
        }
      }
#pragma unroll
      for (int nt = 0; nt < NCT; ++nt) {
        typename Mma<T>::frag ef[KP];
#pragma unroll
        for (int ks = 0; ks < KP; ++ks) ef[ks] = load_kn<T>(s_e + 16 * nt, LDE, ks * Mma<T>::KSTEP);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          if (!live[a]) continue;
          const int I = own[a];
          f32x4_t y = zero4();
#pragma unroll
          for (int ks = 0; ks < KP; ++ks) y = Mma<T>::mma(af[a][ks], ef[ks], y);
          // C[i][n] in the accumulator layout
          const typename Mma<T>::rfrag cf = Mma<T>::rfrag_load_kn(s_c + 16 * I * LDK + 16 * nt, LDK);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float yv = y[r] * sv[a][r];
            acc[a][nt][r] += yv;
            offp[a][r] += yv * Elem<T>::to_f(static_cast<T>(cf[r]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const int64_t offd_base = (bhc * pb.ntg + k.ntile) * Q;
#pragma unroll
    for (int a = 0; a < 2; ++a)
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
      for (int q = 0; q < W; ++q) s += s_red[q];
      pb.endd[bhc * pb.ntg + k.ntile] = s;
    }
  }
  write_rows<T, Q, NTG>(pb, k, pb.dC, pb.dcp, acc, own);
}

// ----------------------------------------------------------------------------
// k_db
// ----------------------------------------------------------------------------
template <typename T, int Q, int P, int NTG>
__global__ __launch_bounds__((DbdcCfg<T, Q, P, NTG>::NTHR)) void k_db(Problem pb) {
  using Cf = DbdcCfg<T, Q, P, NTG>;
  constexpr int NTHR = Cf::NTHR, NCT = Cf::NCT, LDP = Cf::LDP, LDE = Cf::LDE;
  constexpr int KP = P / Mma<T>::KSTEP;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* s_a = reinterpret_cast<T*>(smem);      // slab phase: dCB^T rows [Q][LDA]
  T* s_k = s_a + Q * Cf::LDA;               //             C rows [KSL][LDK]
  T* s_rows = reinterpret_cast<T*>(smem);   // head phase: x rows [Q][LDP]
  T* s_e = s_rows + Q * LDP;                //             dS rows [P][LDE]
  float* s_v = reinterpret_cast<float*>(smem + Cf::R1);
  int* s_seg = reinterpret_cast<int*>(s_v + Q);
  int* s_segstart = s_seg + Q;

  const int tid = threadIdx.x, w = wave_id_s(), l = lane_id(), r16 = l & 15, kg = l >> 4;
  DbdcBlock k = dbdc_block<Q, NTHR>(pb, s_seg, s_segstart);
  k.n0 = k.ntile * NTG;
  const T* xg = static_cast<const T*>(pb.x);
  const T* Cg = static_cast<const T*>(pb.Cm);
  int own[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) own[a] = Cf::Split::col(w, a);

  f32x4_t acc[2][NCT];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nt = 0; nt < NCT; ++nt) acc[a][nt] = zero4();
  if (k.sl == 0)   // (uniform) the dCB part, once per tile
    dcb_slab_product<T, Q, P, NTG>(pb, k, acc, own, static_cast<const T*>(pb.dcbt) + k.bgc * Q * Q, Cg, false, s_a,
                                   s_k);

  // next head's rows: x, dS, and this thread's Acs / dt
  RowStage<T, Q, P, NTHR> st_x;
  RowStage<T, P, NTG, NTHR> st_s;
  float acs_n = 0.f, dt_n = 0.f, acs_end_n = 0.f;
  // per-lane offsets of the x rows and the dS rows of this tile: fixed for
  // the block, only the base moves from head to head
  const auto off_x = RowStage<T, Q, P, NTHR>::offsets(static_cast<uint32_t>(pb.H * P * sizeof(T)), pb.L - k.c * Q);
  const auto off_s = RowStage<T, P, NTG, NTHR>::offsets(static_cast<uint32_t>(pb.N * sizeof(T)), P);
  const T* x_c = xg + (static_cast<int64_t>(k.b) * pb.L + static_cast<int64_t>(k.c) * Q) * pb.H * P;
  auto load_head = [&](int hh) {
    const int h = k.g * pb.hpg + hh;
    const int64_t bhc = (static_cast<int64_t>(k.b) * pb.H + h) * pb.nc + k.c;
    st_x.load_at(x_c + h * P, off_x);
    st_s.load_at(static_cast<const T*>(pb.dstate) + bhc * P * pb.N + k.n0, off_s);
    if (tid < Q) {
      acs_n = pb.acs[bhc * Q + tid];
      dt_n = pb.dtc[bhc * Q + tid];
    }
    acs_end_n = pb.acs[bhc * Q + Q - 1];
  };
  constexpr bool PF = RowStage<T, Q, P, NTHR>::IT + RowStage<T, P, NTG, NTHR>::IT <= 16;
  __syncthreads();   // the slab phase is done with the LDS the head phase reuses
  if (PF && k.hh_lo < k.hh_hi) load_head(k.hh_lo);

  for (int hh = k.hh_lo; hh < k.hh_hi; ++hh) {
    if (!PF) load_head(hh);
    __syncthreads();
    st_x.store(s_rows, LDP);
    st_s.store(s_e, LDE);
    if (tid < Q) s_v[tid] = (tid >= k.lolast) ? Elem<T>::exp(acs_end_n - acs_n) * dt_n : 0.f;
    __syncthreads();
    if (PF && hh + 1 < k.hh_hi) load_head(hh + 1);
    // both owned column tiles take each dS fragment from one LDS read
    bool live[2];
    typename Mma<T>::frag af[2][KP];   // x rows of tile J over p
    f32x4_t wv[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int J = own[a];
      live[a] = 16 * J + 15 >= k.lolast;
#pragma unroll
      for (int ks = 0; ks < KP; ++ks)
        af[a][ks] = Mma<T>::load_k(s_rows + (16 * J + r16) * LDP + kg * Mma<T>::KW + ks * Mma<T>::KSTEP);
      wv[a] = *reinterpret_cast<const f32x4_t*>(s_v + 16 * J + 4 * kg);
    }
#pragma unroll
    for (int nt = 0; nt < NCT; ++nt) {
      typename Mma<T>::frag ef[KP];
#pragma unroll
      for (int ks = 0; ks < KP; ++ks) ef[ks] = load_kn<T>(s_e + 16 * nt, LDE, ks * Mma<T>::KSTEP);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        if (!live[a]) continue;
        f32x4_t u = zero4();
#pragma unroll
        for (int ks = 0; ks < KP; ++ks) u = Mma<T>::mma(af[a][ks], ef[ks], u);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[a][nt][r] += wv[a][r] * u[r];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  write_rows<T, Q, NTG>(pb, k, pb.dB, pb.dbp, acc, own);
}

// dstate tile width of k_dc / k_db
int group_ntile(int N, bool io_bf16) {
  (void)io_bf16;
  if (N % 128 == 0) return 128;
  if (N % 64 == 0) return 64;
  if (N % 32 == 0) return 32;
  return 16;
}

// dC or dB rows from the slices' slots, added in slice order: one thread per
// 4 consecutive columns of one row of one (batch, group, chunk, tile)
template <typename T, int Q, int NTG>
__global__ __launch_bounds__(256) void k_bd_out(Problem pb, const float* part, void* out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  constexpr int CV = NTG / 4;   // 4-column groups per row
  const int64_t ntile_all = static_cast<int64_t>(pb.B) * pb.G * pb.nc * pb.ntg;
  if (i >= ntile_all * Q * CV) return;
  const int cv = static_cast<int>(i % CV);
  const int row = static_cast<int>((i / CV) % Q);
  const int64_t bt = i / (static_cast<int64_t>(CV) * Q);   // (b, g, c, tile)
  const int ntile = static_cast<int>(bt % pb.ntg);
  const int64_t bgc = bt / pb.ntg;
  const int c = static_cast<int>(bgc % pb.nc);
  const int64_t bg = bgc / pb.nc;
  const int g = static_cast<int>(bg % pb.G), b = static_cast<int>(bg / pb.G);
  const int t = c * Q + row;
  if (t >= pb.L) return;
  const float* src = part + bt * pb.nslice_bd * Q * NTG + row * NTG + 4 * cv;
  f32x4_t v = *reinterpret_cast<const f32x4_t*>(src);
  for (int s = 1; s < pb.nslice_bd; ++s) {
    const f32x4_t u = *reinterpret_cast<const f32x4_t*>(src + static_cast<int64_t>(s) * Q * NTG);
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] += u[r];
  }
  store4f<T>(static_cast<T*>(out) + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + ntile * NTG + 4 * cv, v);
}

template <typename T, int Q, int P, int NTG>
static hipError_t launch_dbdc_t(const Problem& pb, hipStream_t s) {
  using Cf = DbdcCfg<T, Q, P, NTG>;
  const bool seq = pb.seq_idx != nullptr;
  hipError_t e = ensure_dynamic_lds(seq ? reinterpret_cast<const void*>(&k_dc<T, Q, P, NTG, true>)
                                        : reinterpret_cast<const void*>(&k_dc<T, Q, P, NTG, false>),
                                    Cf::LDS);
  if (e == hipSuccess) e = ensure_dynamic_lds(reinterpret_cast<const void*>(&k_db<T, Q, P, NTG>), Cf::LDS_DB);
  if (e != hipSuccess) return e;
  const int64_t tiles = static_cast<int64_t>(pb.B) * pb.G * pb.nc * pb.ntg, blocks = tiles * pb.nslice_bd;
  if (seq)
    hipLaunchKernelGGL((k_dc<T, Q, P, NTG, true>), dim3(static_cast<unsigned>(blocks)), dim3(Cf::NTHR), Cf::LDS, s, pb);
  else
    hipLaunchKernelGGL((k_dc<T, Q, P, NTG, false>), dim3(static_cast<unsigned>(blocks)), dim3(Cf::NTHR), Cf::LDS, s,
                       pb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_db<T, Q, P, NTG>), dim3(static_cast<unsigned>(blocks)), dim3(Cf::NTHR), Cf::LDS_DB, s, pb);
  e = hipGetLastError();
  if (e != hipSuccess || pb.nslice_bd == 1) return e;
  const int64_t nthr = tiles * Q * (NTG / 4);
  const dim3 grid(static_cast<unsigned>((nthr + 255) / 256));
  hipLaunchKernelGGL((k_bd_out<T, Q, NTG>), grid, dim3(256), 0, s, pb, static_cast<const float*>(pb.dcp), pb.dC);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_bd_out<T, Q, NTG>), grid, dim3(256), 0, s, pb, static_cast<const float*>(pb.dbp), pb.dB);
  return hipGetLastError();
}

template <typename T, int Q, int P>
static hipError_t launch_dbdc_qp(const Problem& pb, hipStream_t s) {
  switch (pb.N / pb.ntg) {
    case 128: return launch_dbdc_t<T, Q, P, 128>(pb, s);
    case 64: return launch_dbdc_t<T, Q, P, 64>(pb, s);
    case 32: return launch_dbdc_t<T, Q, P, 32>(pb, s);
    case 16: return launch_dbdc_t<T, Q, P, 16>(pb, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t launch_dbdc_any(const Problem& pb, hipStream_t s) {
#define SSD_DBDC_CASE(QQ, PP) \
  if (pb.Q == QQ && pb.P == PP) return launch_dbdc_qp<T, QQ, PP>(pb, s);
  if constexpr (sizeof(T) == 2) {
    SSD_BF16_SHAPES(SSD_DBDC_CASE)
  } else {
    SSD_F32_SHAPES(SSD_DBDC_CASE)
  }
#undef SSD_DBDC_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_dbdc(const Problem& pb, bool io_bf16, hipStream_t s) {
  return io_bf16 ? launch_dbdc_any<bf16_t>(pb, s) : launch_dbdc_any<float>(pb, s);
}

// LDS bytes of k_dc (the larger of the two) for a compiled shape; ~0 when not compiled.
size_t dbdc_lds_bytes(int Q, int P, int NTG, bool bf16) {
  size_t r = ~size_t(0);
#define SSD_DBDC_LDS(TT, QQ, PP)                                   \
  if (Q == QQ && P == PP) {                                        \
    if (NTG == 128) r = DbdcCfg<TT, QQ, PP, 128>::LDS;             \
    if (NTG == 64) r = DbdcCfg<TT, QQ, PP, 64>::LDS;               \
    if (NTG == 32) r = DbdcCfg<TT, QQ, PP, 32>::LDS;               \
    if (NTG == 16) r = DbdcCfg<TT, QQ, PP, 16>::LDS;               \
  }
#define SSD_DBDC_LDS_B(QQ, PP) if (bf16) { SSD_DBDC_LDS(bf16_t, QQ, PP) }
#define SSD_DBDC_LDS_F(QQ, PP) if (!bf16) { SSD_DBDC_LDS(float, QQ, PP) }
  SSD_BF16_SHAPES(SSD_DBDC_LDS_B)
  SSD_F32_SHAPES(SSD_DBDC_LDS_F)
#undef SSD_DBDC_LDS_B
#undef SSD_DBDC_LDS_F
#undef SSD_DBDC_LDS
  return r;
}

}  // namespace ssd
