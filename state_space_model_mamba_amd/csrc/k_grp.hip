// The intra-chunk group gradients of one (batch, group, chunk, 64-row slab,
// dstate tile): the chunk_scan_bwd_dC and chunk_state_bwd_db rows of the
// kernel table on the page "Deterministic bwd kernel for mamba2", together
// with the head-summed dCB that both need, in one pass over the group's
// heads.  Also the chunk's C B^T tiles for the head kernel (k_cb).
//
//   dCB[i,j] = sum_h W_h[i,j] (dy_h,i . x_h,j),  W_h[i,j] = exp(Acs_h,i - Acs_h,j) dt_h,j
//              (j <= i, same segment; else 0)
//   dC_i     = sum_j dCB[i,j] B_j  +  sum_h exp(Acs_h,i) dy_h,i E_h,seg(i)          (rows i of the slab)
//   dB_j     = sum_i dCB[i,j] C_i  +  sum_h w_h,j x_h,j dS_h                        (rows j of the slab)
//              w_j = exp(Acs_end - Acs_j) dt_j on the chunk's last segment, 0 before it
//   offd_h,i = exp(Acs_h,i) dy_h,i . (E_h,seg(i) C_i)   (this dstate tile's part, rows of the slab)
//   endd_h   = <dS_h, E_h,last>                         (this dstate tile's part, from the last slab)
// E is the state entering a row's segment: Hin for a segment that continues
// the previous chunk's sequence, the sequence's initial state otherwise.
// offd and endd are the off-diagonal and chunk-end ddA_cumsum terms; they go
// to slots owned by (batch, head, chunk, tile), summed later in tile order.
//
// A slab's rows need the dCB tiles of its row tiles (for dC) and of its
// column tiles (for dB).  A block forms exactly those: the tiles (I, J) with
// I in the slab and J <= I, then those with J in the slab and I past it --
// 4 T - 6 of the T (T + 1) / 2 causal tiles for T row tiles per chunk, the
// same count for every slab.  Each head adds its terms in ascending head
// order into fp32 accumulators; after the last head the dCB tiles are
// rounded to the I/O dtype into LDS, as dCB rows and as dCB^T rows, and
// multiplied by B and C.  There are no per-head slots and no atomics, and
// every output element has one writer.  The slabs of one (batch, group,
// chunk) are consecutive logical blocks, so their reads of the group's rows
// meet in one XCD's L2.
#include "ssd_problem.h"
#include "ssd_tiles.h"

namespace ssd {

template <typename T, int Q, int P, int NTG>
struct GrpCfg {
  static constexpr int T16 = Q / 16;              // row tiles per chunk
  static constexpr int SH = 4;                    // row tiles per slab
  static constexpr int SL = T16 / SH;             // slabs per chunk
  static constexpr int SR = SH * 16;              // rows per slab
  static constexpr int NOWN = 4 * T16 - 6;        // dCB tiles per block
  static constexpr int W = 8;
  static constexpr int NTHR = W * WAVE;
  static_assert(NTHR >= Q, "one thread per chunk position");
  static_assert(T16 % SH == 0, "whole slabs");
  static constexpr int KMAX = (NOWN + W - 1) / W; // dCB tiles per wave (at most)
  static constexpr int VEC = Vec16<T>::N;
  static constexpr int LDP = P + VEC;             // x / dy rows [i][p]
  static constexpr int NCT = NTG / 16;            // column tiles of the slab's outputs
  static constexpr int CPW = (NCT + 1) / 2;       // column tiles per wave (waves w and w + 4 share a row tile)
  static constexpr int LDE = kn_pitch<T>(NTG);    // E, dS, C, B rows [k][n]
  static constexpr int KSL = P < 32 ? P : 32;     // K slab of the dCB products
  static constexpr int LDA = Q + VEC;             // dCB rows, dCB^T rows [r][k]
  static constexpr int LDO = NTG + VEC;           // output rows [r][n]
  static constexpr int MK = P / Mma<T>::KSTEP;
  static_assert(KSL % Mma<T>::KSTEP == 0 && Q % KSL == 0 && SR % KSL == 0, "K slabs");
  // LDS regions: rows (x and dy rows in the head loop; dCB and dCB^T rows,
  // then the output rows, after it), E and dS (B and C K slabs after the
  // head loop), the slab's C rows, per-position vectors
  static constexpr size_t R_ROWS0 = size_t(2) * Q * LDP * sizeof(T);
  static constexpr size_t R_ROWS1 = size_t(2) * SR * LDA * sizeof(T);
  static constexpr size_t R_ROWS2 = size_t(2) * SR * LDO * sizeof(T);
  static constexpr size_t R_ROWS_MAX = R_ROWS0 > R_ROWS1 ? (R_ROWS0 > R_ROWS2 ? R_ROWS0 : R_ROWS2)
                                                         : (R_ROWS1 > R_ROWS2 ? R_ROWS1 : R_ROWS2);
  static constexpr size_t R_ROWS = (R_ROWS_MAX + 15) / 16 * 16;
  static constexpr size_t R_ES = size_t(2) * P * LDE * sizeof(T);
  static_assert(KSL <= P, "the K slabs fit the E / dS region");
  static constexpr size_t R_C = (size_t(SR) * LDE * sizeof(T) + 15) / 16 * 16;
  // acs, dt, er, ev, wv (Q floats each), seg (Q ints), segment starts (Q + 4
  // ints), offd partials (2 SR floats), per-wave sums (W + 8 floats)
  static constexpr size_t VEC_BYTES = size_t(6) * Q * 4 + size_t(Q + 4) * 4 + size_t(2) * SR * 4 + size_t(W + 8) * 4;
  static constexpr size_t LDS = R_ROWS + R_ES + R_C + VEC_BYTES;
};

// Tile t (0 <= t < 4 T - 6) of the block owning the slab of row tiles
// [I0, I0 + 4): first the slab's rows (row I0 + r holds tiles J = 0 ..
// I0 + r, starting at index r I0 + r (r + 1) / 2), then the column tiles of
// the slab below it (J = I0 + t' % 4, I = I0 + 4 + t' / 4).
__device__ __forceinline__ void grp_tile(int t, int I0, int& I, int& J) {
  const int na = 4 * I0 + 10;
  if (t < na) {
    const int r = t >= 3 * I0 + 6 ? 3 : (t >= 2 * I0 + 3 ? 2 : (t >= I0 + 1 ? 1 : 0));
    I = I0 + r;
    J = t - (r * I0 + r * (r + 1) / 2);
  } else {
    const int u = t - na;
    J = I0 + (u & 3);
    I = I0 + 4 + (u >> 2);
  }
}

template <typename T, int Q, int P, int NTG>
__global__ __launch_bounds__((GrpCfg<T, Q, P, NTG>::NTHR)) void k_grp(Problem pb) {
  using Cf = GrpCfg<T, Q, P, NTG>;
  constexpr int W = Cf::W, NTHR = Cf::NTHR, VEC = Cf::VEC, LDP = Cf::LDP, LDE = Cf::LDE, LDA = Cf::LDA;
  constexpr int SR = Cf::SR, SH = Cf::SH, SL = Cf::SL, NCT = Cf::NCT, CPW = Cf::CPW, MK = Cf::MK;
  constexpr int KS = Mma<T>::KSTEP, KW = Mma<T>::KW, KSL = Cf::KSL, LDO = Cf::LDO;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* const s_x = reinterpret_cast<T*>(smem);        // head loop: x rows [Q][LDP]
  T* const s_dy = s_x + Q * LDP;                     //            dy rows [Q][LDP]
  T* const s_ra = reinterpret_cast<T*>(smem);       // products:  dCB rows of the slab [SR][LDA]
  T* const s_rb = s_ra + SR * LDA;                   //            dCB^T rows of the slab [SR][LDA]
  T* const s_oc = reinterpret_cast<T*>(smem);       // output:    dC rows [SR][LDO]
  T* const s_ob = s_oc + SR * LDO;                   //            dB rows [SR][LDO]
  T* const s_e = reinterpret_cast<T*>(smem + Cf::R_ROWS);   // E rows [P][LDE]
  T* const s_s = s_e + P * LDE;                              // dS rows [P][LDE]
  T* const s_kb = s_e;                                       // products: B rows of a K slab [KSL][LDE]
  T* const s_kc = s_e + KSL * LDE;                           //           C rows of a K slab
  T* const s_c = reinterpret_cast<T*>(smem + Cf::R_ROWS + Cf::R_ES);   // C rows of the slab [SR][LDE]
  float* const s_acs = reinterpret_cast<float*>(smem + Cf::R_ROWS + Cf::R_ES + Cf::R_C);
  float* const s_dt = s_acs + Q;
  float* const s_er = s_dt + Q;
  float* const s_ev = s_er + Q;
  float* const s_wv = s_ev + Q;
  int* const s_seg = reinterpret_cast<int*>(s_wv + Q);
  int* const s_segstart = s_seg + Q;                         // Q + 4 entries
  float* const s_offp = reinterpret_cast<float*>(s_segstart + Q + 4);   // [2][SR]
  float* const s_red = s_offp + 2 * SR;

  // block -> (batch, group, chunk, slab, dstate tile)
  const int64_t total = static_cast<int64_t>(pb.B) * pb.G * pb.nc * SL * pb.ntg;
  const int64_t lb = xcd_logical_block(blockIdx.x, total);
  const int ntile = static_cast<int>(lb % pb.ntg);
  int64_t rest = lb / pb.ntg;
  const int rq = static_cast<int>(rest % SL);
  rest /= SL;
  const int c = static_cast<int>(rest % pb.nc);
  rest /= pb.nc;
  const int g = static_cast<int>(rest % pb.G), b = static_cast<int>(rest / pb.G);
  const int n0 = ntile * NTG, I0 = SH * rq, R0 = 16 * I0;
  const int tid = threadIdx.x, w = wave_id_s(), l = lane_id(), r16 = l & 15, kg = l >> 4;
  const int rt = w & 3;         // the wave's row tile of the slab (outputs)
  const int chalf = w >> 2;     // ... and its column tiles chalf, chalf + 2, ...
  const int64_t bc = static_cast<int64_t>(b) * pb.nc + c;
  const T* xg = static_cast<const T*>(pb.x);
  const T* dyg = static_cast<const T*>(pb.dy);
  const T* Bg = static_cast<const T*>(pb.Bm);
  const T* Cg = static_cast<const T*>(pb.Cm);

  // the chunk's segments
  const int nstart = pb.cinfo[bc * CINFO + 0];
  const int seqbase = pb.cinfo[bc * CINFO + 3];
  if (tid < Q) s_seg[tid] = pb.segpos[bc * Q + tid];
  if (tid == 0) s_segstart[0] = 0;
  __syncthreads();
  const int start0 = seg_rank(s_seg[0]);
  const int nseg = nstart + 1 - start0;
  const int lolast = seg_lo(s_seg[Q - 1]);
  if (tid < Q && tid > 0 && seg_lo(s_seg[tid]) == tid) s_segstart[seg_rank(s_seg[tid]) - start0] = tid;
  if (tid == 0) s_segstart[nseg] = Q;
  // A chunk without sequence starts after position 0 has one segment and a
  // non-increasing Acs: there the decay of an off-diagonal tile is
  // er_i exp(Acs_{16 I} - Acs_j), er_i = exp(Acs_i - Acs_{16 floor(i / 16)}), both factors <= 1.
  const bool uniform = __builtin_amdgcn_readfirstlane(lolast) == 0;

  // the slab's C rows (this dstate tile), for the offd row dots
  auto bc_row = [&](const T* base, int k0) {
    return [=, &pb](int i) -> const T* {
      const int t = c * Q + k0 + i;
      return t < pb.L ? base + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + n0 : nullptr;
    };
  };
  {
    RowStage<T, SR, NTG, NTHR> st_cm;
    st_cm.load(bc_row(Cg, R0));
    st_cm.store(s_c, LDE);
  }
  __syncthreads();   // (segment starts and C rows visible)

  // entering state of segment m of head h: Hin (I/O dtype) when the segment
  // continues the chunk's sequence, h0[s] (fp32) when it starts sequence s,
  // none (zero) when no initial state is given
  struct ESrc {
    const void* p;
    bool f32;
  };
  auto e_src = [&](int h, int m) -> ESrc {
    const int64_t bhc = (static_cast<int64_t>(b) * pb.H + h) * pb.nc + c;
    const int rank = seg_rank(s_seg[s_segstart[m]]);
    if (rank == 0) return {static_cast<const T*>(pb.hin) + bhc * P * pb.N, false};
    if (!pb.h0) return {nullptr, true};
    const int s = clamp_seq(seqbase + rank - 1, pb.nseqs);
    return {pb.h0 + (static_cast<int64_t>(s) * pb.H + h) * P * pb.N, true};
  };
  auto state_row = [&](const auto* base) {
    return [=, &pb](int p) { return base + static_cast<int64_t>(p) * pb.N + n0; };
  };
  auto zero_row = [](int) -> const T* { return nullptr; };
  auto load_e = [&](RowStage<T, P, NTG, NTHR>& st, ESrc e) {
    if (!e.p)
      st.load(zero_row);
    else if (!e.f32)
      st.load(state_row(static_cast<const T*>(e.p)));
    else
      st.load_from_f32(state_row(static_cast<const float*>(e.p)));
  };

  // The next head's rows, requested while the current head runs: x rows
  // [0, R0 + SR) then dy rows [R0, Q) (Q + SR rows), segment 0's entering
  // state when it is Hin, dS, and the per-position Acs / dt.  Every request
  // is unconditional -- row indices past L are clamped and those rows zeroed
  // when stored -- so no branch join waits on a load in flight.
  const int xhi = R0 + SR;
  constexpr int CV = P / VEC, NRV = (Q + SR) * CV, RIT = (NRV + NTHR - 1) / NTHR;
  constexpr int EV = P * (NTG / VEC), EIT = (EV + NTHR - 1) / NTHR;
  // segment 0 continues the chunk's sequence (its E is Hin) in almost every chunk
  const bool e0_hin = start0 == 0;
  struct HeadIn {
    uint4 rbuf[RIT], ebuf[EIT], sbuf[EIT];
    uint32_t rok;   // bit k: row vector k lies before L
    float acs, dt, acs_end;
  };
  auto row_of = [&](int v, int& i, int& cv, bool& isx) {
    const int r = v / CV;
    cv = v % CV;
    isx = r < xhi;
    i = isx ? r : R0 + (r - xhi);
  };
  auto load_head = [&](int hh, HeadIn& in) {
    const int h = g * pb.hpg + hh;
    const int64_t bhc = (static_cast<int64_t>(b) * pb.H + h) * pb.nc + c;
    in.rok = 0;
#pragma unroll
    for (int k = 0; k < RIT; ++k) {
      int i, cv;
      bool isx;
      row_of(min(tid + k * NTHR, NRV - 1), i, cv, isx);
      const int t = c * Q + i;
      const int tt = min(t, pb.L - 1);
      const T* base = isx ? xg : dyg;
      in.rbuf[k] = ld_global16(base + ((static_cast<int64_t>(b) * pb.L + tt) * pb.H + h) * P + cv * VEC);
      in.rok |= (t < pb.L ? 1u : 0u) << k;
    }
    const T* hin = static_cast<const T*>(pb.hin) + bhc * P * pb.N + n0;
    const T* ds = static_cast<const T*>(pb.dstate) + bhc * P * pb.N + n0;
#pragma unroll
    for (int k = 0; k < EIT; ++k) {
      const int v = min(tid + k * NTHR, EV - 1);
      const int64_t off = static_cast<int64_t>(v / (NTG / VEC)) * pb.N + (v % (NTG / VEC)) * VEC;
      in.ebuf[k] = ld_global16(hin + off);
      in.sbuf[k] = ld_global16(ds + off);
    }
    in.acs = pb.acs[bhc * Q + min(tid, Q - 1)];
    in.dt = pb.dtc[bhc * Q + min(tid, Q - 1)];
    in.acs_end = pb.acs[bhc * Q + Q - 1];
  };
  auto store_head = [&](int h, const HeadIn& in) {
#pragma unroll
    for (int k = 0; k < RIT; ++k) {
      const int v = tid + k * NTHR;
      if (NRV % NTHR == 0 || v < NRV) {
        int i, cv;
        bool isx;
        row_of(v, i, cv, isx);
        *reinterpret_cast<uint4*>((isx ? s_x : s_dy) + i * LDP + cv * VEC) = ((in.rok >> k) & 1u) ? in.rbuf[k] : zero_u4();
      }
    }
#pragma unroll
    for (int k = 0; k < EIT; ++k) {
      const int v = tid + k * NTHR;
      if (EV % NTHR == 0 || v < EV) {
        const int p = v / (NTG / VEC), n = (v % (NTG / VEC)) * VEC;
        *reinterpret_cast<uint4*>(s_e + p * LDE + n) = e0_hin ? in.ebuf[k] : zero_u4();
        *reinterpret_cast<uint4*>(s_s + p * LDE + n) = in.sbuf[k];
      }
    }
    if (!e0_hin) {   // (uniform; a sequence starts at the chunk's first position) its initial state, if any
      const ESrc es = e_src(h, 0);
      if (es.p) {
        RowStage<T, P, NTG, NTHR> st_e0;
        load_e(st_e0, es);
        st_e0.store(s_e, LDE);
      }
    }
  };

  f32x4_t dcb[Cf::KMAX], dca[CPW], dba[CPW];
#pragma unroll
  for (int k = 0; k < Cf::KMAX; ++k) dcb[k] = zero4();
#pragma unroll
  for (int q = 0; q < CPW; ++q) dca[q] = dba[q] = zero4();
  // One head of the group: its inputs (requested PFD heads earlier) go to
  // LDS, then the inputs of the head PFD places on are requested into the
  // same registers while this one is computed.  (Two register sets in turn,
  // PFD = 2, measured slower than one: the loop is not bound by the loads'
  // latency.)
  constexpr int PFD = 1;
  auto run_head = [&](int hh, HeadIn& in) {
    const int h = g * pb.hpg + hh;
    const int64_t bhc = (static_cast<int64_t>(b) * pb.H + h) * pb.nc + c;
    __syncthreads();   // the previous head's LDS reads are done
    store_head(h, in);
    {
      const float acs_tile0 = __shfl(in.acs, l & ~15, WAVE);
      if (tid < Q) {
        s_acs[tid] = in.acs;
        s_dt[tid] = in.dt;
        s_er[tid] = uniform ? Elem<T>::exp(in.acs - acs_tile0) : 0.f;
        s_ev[tid] = Elem<T>::exp(in.acs);   // (Acs <= 0: restarted at every segment start)
        s_wv[tid] = tid >= lolast ? Elem<T>::exp(in.acs_end - in.acs) * in.dt : 0.f;
      }
    }
    __syncthreads();
    if (hh + PFD < pb.hpg) load_head(hh + PFD, in);

    // per-head LDS bases and wave index: keeps the compiler from hoisting every
    // tile's addresses and masks out of the head loop (they would hold registers)
    const int oz = opaque_zero();
    const T* const lx = s_x + oz;
    const T* const ldy = s_dy + oz;
    const T* const le = s_e + oz;
    const T* const ls = s_s + oz;
    const T* const lc = s_c + oz;
    const float* const lacs = s_acs + oz;
    const float* const ldt = s_dt + oz;
    const float* const ler = s_er + oz;
    const float* const lev = s_ev + oz;
    const float* const lwv = s_wv + oz;
    const int* const lseg = s_seg + oz;
    const int wz = w + oz;
    // ---- dCB: the block's tiles, W o (dy x^T), wave w taking tiles w, w + W, ...
#pragma unroll
    for (int k = 0; k < Cf::KMAX; ++k) {
      const int t = wz + W * k;
      if (Cf::NOWN % W == 0 || t < Cf::NOWN) {   // (wave-uniform)
        int I, J;
        grp_tile(t, I0, I, J);
        typename Mma<T>::frag ma[MK], mb[MK];
#pragma unroll
        for (int s = 0; s < MK; ++s) {
          ma[s] = Mma<T>::load_k(ldy + (16 * I + r16) * LDP + kg * KW + s * KS);
          mb[s] = Mma<T>::load_k(lx + (16 * J + r16) * LDP + kg * KW + s * KS);
        }
        f32x4_t m = zero4();
#pragma unroll
        for (int s = 0; s < MK; ++s) m = Mma<T>::mma(ma[s], mb[s], m);
        const int j = 16 * J + r16;
        const float aj = lacs[j], dtj = ldt[j];
        f32x4_t e4;   // exp(Acs_i - Acs_j) dt_j where (i, j) is causal and in one segment, else 0
        if (uniform && I != J) {
          const float ec = Elem<T>::exp(lacs[16 * I] - aj) * dtj;
          const f32x4_t er4 = *reinterpret_cast<const f32x4_t*>(ler + 16 * I + 4 * kg);
#pragma unroll
          for (int r = 0; r < 4; ++r) e4[r] = er4[r] * ec;
        } else {
          const f32x4_t ai4 = *reinterpret_cast<const f32x4_t*>(lacs + 16 * I + 4 * kg);
          const int4 sg4 = *reinterpret_cast<const int4*>(lseg + 16 * I + 4 * kg);
          const int loj = seg_lo(lseg[j]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * I + 4 * kg + r;
            const int sgi = r == 0 ? sg4.x : (r == 1 ? sg4.y : (r == 2 ? sg4.z : sg4.w));
            const bool ok = (j <= i) & (seg_lo(sgi) == loj);
            // exp of a non-positive argument only; masked entries use a zero argument
            const float e = Elem<T>::exp(ok ? ai4[r] - aj : 0.f);
            e4[r] = ok ? e * dtj : 0.f;
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) dcb[k][r] += e4[r] * m[r];
      }
      // one tile at a time: keeps the next tiles' operands out of this tile's registers
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- dC: exp(Acs_i) dy_i E_seg(i), segment by segment, and the offd row dots
    const int I = I0 + rt;
    float offp[4] = {0.f, 0.f, 0.f, 0.f};
    for (int m = 0; m < nseg; ++m) {
      const int lo = s_segstart[m], hi = s_segstart[m + 1];
      if (hi <= R0 || lo >= R0 + SR) continue;   // (uniform) the segment misses the slab
      const ESrc es = e_src(h, m);
      if (m > 0) {
        // a sequence starts inside the chunk: stage this segment's E
        RowStage<T, P, NTG, NTHR> st_e2;
        load_e(st_e2, es);
        __syncthreads();   // the previous segment's E is read
        st_e2.store(s_e, LDE);
        __syncthreads();
      }
      if (!es.p) continue;                        // (uniform) no entering state
      if (16 * I + 15 < lo || 16 * I >= hi) continue;   // (wave-uniform)
      typename Mma<T>::frag af[MK];   // dy rows of tile I over p
#pragma unroll
      for (int s = 0; s < MK; ++s) af[s] = Mma<T>::load_k(ldy + (16 * I + r16) * LDP + kg * KW + s * KS);
      f32x4_t sv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * kg + r;
        sv[r] = (i >= lo && i < hi) ? lev[i] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < CPW; ++q) {
        const int ct = chalf + 2 * q;
        if (NCT % 2 == 0 || ct < NCT) {
          f32x4_t y = zero4();
#pragma unroll
          for (int s = 0; s < MK; ++s) y = Mma<T>::mma(af[s], load_kn<T>(le + 16 * ct, LDE, s * KS), y);
          // C[i][n] of the slab in the accumulator layout
          const typename Mma<T>::rfrag cf = Mma<T>::rfrag_load_kn(lc + 16 * rt * LDE + 16 * ct, LDE);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float yv = y[r] * sv[r];
            dca[q][r] += yv;
            offp[r] += yv * Elem<T>::to_f(static_cast<T>(cf[r]));
          }
        }
      }
    }

    // ---- dB: w_j x_j dS over the chunk's last segment
    if (16 * I + 15 >= lolast) {   // (wave-uniform)
      typename Mma<T>::frag af[MK];   // x rows of tile I over p
#pragma unroll
      for (int s = 0; s < MK; ++s) af[s] = Mma<T>::load_k(lx + (16 * I + r16) * LDP + kg * KW + s * KS);
      const f32x4_t wv = *reinterpret_cast<const f32x4_t*>(lwv + 16 * I + 4 * kg);
#pragma unroll
      for (int q = 0; q < CPW; ++q) {
        const int ct = chalf + 2 * q;
        if (NCT % 2 == 0 || ct < NCT) {
          f32x4_t u = zero4();
#pragma unroll
          for (int s = 0; s < MK; ++s) u = Mma<T>::mma(af[s], load_kn<T>(ls + 16 * ct, LDE, s * KS), u);
#pragma unroll
          for (int r = 0; r < 4; ++r) dba[q][r] += wv[r] * u[r];
        }
      }
    }

    // ---- offd of the slab's rows: each lane row's sum over the 16 columns of
    // its tiles, the two waves of a row tile added in wave order; endd from
    // the last slab: <dS, E_last> over this dstate tile
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = sum16(offp[r]);
      if (r16 == 0) s_offp[chalf * SR + 16 * rt + 4 * kg + r] = v;
    }
    if (rq == SL - 1) {   // (uniform) the last segment's E is in s_e (it touches the last slab)
      float endp = 0.f;
      if (e_src(h, nseg - 1).p) {
        for (int v = tid; v < P * (NTG / VEC); v += NTHR) {
          const int p = v / (NTG / VEC), n = (v % (NTG / VEC)) * VEC;
          const uint4 sv4 = *reinterpret_cast<const uint4*>(ls + p * LDE + n);
          const uint4 ev4 = *reinterpret_cast<const uint4*>(le + p * LDE + n);
#pragma unroll
          for (int e = 0; e < VEC; ++e) endp += vget<T>(sv4, e) * vget<T>(ev4, e);
        }
      }
      endp = wave_sum(endp);
      if (l == 0) s_red[w] = endp;
    }
    __syncthreads();
    if (tid < SR)   // every row of the slab (rows past L are zeros: the head kernel's cumsum reads them)
      pb.offd[(bhc * pb.ntg + ntile) * Q + R0 + tid] = s_offp[tid] + s_offp[SR + tid];
    if (rq == SL - 1 && tid == 0) {
      float sum = 0.f;
      for (int q = 0; q < W; ++q) sum += s_red[q];
      pb.endd[bhc * pb.ntg + ntile] = sum;
    }
  };

  if constexpr (PFD == 1) {
    HeadIn in0;
    load_head(0, in0);
    for (int hh = 0; hh < pb.hpg; ++hh) run_head(hh, in0);
  } else {   // two register sets of inputs in flight, taken in turn
    HeadIn in0, in1;
    load_head(0, in0);
    if (pb.hpg > 1) load_head(1, in1);
    for (int hh = 0; hh < pb.hpg; hh += 2) {
      run_head(hh, in0);
      if (hh + 1 < pb.hpg) run_head(hh + 1, in1);
    }
  }

  // ---- the dCB products: the tiles, rounded to the I/O dtype, as the slab's
  // dCB rows (for dC) and dCB^T rows (for dB); entries no tile covers are zero
  __syncthreads();   // every wave is done with the x / dy rows
  for (int v = tid; v < 2 * SR * LDA / VEC; v += NTHR) *reinterpret_cast<uint4*>(s_ra + v * VEC) = zero_u4();
  __syncthreads();
#pragma unroll
  for (int k = 0; k < Cf::KMAX; ++k) {
    const int t = w + W * k;
    if (Cf::NOWN % W == 0 || t < Cf::NOWN) {
      int I, J;
      grp_tile(t, I0, I, J);
      if (I < I0 + SH) {   // a row tile of the slab: dCB[i][16 J + r16]
#pragma unroll
        for (int r = 0; r < 4; ++r) s_ra[(16 * (I - I0) + 4 * kg + r) * LDA + 16 * J + r16] = Elem<T>::from_f(dcb[k][r]);
      }
      if (J >= I0 && J < I0 + SH)   // a column tile of the slab: dCB^T[j][16 I + 4 kg .. + 3]
        store4f<T>(s_rb + (16 * (J - I0) + r16) * LDA + 16 * I + 4 * kg, dcb[k]);
    }
  }
  // dC += dCB[slab rows][j] B_j over j < R0 + SR; dB += dCB^T[slab rows][i] C_i over i >= R0
  {
    RowStage<T, KSL, NTG, NTHR> st_kb, st_kc;
    constexpr int KK = KSL / KS;
    for (int k0 = 0; k0 < Q; k0 += KSL) {
      const bool for_c = k0 < R0 + SR, for_b = k0 >= R0;   // (uniform)
      if (for_c) st_kb.load(bc_row(Bg, k0));
      if (for_b) st_kc.load(bc_row(Cg, k0));
      __syncthreads();   // the tiles are in LDS (first slab) / the previous slab is read
      if (for_c) st_kb.store(s_kb, LDE);
      if (for_b) st_kc.store(s_kc, LDE);
      __syncthreads();
      if (for_c) {
        typename Mma<T>::frag af[KK];
#pragma unroll
        for (int s = 0; s < KK; ++s) af[s] = Mma<T>::load_k(s_ra + (16 * rt + r16) * LDA + k0 + kg * KW + s * KS);
#pragma unroll
        for (int q = 0; q < CPW; ++q) {
          const int ct = chalf + 2 * q;
          if (NCT % 2 == 0 || ct < NCT) {
#pragma unroll
            for (int s = 0; s < KK; ++s) dca[q] = Mma<T>::mma(af[s], load_kn<T>(s_kb + 16 * ct, LDE, s * KS), dca[q]);
          }
        }
      }
      if (for_b) {
        typename Mma<T>::frag af[KK];
#pragma unroll
        for (int s = 0; s < KK; ++s) af[s] = Mma<T>::load_k(s_rb + (16 * rt + r16) * LDA + k0 + kg * KW + s * KS);
#pragma unroll
        for (int q = 0; q < CPW; ++q) {
          const int ct = chalf + 2 * q;
          if (NCT % 2 == 0 || ct < NCT) {
#pragma unroll
            for (int s = 0; s < KK; ++s) dba[q] = Mma<T>::mma(af[s], load_kn<T>(s_kc + 16 * ct, LDE, s * KS), dba[q]);
          }
        }
      }
    }
  }

  // ---- dC and dB rows of the slab through LDS, out as 16-byte pieces
  __syncthreads();   // the dCB rows are read
#pragma unroll
  for (int q = 0; q < CPW; ++q) {
    const int ct = chalf + 2 * q;
    if (NCT % 2 == 0 || ct < NCT) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s_oc[(16 * rt + 4 * kg + r) * LDO + 16 * ct + r16] = Elem<T>::from_f(dca[q][r]);
        s_ob[(16 * rt + 4 * kg + r) * LDO + 16 * ct + r16] = Elem<T>::from_f(dba[q][r]);
      }
    }
  }
  __syncthreads();
  constexpr int OV = NTG / VEC;
  for (int v = tid; v < SR * OV; v += NTHR) {
    const int row = v / OV, cv = v % OV, t = c * Q + R0 + row;
    if (t >= pb.L) continue;
    const int64_t off = ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + n0 + cv * VEC;
    *reinterpret_cast<uint4*>(static_cast<T*>(pb.dC) + off) = *reinterpret_cast<const uint4*>(s_oc + row * LDO + cv * VEC);
    *reinterpret_cast<uint4*>(static_cast<T*>(pb.dB) + off) = *reinterpret_cast<const uint4*>(s_ob + row * LDO + cv * VEC);
  }
}

// ----------------------------------------------------------------------------
// k_cb: C B^T of each (batch, group, chunk) over the causal tiles, for the
// head kernel: fp32, in that kernel's causal split (wave, tile) order and
// accumulator lane layout, one 16-byte piece per lane and tile.
// ----------------------------------------------------------------------------
template <typename T, int Q>
struct CbCfg {
  static constexpr int T16 = Q / 16;
  static constexpr int W = causal_waves<Q>();   // the head kernel's split
  using Split = CausalSplit<T16, W>;
  static constexpr int NTHR = W * WAVE;
  static constexpr int VEC = Vec16<T>::N;
  static constexpr int NOWN = Split::NOWN;
  static constexpr int NS = sizeof(T) == 2 ? 32 : 16;   // dstate slab of the product
  static constexpr int NSL = 4;                         // slabs in flight
  static constexpr int LDN = NS + VEC;
  static constexpr size_t LDS = size_t(2) * Q * LDN * sizeof(T);
};

template <typename T, int Q>
__global__ __launch_bounds__((CbCfg<T, Q>::NTHR)) void k_cb(Problem pb) {
  using Cf = CbCfg<T, Q>;
  constexpr int NTHR = Cf::NTHR, NS = Cf::NS, NSL = Cf::NSL, LDN = Cf::LDN;
  __shared__ __attribute__((aligned(16))) T s_ck[Q * LDN];
  __shared__ __attribute__((aligned(16))) T s_bk[Q * LDN];
  const int64_t total = static_cast<int64_t>(pb.B) * pb.G * pb.nc;
  const int64_t lb = xcd_logical_block(blockIdx.x, total);
  const int c = static_cast<int>(lb % pb.nc);
  const int64_t bg = lb / pb.nc;
  const int g = static_cast<int>(bg % pb.G), b = static_cast<int>(bg / pb.G);
  const int w = wave_id_s(), l = lane_id();
  const int64_t bgc = (static_cast<int64_t>(b) * pb.G + g) * pb.nc + c;
  const T* Bg = static_cast<const T*>(pb.Bm);
  const T* Cg = static_cast<const T*>(pb.Cm);
  auto bc_row = [&](const T* base, int n0) {
    return [=, &pb](int i) -> const T* {
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

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------
// dstate tile width of k_grp (and of the offd / endd slots): up to 128
// columns in bf16, 64 in fp32 (whose rows take twice the LDS)
int grp_ntile(int N, bool io_bf16) {
  if (io_bf16 && N % 128 == 0) return 128;
  if (N % 64 == 0) return 64;
  if (N % 32 == 0) return 32;
  return 16;
}

template <typename T, int Q, int P, int NTG>
static hipError_t launch_grp_t(const Problem& pb, hipStream_t s) {
  using Cf = GrpCfg<T, Q, P, NTG>;
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&k_grp<T, Q, P, NTG>), Cf::LDS);
  if (e != hipSuccess) return e;
  const int64_t blocks = static_cast<int64_t>(pb.B) * pb.G * pb.nc * Cf::SL * pb.ntg;
  hipLaunchKernelGGL((k_grp<T, Q, P, NTG>), dim3(static_cast<unsigned>(blocks)), dim3(Cf::NTHR), Cf::LDS, s, pb);
  return hipGetLastError();
}

template <typename T, int Q, int P>
static hipError_t launch_grp_qp(const Problem& pb, hipStream_t s) {
  switch (pb.N / pb.ntg) {
    case 128: return launch_grp_t<T, Q, P, 128>(pb, s);
    case 64: return launch_grp_t<T, Q, P, 64>(pb, s);
    case 32: return launch_grp_t<T, Q, P, 32>(pb, s);
    case 16: return launch_grp_t<T, Q, P, 16>(pb, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t launch_grp_any(const Problem& pb, hipStream_t s) {
#define SSD_GRP_CASE(QQ, PP) \
  if (pb.Q == QQ && pb.P == PP) return launch_grp_qp<T, QQ, PP>(pb, s);
  if constexpr (sizeof(T) == 2) {
    SSD_BF16_SHAPES(SSD_GRP_CASE)
  } else {
    SSD_F32_SHAPES(SSD_GRP_CASE)
  }
#undef SSD_GRP_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_grp(const Problem& pb, bool io_bf16, hipStream_t s) {
  return io_bf16 ? launch_grp_any<bf16_t>(pb, s) : launch_grp_any<float>(pb, s);
}

template <typename T>
static hipError_t launch_cb_any(const Problem& pb, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(pb.B) * pb.G * pb.nc;
  switch (pb.Q) {
    case 64: hipLaunchKernelGGL((k_cb<T, 64>), dim3(static_cast<unsigned>(blocks)), dim3(CbCfg<T, 64>::NTHR), 0, s, pb); break;
    case 128: hipLaunchKernelGGL((k_cb<T, 128>), dim3(static_cast<unsigned>(blocks)), dim3(CbCfg<T, 128>::NTHR), 0, s, pb); break;
    case 256: hipLaunchKernelGGL((k_cb<T, 256>), dim3(static_cast<unsigned>(blocks)), dim3(CbCfg<T, 256>::NTHR), 0, s, pb); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_cb(const Problem& pb, bool io_bf16, hipStream_t s) {
  return io_bf16 ? launch_cb_any<bf16_t>(pb, s) : launch_cb_any<float>(pb, s);
}

// LDS bytes of k_grp for a compiled shape; ~0 when not compiled.
size_t grp_lds_bytes(int Q, int P, int NTG, bool bf16) {
  size_t r = ~size_t(0);
#define SSD_GRP_LDS(TT, QQ, PP)                          \
  if (Q == QQ && P == PP) {                              \
    if (NTG == 128) r = GrpCfg<TT, QQ, PP, 128>::LDS;    \
    if (NTG == 64) r = GrpCfg<TT, QQ, PP, 64>::LDS;      \
    if (NTG == 32) r = GrpCfg<TT, QQ, PP, 32>::LDS;      \
    if (NTG == 16) r = GrpCfg<TT, QQ, PP, 16>::LDS;      \
  }
#define SSD_GRP_LDS_B(QQ, PP) if (bf16) { SSD_GRP_LDS(bf16_t, QQ, PP) }
#define SSD_GRP_LDS_F(QQ, PP) if (!bf16) { SSD_GRP_LDS(float, QQ, PP) }
  SSD_BF16_SHAPES(SSD_GRP_LDS_B)
  SSD_F32_SHAPES(SSD_GRP_LDS_F)
#undef SSD_GRP_LDS_B
#undef SSD_GRP_LDS_F
#undef SSD_GRP_LDS
  return r;
}

}  // namespace ssd
