// Head kernel: everything of one (batch, head, chunk) that needs no head sum
// -- combined_bwd_dx (dx), chunk_scan_bwd_ddAcs + chunk_state_bwd_ddAcs
// (ddA_cumsum) and chunk_cumsum_bwd (ddt and the dA partial) in the kernel
// list of the page "Deterministic bwd kernel for mamba2".
//
//   CB        = C B^T                         (Q x Q causal, from the dCB kernel)
//   G[i,j]    = CB[i,j] exp(Acs_i - Acs_j)    (j <= i, same segment; else 0)
//   M         = dy x^T                        (MFMA over P)
//   Z^T       = dS B^T                        (P x Q, MFMA over N)
//   dx_j      = dt_j sum_i G[i,j] dy_i  +  w_j Z_j  +  D dy_j
//               (the first product takes the G tiles straight from the
//                accumulator registers as the MFMA B operand)
//   ddt_j     = sum_i G[i,j] M[i,j]  +  e_j x_j . Z_j  +  A da_j
//   V[i,j]    = G[i,j] M[i,j] dt_j
//   da_k      = sum_{i >= k > j} V[i,j]                 (intra-chunk decays)
//             + sum_{i >= k, same segment} ddAcs_i      (every other Acs use)
//   ddAcs_i   = offd_i - s_i  (+ at i = Q-1: sum_j s_j + exp(Acs_end) endd)
//   s_j       = w_j x_j . Z_j,   w_j = e_j dt_j,  e_j = exp(Acs_end - Acs_j) on the last segment
//
// The intra-chunk da is formed the "stable" way that the page "Fix Incorrect
// Gradients and Illegal Memory Access Error in Mamba2" discusses for its
// ddA_cumsum kernel: straight from V, never as the difference of a row sum
// and a column sum, so nothing cancels.  The wave that owns column tile J
// walks its tiles from the bottom (I = T-1) up to the diagonal, carrying each
// lane's column sum of V over the tiles already passed.  For row tile K and
// kappa in [0, 16) it forms, per column j of the tile,
//   S[kappa][j] = sum over rows i >= 16K + kappa of V[i][j]
// (in-lane suffix sums, the other row groups' sums gathered with the row
// swaps, plus the carried column sum), and the row sum of S over j (only
// j < 16K + kappa on the diagonal tile) is column tile J's share of da at
// position 16K + kappa.  da_intra is the sum of the shares over J <= K in
// ascending J.  CB itself comes from the dCB kernel (same causal split).
// Every element of ddt, dx and of the slots is written once, by its owner, at
// an absolute index.
#include "ssd_problem.h"
#include "ssd_tiles.h"

namespace ssd {

template <typename T, int Q, int P>
struct HeadCfg {
  static constexpr int T16 = Q / 16;
  static constexpr int W = causal_waves<Q>();   // the dCB kernel's split (8 waves at Q = 256)
  using Split = CausalSplit<T16, W>;
  static constexpr int NCOL = Split::NCOL;
  static constexpr int NTHR = W * WAVE;
  static_assert(NTHR >= Q, "one thread per chunk position");
  static constexpr int PT = P / 16;
  static constexpr int VEC = Vec16<T>::N;
  static constexpr int NBLK = 128;                      // dstate columns per phase-B2 round
  static constexpr int LDSN = NBLK + VEC;               // dS rows [p][n] of one round
  static constexpr int LDP = P + VEC;
  static constexpr int NOWN = Split::NOWN;
  static constexpr int CBD = NOWN < 2 ? NOWN : 2;   // CB tiles requested ahead of their use
  static constexpr int DSV = (P * NBLK / VEC + NTHR - 1) / NTHR;   // 16-byte dS vectors per thread per round
  static constexpr int NKB = NBLK / Mma<T>::KSTEP;      // B fragments per owned column per round
  static constexpr size_t RA = (size_t(2) * Q * LDP + size_t(P) * LDSN) * sizeof(T);  // x, dy, dS rows
  // da shares: [column tile J][position]
  static constexpr size_t RS_FLOATS = size_t(T16) * Q;
  // vectors: acs dt w ee ddacs ddtp sj daint er dfe (10 Q floats) + seg (Q ints) + red (W + 8)
  // + per-channel dD partials (W x P) + the head's D per channel (P)
  static constexpr size_t RV_FLOATS = size_t(11) * Q + ((W + 8 + 3) & ~3) + size_t(W + 1) * P;
  static constexpr size_t OFF_RS = (RA + 15) / 16 * 16;
  static constexpr size_t OFF_RV = OFF_RS + RS_FLOATS * 4;
  // two sets of vectors, taken by consecutive items of a block in turn
  static constexpr size_t RV_BYTES = (RV_FLOATS * 4 + 15) / 16 * 16;
  static constexpr size_t LDS = OFF_RV + 2 * RV_BYTES;
};

// Phase B over the wave's causal tiles (see the top of the file): G, M,
// ddt_intra partials, da shares and dx_intra.  UNI: the chunk has a single
// segment (off-diagonal decays factored through the per-row table er); the
// two versions keep the unrolled tile sequence free of branches on it.
// PF: the dS rows of the first phase-B2 round (see B2Operands) are requested
// in the middle of the tile sequence, into registers the CB tiles already
// used have freed (every tile sequence reaches that point).
// Operands of phase B2 (Z^T = dS B^T) for one round of NBLK dstate columns:
// dS (P x NBLK in the I/O dtype, one 16-byte piece per thread and slot) and this lane's B
// fragments of the two owned column tiles (bf16: one 16-byte piece per k-step).
template <typename T, int Q, int P>
struct B2Operands {
  using Cf = HeadCfg<T, Q, P>;
  static constexpr int KS = Mma<T>::KSTEP, KW = Mma<T>::KW;
  uint4 dsr[Cf::DSV];
  typename Mma<T>::frag bf[2][KW == 8 ? Cf::NKB : 1];
  const T* ds_base;       // dS of this (b, h, c): [P][N]
  const T* brow[2];       // this lane's B row of each owned column tile, at k = 8 (lane / 16) (nullptr past L)
  int N;
  __device__ __forceinline__ int cols(int nb) const { return N - nb * Cf::NBLK < Cf::NBLK ? N - nb * Cf::NBLK : Cf::NBLK; }
  __device__ __forceinline__ void load_ds(int nb) {
    constexpr int VEC = Cf::VEC;
    const int vr = cols(nb) / VEC, nv = P * vr;
#pragma unroll
    for (int q = 0; q < Cf::DSV; ++q) {
      const int v = static_cast<int>(threadIdx.x) + q * Cf::NTHR;
      dsr[q] = zero_u4();
      if (v < nv) dsr[q] = ld_global16(ds_base + (v / vr) * N + nb * Cf::NBLK + VEC * (v % vr));
    }
  }
  __device__ __forceinline__ void load_b(int nb) {
    if constexpr (KW == 8) {
#pragma unroll
      for (int kb = 0; kb < Cf::NKB; ++kb)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          bf[a][kb] = Mma<T>::zero();
          if (brow[a] && kb * KS < cols(nb))
            bf[a][kb] = __builtin_bit_cast(typename Mma<T>::frag, ld_global16(brow[a] + nb * Cf::NBLK + kb * KS));
        }
    }
  }
  // dS round nb -> LDS rows [p][n]
  __device__ __forceinline__ void store_ds(int nb, T* s_dsk) const {
    constexpr int VEC = Cf::VEC;
    const int vr = cols(nb) / VEC, nv = P * vr;
#pragma unroll
    for (int q = 0; q < Cf::DSV; ++q) {
      const int v = static_cast<int>(threadIdx.x) + q * Cf::NTHR;
      if (v < nv) *reinterpret_cast<uint4*>(s_dsk + (v / vr) * Cf::LDSN + VEC * (v % vr)) = dsr[q];
    }
  }
};

// Row sums over the 16 lanes of a row group (the columns of a tile) of a
// tile's 4 values per lane: a butterfly that halves the values per lane at
// each step; lane r16 < 4 ends with row 2 (r16 & 1) + (r16 >> 1) of its group.
__device__ __forceinline__ float rowsum_quads(const float (&x)[4], int r16) {
  const bool odd = (r16 & 1) != 0, hi = (r16 & 2) != 0;
  const float k0 = odd ? x[2] : x[0], k1 = odd ? x[3] : x[1];
  const float t0 = odd ? x[0] : x[2], t1 = odd ? x[1] : x[3];
  const float a0 = k0 + dpp_move<0xB1>(t0);   // quad_perm [1,0,3,2]
  const float a1 = k1 + dpp_move<0xB1>(t1);
  const float kk = hi ? a1 : a0, tt = hi ? a0 : a1;
  float rsum = kk + dpp_move<0x4E>(tt);      // quad_perm [2,3,0,1]
  rsum += dpp_move<0x124>(rsum);             // row_ror:4
  rsum += dpp_move<0x128>(rsum);             // row_ror:8
  return rsum;
}

// One step of an inclusive segmented prefix sum over the lanes of a wave
// (a lane whose flag is set starts a segment): the value and flag of the lane
// that the DPP control CTRL reads in the rows ROWS (0 where it reads none)
// join this lane's unless this lane's range already holds a segment start.
template <int CTRL, int ROWS>
__device__ __forceinline__ void seg_scan_step(float& v, int& f) {
  const float tv = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false));
  const int tf = __builtin_amdgcn_update_dpp(0, f, CTRL, ROWS, 0xF, false);
  v = f ? v : v + tv;
  f |= tf;
}

// Inclusive segmented prefix sum over the 64 lanes in a fixed order: a
// doubling scan within each row of 16 lanes (row_shr 1, 2, 4, 8), then row
// 0's total into row 1 and row 2's into row 3 (row_bcast:15), then the first
// half's total into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ void seg_prefix_lanes(float& v, int& f) {
  seg_scan_step<0x111, 0xF>(v, f);
  seg_scan_step<0x112, 0xF>(v, f);
  seg_scan_step<0x114, 0xF>(v, f);
  seg_scan_step<0x118, 0xF>(v, f);
  seg_scan_step<0x142, 0xA>(v, f);
  seg_scan_step<0x143, 0xC>(v, f);
}

// LDS operands of one causal tile, requested one tile ahead so that their
// latency hides behind the previous tile's arithmetic.
template <typename T, int Q, int P, bool UNI>
struct TileIn {
  static constexpr int MK = P / Mma<T>::KSTEP;   // k-steps of M = dy x^T
  typename Mma<T>::frag ma[MK];                   // dy rows of tile I
  typename Mma<T>::rfrag av[P / 16];              // dy^T of rows I (the dx product's A operand)
  f32x4_t rowv;   // UNI off-diagonal: er of rows I; otherwise Acs of rows I
  int4 seg4;      // segments of rows I (not UNI off-diagonal)
  float acs_i0;   // Acs at row 16 I (UNI off-diagonal)
};

// Column operands of the column tile being walked: the x rows (B operand of
// M = dy x^T) and this lane's column's Acs, dt and segment.
template <typename T, int P>
struct HeadColumn {
  typename Mma<T>::frag mb[P / Mma<T>::KSTEP];
  float aj, dtj;
  int segj;
};

template <typename T, int Q, int P>
__device__ __forceinline__ void head_column_load(HeadColumn<T, P>& cl, int J, const T* s_xk, const float* s_acs,
                                                 const float* s_dt, const int* s_seg) {
  constexpr int LDP = HeadCfg<T, Q, P>::LDP, KW = Mma<T>::KW, KS = Mma<T>::KSTEP;
  const int l = lane_id(), r16 = l & 15, kg = l >> 4;
  const T* bp = s_xk + (16 * J + r16) * LDP + kg * KW;
#pragma unroll
  for (int s = 0; s < P / KS; ++s) cl.mb[s] = Mma<T>::load_k(bp + s * KS);
  const int j = 16 * J + r16;
  cl.aj = s_acs[j];
  cl.dtj = s_dt[j];
  cl.segj = s_seg[j];
}

template <typename T, int Q, int P, bool UNI, bool DIAG>
__device__ __forceinline__ void tile_load(TileIn<T, Q, P, UNI>& in, int I, const T* s_dyk, const float* s_acs,
                                          const float* s_er, const int* s_seg) {
  using Cf = HeadCfg<T, Q, P>;
  constexpr int LDP = Cf::LDP, KW = Mma<T>::KW, KS = Mma<T>::KSTEP;
  const int l = lane_id(), r16 = l & 15, kg = l >> 4;
  const T* ap = s_dyk + (16 * I + r16) * LDP + kg * KW;
#pragma unroll
  for (int s = 0; s < TileIn<T, Q, P, UNI>::MK; ++s) in.ma[s] = Mma<T>::load_k(ap + s * KS);
#pragma unroll
  for (int pt = 0; pt < P / 16; ++pt) in.av[pt] = Mma<T>::rfrag_load_kn(s_dyk + 16 * I * LDP + 16 * pt, LDP);
  if constexpr (UNI && !DIAG) {
    in.acs_i0 = s_acs[16 * I];
    in.rowv = *reinterpret_cast<const f32x4_t*>(s_er + 16 * I + 4 * kg);
  } else {
    in.rowv = *reinterpret_cast<const f32x4_t*>(s_acs + 16 * I + 4 * kg);
    in.seg4 = *reinterpret_cast<const int4*>(s_seg + 16 * I + 4 * kg);
  }
}

template <typename T, int Q, int P, bool UNI, bool PF>
__device__ __forceinline__ void head_tiles(f32x4_t (&cb)[Q / 16 + 1], f32x4_t (&dxt)[2][P / 16], float (&ddti)[2],
                                           float& mdiag,
                                           const T* s_xk, const T* s_dyk, const float* s_acs, const float* s_dt,
                                           const float* s_er, const int* s_seg, float* s_share, int w,
                                           B2Operands<T, Q, P>& b2, const float* cbsrc) {
  using Cf = HeadCfg<T, Q, P>;
  using Split = typename Cf::Split;
  using In = TileIn<T, Q, P, UNI>;
  constexpr int CBD = Cf::CBD;
  constexpr int PT = Cf::PT;
  const int l = lane_id(), r16 = l & 15, kg = l >> 4;
  // per owned column (slot 1 for the column being walked, slot 0 for the
  // first column once it ends): this lane's part (its 4 rows) of the column
  // sums of V over the tiles passed; and the totals of the walked column's
  // tiles passed
  float colp0 = 0.f, colp1 = 0.f, bsum = 0.f;
  const int n0 = Cf::T16 - 1 - w;   // off-diagonal tiles of the first column
  In cur;
  HeadColumn<T, P> col;
  {
    int I, J;
    bool second;
    Split::tile(w, 0, I, J, second);
    tile_load<T, Q, P, UNI, Split::NOFF == 0>(cur, I, s_dyk, s_acs, s_er, s_seg);
    head_column_load<T, Q, P>(col, J, s_xk, s_acs, s_dt, s_seg);
  }
#pragma clang loop unroll(full)
  for (int k = 0; k < Split::NOWN; ++k) {
    int I, J;
    bool second;
    Split::tile(w, k, I, J, second);
    const bool diag = k >= Split::NOFF;   // a constant once unrolled
    if (k + CBD < Split::NOWN) cb[k + CBD] = *reinterpret_cast<const f32x4_t*>(cbsrc + (k + CBD) * 256);
    In nxt;
    if (k + 1 < Split::NOWN) {
      int In_, Jn;
      bool sn;
      Split::tile(w, k + 1, In_, Jn, sn);
      if (k + 1 >= Split::NOFF)
        tile_load<T, Q, P, UNI, true>(nxt, In_, s_dyk, s_acs, s_er, s_seg);
      else
        tile_load<T, Q, P, UNI, false>(nxt, In_, s_dyk, s_acs, s_er, s_seg);
    }
    f32x4_t m = zero4();
#pragma unroll
    for (int s = 0; s < In::MK; ++s) m = Mma<T>::mma(cur.ma[s], col.mb[s], m);
    const int j = 16 * J + r16;
    const float aj = col.aj, dtj = col.dtj;
    f32x4_t e4;   // exp(Acs_i - Acs_j) where (i, j) is causal and in one segment, else 0
    if (UNI && !diag) {
      const float ec = Elem<T>::exp(cur.acs_i0 - aj);
#pragma unroll
      for (int r = 0; r < 4; ++r) e4[r] = cur.rowv[r] * ec;
    } else {
      const int loj = seg_lo(col.segj);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * kg + r;
        const int sgi = r == 0 ? cur.seg4.x : (r == 1 ? cur.seg4.y : (r == 2 ? cur.seg4.z : cur.seg4.w));
        const bool ok = (j <= i) & (seg_lo(sgi) == loj);
        // exp of a non-positive argument only; masked entries use a zero argument
        const float e = Elem<T>::exp(ok ? cur.rowv[r] - aj : 0.f);
        e4[r] = ok ? e : 0.f;
      }
    }
    f32x4_t gm;   // G o M
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float gv = cb[k][r] * e4[r];
      cb[k][r] = gv;
      gm[r] = gv * m[r];
    }
    // column tile J's share of da at the rows of tile I (see the top of the
    // file).  The lane's 4 values share the column j, so the in-lane suffix
    // sums of V = G o M dt_j are dt_j times those of G o M, and the first of
    // those is the tile's ddt_intra part of column j.
    float sg[4];
    sg[3] = gm[3];
    sg[2] = gm[2] + sg[3];
    sg[1] = gm[1] + sg[2];
    sg[0] = gm[0] + sg[1];
    const float gms = sg[0];
    float sfx[4];   // in-lane suffix sums of V over the lane's 4 rows
#pragma unroll
    for (int r = 0; r < 4; ++r) sfx[r] = sg[r] * dtj;
    if (diag) {
      // this lane's entries of M's diagonal, M[i][i] = dy_i . x_i (their sum over
      // the chunk is the head's dD term)
#pragma unroll
      for (int r = 0; r < 4; ++r) mdiag += (r16 == 4 * kg + r) ? m[r] : 0.f;
      // S[kappa][j] = sum over rows i >= kappa of V[i][j] (all of column j's
      // tiles below included), kept for j < kappa only, then summed over j
      const int sl = k == Split::NOFF ? 0 : 1;   // a constant once unrolled
      const float below = sum_kgroups(sl ? colp1 : colp0);
      float grp[4];
      gather_kgroups(sfx[0], grp);   // the 4 row groups' sums of column j
      const float s2 = grp[3], s1 = s2 + grp[2], s0 = s1 + grp[1];
      const float lower = kg == 0 ? s0 : (kg == 1 ? s1 : (kg == 2 ? s2 : 0.f));
      const float base = below + lower;
      float sh[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sh[r] = (r16 < 4 * kg + r) ? base + sfx[r] : 0.f;
      const float rsum = rowsum_quads(sh, r16);
      if (r16 < 4) s_share[J * Q + 16 * I + 4 * kg + 2 * (r16 & 1) + (r16 >> 1)] = rsum;
    } else {
      // Every column of an off-diagonal tile lies before every row, so the
      // share at row kappa is the tile's row-suffix sum at kappa plus the
      // totals of the column's tiles below: row sums of the in-lane suffixes,
      // then the later row groups' totals (read from one lane each) and the
      // running total below, all in one fixed order.
      colp1 += sfx[0];   // this lane's part of its column's sum
      const float rsum = rowsum_quads(sfx, r16);
      const float t0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rsum), 0));
      const float t1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rsum), 16));
      const float t2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rsum), 32));
      const float t3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rsum), 48));
      const float u2 = t3, u1 = u2 + t2, u0 = u1 + t1;
      const float lower = kg == 0 ? u0 : (kg == 1 ? u1 : (kg == 2 ? u2 : 0.f));
      if (r16 < 4) s_share[J * Q + 16 * I + 4 * kg + 2 * (r16 & 1) + (r16 >> 1)] = rsum + (lower + bsum);
      bsum += u0 + t0;
    }
    // register-direct operands: dy^T values (raw) and the G tile (converted once)
    const typename Mma<T>::rfrag(&av)[PT] = cur.av;
    const typename Mma<T>::rfrag gfrag = Mma<T>::rfrag_from_acc(cb[k]);
    // dx^T of the tile's column: the off-diagonal tiles of both columns
    // accumulate into slot 1, whose content moves to slot 0 when the first
    // column ends (see below); the diagonal tiles come last, one per slot.
    if (diag) {
      const int sl = k == Split::NOFF ? 0 : 1;   // a constant once unrolled
      ddti[sl] += gms;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) dxt[sl][pt] = Mma<T>::mma_rd(av[pt], gfrag, dxt[sl][pt]);
    } else {
      ddti[1] += gms;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) dxt[1][pt] = Mma<T>::mma_rd(av[pt], gfrag, dxt[1][pt]);
      // The wave's first column ends after tile n0 - 1 (a wave-uniform
      // branch, taken once): its sums move to slot 0 and slot 1 restarts for
      // the second column.
      if (k >= Cf::T16 / 2 - 1 && k + 1 == n0) {
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          dxt[0][pt] = dxt[1][pt];
          dxt[1][pt] = zero4();
        }
        ddti[0] = ddti[1];
        ddti[1] = 0.f;
        colp0 = colp1;
        colp1 = 0.f;
        bsum = 0.f;
        head_column_load<T, Q, P>(col, Cf::T16 - 1 - w, s_xk, s_acs, s_dt, s_seg);
      }
    }
    // the diagonal tiles: the first column's, then the second's
    if (k + 1 == Split::NOFF) head_column_load<T, Q, P>(col, w, s_xk, s_acs, s_dt, s_seg);
    if (k + 1 == Split::NOFF + 1) head_column_load<T, Q, P>(col, Cf::T16 - 1 - w, s_xk, s_acs, s_dt, s_seg);
    if (PF && k == (Split::NOFF + 1) / 2) b2.load_ds(0);
    if (k + 1 < Split::NOWN) cur = nxt;
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Coordinates of item lb: items run head-in-group fastest, then chunk, then
// group, then batch.  In 32-bit arithmetic (the shape check keeps the item
// count below 2^30): a 64-bit division is a long software sequence, and the
// items are decoded twice per item.
struct ItemCoords {
  int b, g, c, hh, h;
};

__device__ __forceinline__ ItemCoords item_coords(const Problem& pb, int64_t lb) {
  const uint32_t x = static_cast<uint32_t>(lb);
  const uint32_t hpg = static_cast<uint32_t>(pb.hpg), nc = static_cast<uint32_t>(pb.nc);
  const uint32_t G = static_cast<uint32_t>(pb.G);
  const uint32_t r1 = x / hpg, r2 = r1 / nc, b = r2 / G;
  ItemCoords it;
  it.hh = static_cast<int>(x - r1 * hpg);
  it.c = static_cast<int>(r1 - r2 * nc);
  it.g = static_cast<int>(r2 - b * G);
  it.b = static_cast<int>(b);
  it.h = it.g * pb.hpg + it.hh;
  return it;
}

// x and dy rows of item lb -> registers (rows past L read as zero), at
// 32-bit lane offsets (the rows of all heads at their pitch; the shape check
// bounds a chunk's rows at 2^31 bytes) from a wave-uniform base.
template <typename T, int Q, int P>
__device__ __forceinline__ void load_item_rows(const Problem& pb, int64_t lb,
                                               RowStage<T, Q, P, HeadCfg<T, Q, P>::NTHR>& st_x,
                                               RowStage<T, Q, P, HeadCfg<T, Q, P>::NTHR>& st_dy) {
  using St = RowStage<T, Q, P, HeadCfg<T, Q, P>::NTHR>;
  const typename St::Offs off = St::offsets(static_cast<uint32_t>(pb.H * P * sizeof(T)), Q);
  const ItemCoords it = item_coords(pb, lb);
  const int64_t row0 = ((static_cast<int64_t>(it.b) * pb.L + static_cast<int64_t>(it.c) * Q) * pb.H + it.h) * P;
  const int nrows = pb.L - it.c * Q;
  st_x.load_at(static_cast<const T*>(pb.x) + row0, off, nrows);
  st_dy.load_at(static_cast<const T*>(pb.dy) + row0, off, nrows);
}

// One (batch, head, chunk) work item, logical index lb, whose x and dy rows
// are already requested into st_x / st_dy.  At the start of phase D (those
// rows are in LDS by then, and few registers are live) it requests item
// lb_next's rows into the same registers.
template <typename T, int Q, int P>
__device__ __forceinline__ void head_item(const Problem& pb, int64_t lb, char* smem,
                                          RowStage<T, Q, P, HeadCfg<T, Q, P>::NTHR>& st_x,
                                          RowStage<T, Q, P, HeadCfg<T, Q, P>::NTHR>& st_dy, int64_t lb_next, int par) {
  using Cf = HeadCfg<T, Q, P>;
  constexpr int T16 = Cf::T16, W = Cf::W, NTHR = Cf::NTHR, PT = Cf::PT, VEC = Cf::VEC;
  constexpr int LDP = Cf::LDP, LDSN = Cf::LDSN;
  constexpr int R = Q / WAVE;
  smem += opaque_zero();   // keeps the item's LDS addresses from being hoisted out of the item loop
  T* s_xk = reinterpret_cast<T*>(smem);
  T* s_dyk = s_xk + Q * LDP;
  T* s_dsk = s_dyk + Q * LDP;   // dS rows [p][n] in the I/O dtype
  float* s_share = reinterpret_cast<float*>(smem + Cf::OFF_RS);
  float* s_acs = reinterpret_cast<float*>(smem + Cf::OFF_RV + par * Cf::RV_BYTES);
  float* s_dt = s_acs + Q;
  float* s_w = s_dt + Q;
  float* s_ee = s_w + Q;
  float* s_ddacs = s_ee + Q;
  float* s_ddtp = s_ddacs + Q;
  float* s_sj = s_ddtp + Q;
  float* s_daint = s_sj + Q;
  float* s_er = s_daint + Q;
  float* s_dfe = s_er + Q;
  int* s_seg = reinterpret_cast<int*>(s_dfe + Q);
  float* s_red = reinterpret_cast<float*>(s_seg + Q);
  float* s_redp = s_red + ((W + 8 + 3) & ~3);   // (16-byte aligned)
  float* s_Dp = s_redp + W * P;   // D of this head, per channel (the scalar D repeated)

  const ItemCoords it = item_coords(pb, lb);
  const int c = it.c, g = it.g, b = it.b, h = it.h;
  const int tid = threadIdx.x, w = wave_id_s(), l = lane_id(), r16 = l & 15, kg = l >> 4;
  const int64_t bc = static_cast<int64_t>(b) * pb.nc + c;
  const int64_t bhc = (static_cast<int64_t>(b) * pb.H + h) * pb.nc + c;
  const T* Bg = static_cast<const T*>(pb.Bm);
  const int64_t bgc = (static_cast<int64_t>(b) * pb.G + g) * pb.nc + c;

  // per-position metadata, loaded first so that the bulk loads below do not
  // delay it.  The second half of the threads owns the positions (thread tid
  // position tid - Q): wave 0, which may still be finishing the previous
  // item's phase D, then has only its rows to store before phase B.
  static_assert(NTHR == 2 * Q, "a thread per position in each half of the block");
  const int pos = tid - Q;
  float acs_i = 0.f, dt_i = 0.f, offd_i = 0.f, dfe_i = 1.f;
  int seg_i = 0;
  if (pos >= 0) {
    acs_i = pb.acs[bhc * Q + pos];
    dt_i = pb.dtc[bhc * Q + pos];
    if (pb.fe) dfe_i = pb.dfe[bhc * Q + pos];
    seg_i = pb.segpos[bc * Q + pos];
    for (int nt = 0; nt < pb.ntg; ++nt) offd_i += pb.offd[(bhc * pb.ntg + nt) * Q + pos];
  }
  const float acs_end = pb.acs[bhc * Q + Q - 1];
  const int lolast = seg_lo(pb.segpos[bc * Q + Q - 1]);
  const float Dh = pb.D && !pb.d_hp ? pb.D[h] : 0.f;
  float Dp = Dh;
  if (pb.d_hp && pb.D && pos >= 0 && pos < P) Dp = pb.D[h * P + pos];
  const float Ah = pb.A[h];
  float endd = 0.f;   // the chunk-end term's dstate-tile partials, in tile order (used by wave 0)
  if (tid < WAVE)
    for (int nt = 0; nt < pb.ntg; ++nt) endd += pb.endd[bhc * pb.ntg + nt];

  // ---- phase A: the CB tiles of this wave (formed once per group by the
  // dCB kernel, same split); the x, dy rows were requested by the previous
  // item (or before the item loop)
  f32x4_t cb[Cf::NOWN];   // the first CBD now, the others during phase B
  const float* cbsrc = pb.cbt + (bgc * W + w) * Cf::NOWN * 256 + l * 4;
  {
#pragma unroll
    for (int k = 0; k < Cf::CBD; ++k) cb[k] = *reinterpret_cast<const f32x4_t*>(cbsrc + k * 256);
  }

  // A chunk without sequence starts after position 0 has one segment, and its
  // Acs never increases; there exp(Acs_i - Acs_j) of an off-diagonal tile is
  // formed as er_i * exp(Acs_{16I} - Acs_j), both factors <= 1, with
  // er_i = exp(Acs_i - Acs_{16I}) tabled once per block.
  const bool uniform = __builtin_amdgcn_readfirstlane(lolast) == 0;
  const float acs_tile0 = __shfl(acs_i, l & ~15, WAVE);
  if (pos >= 0) {
    s_acs[pos] = acs_i;
    s_dt[pos] = dt_i;
    s_seg[pos] = seg_i;
    s_ddacs[pos] = offd_i;
    const float e = (pos >= lolast) ? Elem<T>::exp(acs_end - acs_i) : 0.f;
    s_ee[pos] = e;
    s_w[pos] = e * dt_i;
    s_er[pos] = uniform ? Elem<T>::exp(acs_i - acs_tile0) : 0.f;
    s_dfe[pos] = dfe_i;
    if (pos < P) s_Dp[pos] = Dp;
  }

  // ---- phase B: x, dy rows; decays; M; ddt_intra; da shares; dx_intra
  st_x.store(s_xk, LDP);
  st_dy.store(s_dyk, LDP);
  __syncthreads();
  // dD of the head (scalar D): the trace of M = dy x^T, summed from the
  // diagonal tiles of phase B; per channel (d_hp): the channel sums of dy x
  if (pb.d_hp) {    // (uniform) a thread's vectors all start at p0 = VEC (tid mod P / VEC)
    static_assert(NTHR % (P / VEC) == 0 && WAVE % (P / VEC) == 0, "fixed channel group per thread");
    float dd[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) dd[e] = 0.f;
    for (int v = tid; v < Q * P / VEC; v += NTHR) {
      const int i = v / (P / VEC), p0 = (v % (P / VEC)) * VEC;
      const uint4 dv = *reinterpret_cast<const uint4*>(s_dyk + i * LDP + p0);
      const uint4 xv = *reinterpret_cast<const uint4*>(s_xk + i * LDP + p0);
#pragma unroll
      for (int e = 0; e < VEC; ++e) dd[e] += vget<T>(dv, e) * vget<T>(xv, e);
    }
    // over the lanes of one channel group (fixed xor order), then per wave to LDS
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      for (int m = P / VEC; m < WAVE; m <<= 1) dd[e] += __shfl_xor(dd[e], m, WAVE);
    if (l < P / VEC)
#pragma unroll
      for (int e = 0; e < VEC; ++e) s_redp[w * P + l * VEC + e] = dd[e];
  }

  f32x4_t dxt[Cf::NCOL][PT];
#pragma unroll
  for (int a = 0; a < Cf::NCOL; ++a)
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) dxt[a][pt] = zero4();
  float ddti[Cf::NCOL];   // per-lane partial sums of G o M over a column's tiles
#pragma unroll
  for (int a = 0; a < Cf::NCOL; ++a) ddti[a] = 0.f;
  B2Operands<T, Q, P> b2;
  b2.ds_base = static_cast<const T*>(pb.dstate) + bhc * P * pb.N;
  b2.N = pb.N;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int t = c * Q + 16 * Cf::Split::col(w, a) + r16;
    b2.brow[a] = t < pb.L ? Bg + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + kg * Mma<T>::KW
                          : nullptr;
  }
  constexpr bool PF = Mma<T>::KW == 8;   // bf16: first B2 round prefetched during phase B
  float mdiag = 0.f;   // this lane's part of the trace of M
  if (uniform)
    head_tiles<T, Q, P, true, PF>(cb, dxt, ddti, mdiag, s_xk, s_dyk, s_acs, s_dt, s_er, s_seg, s_share, w, b2, cbsrc);
  else
    head_tiles<T, Q, P, false, PF>(cb, dxt, ddti, mdiag, s_xk, s_dyk, s_acs, s_dt, s_er, s_seg, s_share, w, b2, cbsrc);
  if (!pb.d_hp) {   // (uniform) the wave's share of the trace, summed over waves in phase D
    const float dd = wave_sum(mdiag);
    if (l == 0) s_red[w] = dd;
  }

  // ---- phase B2: Z^T = dS B^T for the owned column tiles, in rounds of NBLK
  // dstate columns: dS rows from LDS (A operand), the owned columns' B rows
  // straight from memory (B operand)
  f32x4_t zt[Cf::NCOL][PT];
#pragma unroll
  for (int a = 0; a < Cf::NCOL; ++a)
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) zt[a][pt] = zero4();
  {
    constexpr int KS = Mma<T>::KSTEP, KW = Mma<T>::KW;
    for (int nb = 0; nb * Cf::NBLK < pb.N; ++nb) {
      if (!PF || nb > 0) b2.load_ds(nb);
      b2.load_b(nb);
      if (nb > 0) __syncthreads();   // the previous round's dS rows are read
      b2.store_ds(nb, s_dsk);
      __syncthreads();
      if (nb == 0) {
        // every wave's phase B is done: the intra-chunk da of each position
        // (the second half of the block, as in phase A) and, per channel, the
        // dD slot of this (b, c, h), waves in order
        if (pos >= 0) {
          const int k = pos, K = k / 16;
          float da = 0.f;
#pragma unroll
          for (int J = 0; J < T16; ++J) {
            const float v = s_share[J * Q + k];
            da += (J <= K) ? v : 0.f;
          }
          s_daint[k] = da;
        }
        if (pb.d_hp && tid < P) {
          float dd = 0.f;
          for (int k = 0; k < W; ++k) dd += s_redp[k * P + tid];
          pb.slot_dDp[(bc * pb.H + h) * P + tid] = dd;
        }
      }
      const int ncols = b2.cols(nb);
      if constexpr (KW == 8) {
#pragma unroll
        for (int kb = 0; kb < Cf::NKB; ++kb) {
          if (kb * KS >= ncols) break;
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) {
            const auto af = Mma<T>::load_k(s_dsk + (16 * pt + r16) * LDSN + kg * KW + kb * KS);
#pragma unroll
            for (int a = 0; a < Cf::NCOL; ++a) zt[a][pt] = Mma<T>::mma(af, b2.bf[a][kb], zt[a][pt]);
          }
        }
      } else {
        for (int k0 = 0; k0 < ncols; k0 += KS) {
          typename Mma<T>::frag bf[Cf::NCOL];
#pragma unroll
          for (int a = 0; a < Cf::NCOL; ++a) bf[a] = b2.brow[a] ? b2.brow[a][nb * Cf::NBLK + k0] : 0.f;
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) {
            const auto af = Mma<T>::load_k(s_dsk + (16 * pt + r16) * LDSN + kg * KW + k0);
#pragma unroll
            for (int a = 0; a < Cf::NCOL; ++a) zt[a][pt] = Mma<T>::mma(af, bf[a], zt[a][pt]);
          }
        }
      }
    }
  }

  // ---- phase C: dx, and per column the ddt parts and s_j
#pragma unroll
  for (int a = 0; a < Cf::NCOL; ++a) {
    const int J = Cf::Split::col(w, a);
    const int j = 16 * J + r16, t = c * Q + j;
    const float dtj = s_dt[j], wj = s_w[j], eej = s_ee[j];
    float xz = 0.f;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      const f32x4_t dyv = load4f<T>(s_dyk + j * LDP + 16 * pt + 4 * kg);
      const f32x4_t xv = load4f<T>(s_xk + j * LDP + 16 * pt + 4 * kg);
      const f32x4_t D4 = *reinterpret_cast<const f32x4_t*>(s_Dp + 16 * pt + 4 * kg);
      f32x4_t outv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        outv[r] = dtj * dxt[a][pt][r] + wj * zt[a][pt][r] + D4[r] * dyv[r];
        xz += xv[r] * zt[a][pt][r];
      }
      if (t < pb.L)
        store4f<T>(static_cast<T*>(pb.dx) + ((static_cast<int64_t>(b) * pb.L + t) * pb.H + h) * P + 16 * pt + 4 * kg,
                   outv);
    }
    xz = sum_kgroups(xz);
    const float gsum = sum_kgroups(ddti[a]);
    if (kg == 0) {
      s_ddtp[j] = gsum + eej * xz;
      s_sj[j] = wj * xz;
    }
  }
  __syncthreads();

  load_item_rows<T, Q, P>(pb, lb_next, st_x, st_dy);

  // ---- phase D: da and its consumers, in wave 0 alone (the intra-chunk da
  // was formed during phase B2; the other waves go on to the next item)
  if (w == 0) {
    float tail;   // chunk-end terms of ddAcs at position Q-1
    {
      float v = 0.f;
#pragma unroll
      for (int e = 0; e < R; ++e) v += s_sj[l * R + e];
      const float sum_s = wave_sum(v);
      tail = sum_s + Elem<T>::exp(acs_end) * endd;
      tail = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, tail)));
    }
    // reverse in-chunk, in-segment cumulative sum of ddAcs (fixed order).  The
    // lanes hold the positions in reverse order (lane l: positions from
    // (63 - l) R), so the sum over later positions is a prefix over lanes.
    const int lp = (WAVE - 1 - l) * R;   // this lane's first position
    float v[R], loc[R];
    int f[R];
#pragma unroll
    for (int e = 0; e < R; ++e) {
      const int i = lp + e;
      v[e] = s_ddacs[i] - s_sj[i];
      if (i == Q - 1) v[e] += tail;
      f[e] = (i == Q - 1) || (seg_lo(s_seg[i + 1]) == i + 1);
    }
    float run = 0.f;
    int any = 0;
#pragma unroll
    for (int e = R - 1; e >= 0; --e) {
      if (f[e]) {
        run = v[e];
        any = 1;
      } else {
        run += v[e];
      }
      loc[e] = run;
    }
    // lane l's run continues into the lanes below it (earlier positions) until
    // a lane that holds a segment end: the segmented prefix over lanes, and the
    // carry into lane l is lane l - 1's value (wave_shr:1; 0 for lane 0)
    float vl = run;
    int fl = any;
    seg_prefix_lanes(vl, fl);
    const float carry = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, vl), 0x138, 0xF, 0xF, false));
    int seen = 0;
    float dap = 0.f, dbp = 0.f;
    float da_k[R];
#pragma unroll
    for (int e = R - 1; e >= 0; --e) {
      const int k = lp + e;
      if (f[e]) seen = 1;
      const float rc = seen ? loc[e] : loc[e] + carry;
      da_k[e] = s_daint[k] + rc;
      dap += s_dt[k] * da_k[e];
    }
    if (!pb.fe) {   // (uniform) ddt with respect to the dt the recurrence uses
#pragma unroll
      for (int e = R - 1; e >= 0; --e) {
        const int k = lp + e, t = c * Q + k;
        if (t < pb.L) pb.ddt[(static_cast<int64_t>(b) * pb.L + t) * pb.H + h] = s_ddtp[k] + Ah * da_k[e];
      }
    } else {        // ... and on to the raw dt, through the front-end's derivative
#pragma unroll
      for (int e = R - 1; e >= 0; --e) {
        const int k = lp + e, t = c * Q + k;
        const float ddt = (s_ddtp[k] + Ah * da_k[e]) * s_dfe[k];
        if (t < pb.L) {
          pb.ddt[(static_cast<int64_t>(b) * pb.L + t) * pb.H + h] = ddt;
          dbp += ddt;
        }
      }
    }
    dap = wave_sum(dap);
    if (pb.ddt_bias) dbp = wave_sum(dbp);
    if (l == 0) {
      if (pb.ddt_bias) pb.slot_ddtb[bc * pb.H + h] = dbp;
      pb.slot_dA[bc * pb.H + h] = dap;
      if (!pb.d_hp) {
        float dd = 0.f;
        for (int k = 0; k < W; ++k) dd += s_red[k];
        pb.slot_dD[bc * pb.H + h] = dd;
      }
    }
  }
}

// Persistent blocks: the blocks on one XCD (block i runs on XCD i % 8) take
// the logical items of that XCD's contiguous share in order, so the heads of
// one (group, chunk), which read the same CB tiles, run on one XCD at about
// the same time.  With fewer than 8 blocks the items are split into as many
// shares as there are blocks, so every item has a block at any grid size.
// Every item is computed the same way whichever block takes it.
template <typename T, int Q, int P>
__global__ __launch_bounds__((HeadCfg<T, Q, P>::NTHR)) void k_head_bwd(Problem pb) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int64_t total = static_cast<int64_t>(pb.B) * pb.H * pb.nc;
  const int64_t nblk = gridDim.x;
  const int64_t NXCD = nblk < 8 ? nblk : 8;
  const int64_t xcd = blockIdx.x % NXCD, slot = blockIdx.x / NXCD;
  const int64_t nb_x = nblk / NXCD + (xcd < nblk % NXCD ? 1 : 0);   // blocks on this XCD
  const int64_t q = total / NXCD, r = total % NXCD;
  const int64_t begin = xcd * q + (xcd < r ? xcd : r), count = q + (xcd < r ? 1 : 0);
  RowStage<T, Q, P, HeadCfg<T, Q, P>::NTHR> st_x, st_dy;
  if (slot < count) load_item_rows<T, Q, P>(pb, begin + slot, st_x, st_dy);
  // No barrier between items: an item's phase A writes its x and dy rows,
  // which the previous item last read before its phase-C barrier, and its own
  // set of vectors (the two sets alternate), which the previous item's phase
  // D may still be reading in wave 0; so the other waves start the item while
  // wave 0 finishes the previous one's scan.
  int par = 0;
  for (int64_t k = slot; k < count; k += nb_x, par ^= 1) {
    // (after the last item the rows requested are its own again: unused, but
    // keeps the request unconditional)
    const int64_t next = k + nb_x < count ? begin + k + nb_x : begin + k;
    head_item<T, Q, P>(pb, begin + k, smem, st_x, st_dy, next, par);
  }
}

template <typename T, int Q, int P>
static hipError_t launch_head_t(const Problem& pb, hipStream_t s) {
  using Cf = HeadCfg<T, Q, P>;
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&k_head_bwd<T, Q, P>), Cf::LDS);
  if (e != hipSuccess) return e;
  // a fixed number of persistent blocks (one per CU of an MI355X at one block
  // per CU), or the test override; each block's items and every item's
  // arithmetic are the same whatever the count
  const int64_t items = static_cast<int64_t>(pb.B) * pb.H * pb.nc;
  const int ov = head_blocks_override();
  const int64_t want = ov > 0 ? ov : kHeadBlocks;
  const int64_t blocks = items < want ? items : want;
  hipLaunchKernelGGL((k_head_bwd<T, Q, P>), dim3(static_cast<unsigned>(blocks)), dim3(Cf::NTHR), Cf::LDS, s, pb);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_head_any(const Problem& pb, hipStream_t s) {
#define SSD_HEAD_CASE(QQ, PP) \
  if (pb.Q == QQ && pb.P == PP) return launch_head_t<T, QQ, PP>(pb, s);
  if constexpr (sizeof(T) == 2) {
    SSD_BF16_SHAPES(SSD_HEAD_CASE)
  } else {
    SSD_F32_SHAPES(SSD_HEAD_CASE)
  }
#undef SSD_HEAD_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_head_bwd(const Problem& pb, bool io_bf16, hipStream_t s) {
  return io_bf16 ? launch_head_any<bf16_t>(pb, s) : launch_head_any<float>(pb, s);
}

// LDS bytes of the head kernel for a compiled shape (host-side support check);
// ~0 when the shape is not compiled.
size_t head_lds_bytes(int Q, int P, bool bf16) {
#define SSD_HEAD_LDS_B(QQ, PP) \
  if (bf16 && Q == QQ && P == PP) return HeadCfg<bf16_t, QQ, PP>::LDS;
#define SSD_HEAD_LDS_F(QQ, PP) \
  if (!bf16 && Q == QQ && P == PP) return HeadCfg<float, QQ, PP>::LDS;
  SSD_BF16_SHAPES(SSD_HEAD_LDS_B)
  SSD_F32_SHAPES(SSD_HEAD_LDS_F)
#undef SSD_HEAD_LDS_B
#undef SSD_HEAD_LDS_F
  return ~size_t(0);
}

}  // namespace ssd
