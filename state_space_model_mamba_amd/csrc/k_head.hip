// Head kernel: everything of one (batch, head, chunk) that needs no head sum
// -- combined_bwd_dx (dx), chunk_scan_bwd_ddAcs + chunk_state_bwd_ddAcs
// (ddA_cumsum) and chunk_cumsum_bwd (ddt and the dA partial) in the kernel
// list of the page "Deterministic bwd kernel for mamba2".
//
//   CB        = C B^T                         (Q x Q causal, MFMA over N)
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
// and a column sum, so nothing cancels.  With k = 16K + kappa it splits over
// 16x16 tiles into (full tiles strictly below-left) + (row tile K, rows >= k)
// + (column tile K, columns < k) + (the diagonal tile); each piece is a sum of
// per-tile row sums / column sums / totals taken in a fixed order.  Every
// element of ddt, dx and of the slots is written once, by its owner, at an
// absolute index.
#include "ssd_problem.h"
#include "ssd_tiles.h"

namespace ssd {

template <typename T, int Q, int P>
struct HeadCfg {
  static constexpr int T16 = Q / 16;
  static constexpr int W = causal_waves<Q>();
  using Split = CausalSplit<T16, W>;
  static constexpr int NCOL = Split::NCOL;
  static constexpr int NTHR = W * WAVE;
  static constexpr int NCAUS = T16 * (T16 + 1) / 2;
  static constexpr int PT = P / 16;
  static constexpr int VEC = Vec16<T>::N;
  static constexpr int NS = sizeof(T) == 2 ? 32 : 16;   // dstate slab (divides N)
  static constexpr int LDN = NS + VEC;
  static constexpr int LDP = P + VEC;
  static constexpr int NOWN = Split::NOWN;
  static constexpr size_t RA_A = size_t(2) * Q * LDN * sizeof(T);                 // C, B slabs
  static constexpr size_t RA_B = (size_t(2) * Q * LDP + size_t(Q + P) * LDN) * sizeof(T);  // x, dy rows + B, dS slabs
  static constexpr size_t RA = RA_A > RA_B ? RA_A : RA_B;
  // tile sums: rs, cs [NCAUS*16], tot [NCAUS], vdiag [T16*256], t1 [T16], rs2 [Q], cs3 [Q]
  static constexpr size_t RS_FLOATS = size_t(NCAUS) * 33 + size_t(T16) * 257 + size_t(2) * Q;
  // vectors: acs dt w ee ddacs ddtp sj dd daint (9 Q floats) + seg (Q ints) + red (W + 8)
  static constexpr size_t RV_FLOATS = size_t(10) * Q + W + 8;
  static constexpr size_t OFF_RS = (RA + 15) / 16 * 16;
  static constexpr size_t OFF_RV = OFF_RS + RS_FLOATS * 4;
  static constexpr size_t LDS = OFF_RV + RV_FLOATS * 4;
};

__device__ __forceinline__ int causal_index(int I, int J) { return I * (I + 1) / 2 + J; }

template <typename T, int Q, int P>
__global__ __launch_bounds__((HeadCfg<T, Q, P>::NTHR)) void k_head_bwd(Problem pb) {
  using Cf = HeadCfg<T, Q, P>;
  constexpr int T16 = Cf::T16, W = Cf::W, NTHR = Cf::NTHR, PT = Cf::PT, VEC = Cf::VEC;
  constexpr int NS = Cf::NS, LDN = Cf::LDN, LDP = Cf::LDP, NCAUS = Cf::NCAUS;
  constexpr int R = Q / WAVE;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // phase A
  T* s_ck = reinterpret_cast<T*>(smem);
  T* s_bk = s_ck + Q * LDN;
  // phase B (aliases phase A)
  T* s_xk = reinterpret_cast<T*>(smem);
  T* s_dyk = s_xk + Q * LDP;
  T* s_bz = s_dyk + Q * LDP;
  T* s_dsz = s_bz + Q * LDN;
  float* s_rs = reinterpret_cast<float*>(smem + Cf::OFF_RS);
  float* s_cs = s_rs + NCAUS * 16;
  float* s_tot = s_cs + NCAUS * 16;
  float* s_vdiag = s_tot + NCAUS;
  float* s_t1 = s_vdiag + T16 * 256;
  float* s_rs2 = s_t1 + T16;
  float* s_cs3 = s_rs2 + Q;
  float* s_acs = reinterpret_cast<float*>(smem + Cf::OFF_RV);
  float* s_dt = s_acs + Q;
  float* s_w = s_dt + Q;
  float* s_ee = s_w + Q;
  float* s_ddacs = s_ee + Q;
  float* s_ddtp = s_ddacs + Q;
  float* s_sj = s_ddtp + Q;
  float* s_dd = s_sj + Q;
  float* s_daint = s_dd + Q;
  int* s_seg = reinterpret_cast<int*>(s_daint + Q);
  float* s_red = reinterpret_cast<float*>(s_seg + Q);

  const int64_t total = static_cast<int64_t>(pb.B) * pb.H * pb.nc;
  const int64_t lb = xcd_logical_block(blockIdx.x, total);
  const int hh = static_cast<int>(lb % pb.hpg);
  int64_t rest = lb / pb.hpg;
  const int c = static_cast<int>(rest % pb.nc);
  rest /= pb.nc;
  const int g = static_cast<int>(rest % pb.G);
  const int b = static_cast<int>(rest / pb.G);
  const int h = g * pb.hpg + hh;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r16 = l & 15, kg = l >> 4;
  const int64_t bc = static_cast<int64_t>(b) * pb.nc + c;
  const int64_t bhc = (static_cast<int64_t>(b) * pb.H + h) * pb.nc + c;
  const T* xg = static_cast<const T*>(pb.x);
  const T* dyg = static_cast<const T*>(pb.dy);
  const T* Bg = static_cast<const T*>(pb.Bm);
  const T* Cg = static_cast<const T*>(pb.Cm);

  for (int i = tid; i < Q; i += NTHR) {
    s_acs[i] = pb.acs[bhc * Q + i];
    s_dt[i] = pb.dtc[bhc * Q + i];
    s_seg[i] = pb.segpos[bc * Q + i];
    float o = 0.f;
    for (int nt = 0; nt < pb.ntg; ++nt) o += pb.offd[(bhc * pb.ntg + nt) * Q + i];
    s_ddacs[i] = o;
  }
  __syncthreads();
  const int lolast = seg_lo(s_seg[Q - 1]);
  const float acs_end = s_acs[Q - 1];
  for (int i = tid; i < Q; i += NTHR) {
    const float e = (i >= lolast) ? Elem<T>::exp(acs_end - s_acs[i]) : 0.f;
    s_ee[i] = e;
    s_w[i] = e * s_dt[i];
  }
  constexpr int NCOL = Cf::NCOL;

  // Row sources of the global tiles this block stages (nullptr = zero row).
  auto bc_row = [&](const T* base, int n0) {
    return [=](int i) -> const T* {
      const int t = c * Q + i;
      return t < pb.L ? base + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + n0 : nullptr;
    };
  };
  auto head_row = [&](const T* base) {
    return [=](int i) -> const T* {
      const int t = c * Q + i;
      return t < pb.L ? base + ((static_cast<int64_t>(b) * pb.L + t) * pb.H + h) * P : nullptr;
    };
  };
  auto ds_row = [&](int n0) {
    return [=](int p) -> const float* { return pb.dstate + (bhc * P + p) * pb.N + n0; };
  };

  // ---- phase A: CB over the owned causal tiles, slab by slab over N; the
  // next slab is loaded into registers while the current one is multiplied
  f32x4_t cb[Cf::NOWN];
#pragma unroll
  for (int k = 0; k < Cf::NOWN; ++k) cb[k] = zero4();
  RowStage<T, Q, NS, NTHR> st_c, st_b;
  RowStage<T, Q, P, NTHR> st_x, st_dy;
  st_c.load(bc_row(Cg, 0));
  st_b.load(bc_row(Bg, 0));
  for (int n0 = 0; n0 < pb.N; n0 += NS) {
    __syncthreads();
    st_c.store(s_ck, LDN);
    st_b.store(s_bk, LDN);
    __syncthreads();
    if (n0 + NS < pb.N) {
      st_c.load(bc_row(Cg, n0 + NS));
      st_b.load(bc_row(Bg, n0 + NS));
    } else {
      st_x.load(head_row(xg));
      st_dy.load(head_row(dyg));
    }
    const int z = opaque_zero();
    const int wz = w + z;
#pragma clang loop unroll(full)
    for (int k = 0; k < Cf::NOWN; ++k) {
      int I, J;
      bool second;
      Cf::Split::tile(wz, k, I, J, second);
      cb[k] = tile_mma_kk<T>(cb[k], s_ck + z + 16 * I * LDN, LDN, s_bk + z + 16 * J * LDN, LDN, 0, NS);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();

  // ---- phase B: x, dy rows; decays; M; ddt_intra; V tile sums; dx_intra
  st_x.store(s_xk, LDP);
  st_dy.store(s_dyk, LDP);
  __syncthreads();
  // first slab of phase B2 in flight during phase B
  RowStage<float, P, NS, NTHR> st_ds;
  st_b.load(bc_row(Bg, 0));
  st_ds.load(ds_row(0));
  {
    float dd = 0.f;
    for (int v = tid; v < Q * P; v += NTHR) {
      const int i = v / P, p = v % P;
      dd += Elem<T>::to_f(s_dyk[i * LDP + p]) * Elem<T>::to_f(s_xk[i * LDP + p]);
    }
    dd = wave_sum(dd);
    if (l == 0) s_red[w] = dd;
  }

  f32x4_t dxt[NCOL][PT];
#pragma unroll
  for (int a = 0; a < NCOL; ++a)
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) dxt[a][pt] = zero4();
  float ddti[NCOL];
#pragma unroll
  for (int a = 0; a < NCOL; ++a) ddti[a] = 0.f;
#pragma clang loop unroll(full)
  for (int k = 0; k < Cf::NOWN; ++k) {
    int I, J;
    bool second;
    Cf::Split::tile(w, k, I, J, second);
    const f32x4_t m = tile_mma_kk<T>(zero4(), s_dyk + 16 * I * LDP, LDP, s_xk + 16 * J * LDP, LDP, 0, P);
    const int j = 16 * J + r16;
    const int loj = seg_lo(s_seg[j]);
    const float aj = s_acs[j], dtj = s_dt[j];
    float colgm = 0.f, colv = 0.f, vr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * I + 4 * kg + r;
      const bool ok = (j <= i) && (seg_lo(s_seg[i]) == loj);
      // exp of a non-positive argument only; masked entries use a zero argument
      const float e = Elem<T>::exp(ok ? s_acs[i] - aj : 0.f);
      const float gv = ok ? cb[k][r] * e : 0.f;
      cb[k][r] = gv;
      const float gm = gv * m[r];
      colgm += gm;
      vr[r] = gm * dtj;
      colv += vr[r];
    }
    colgm = sum_kgroups(colgm);
    const int tix = causal_index(I, J);
    colv = sum_kgroups(colv);
    if (kg == 0) s_cs[tix * 16 + r16] = colv;
    const float tot = sum16(colv);
    if (l == 0) s_tot[tix] = tot;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float rsum = sum16(vr[r]);
      if (r16 == 0) s_rs[tix * 16 + 4 * kg + r] = rsum;
    }
    if (I == J) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s_vdiag[I * 256 + (4 * kg + r) * 16 + r16] = vr[r];
    }
    // register-direct operands: dy^T values (raw) and the G tile (converted once)
    typename Mma<T>::rfrag av[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) av[pt] = Mma<T>::rfrag_load(s_dyk + (16 * I + 4 * kg) * LDP + 16 * pt + r16, LDP);
    const typename Mma<T>::rfrag gfrag = Mma<T>::rfrag_from_acc(cb[k]);
    // dx^T of the tile's column: slot 2q or 2q+1 of its pair (a wave-uniform
    // choice); both slot indices are constants once the loop is unrolled
    const int q = k / (T16 + 1);
    if (!second) {
      ddti[2 * q] += colgm;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) dxt[2 * q][pt] = Mma<T>::mma_rd(av[pt], gfrag, dxt[2 * q][pt]);
    } else {
      ddti[2 * q + 1] += colgm;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt)
        dxt[2 * q + 1][pt] = Mma<T>::mma_rd(av[pt], gfrag, dxt[2 * q + 1][pt]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- phase B2: Z^T = dS B^T for the owned column tiles, slab by slab over N
  // (x and dy rows stay in LDS; B and dS slabs go to the region behind them)
  f32x4_t zt[NCOL][PT];
#pragma unroll
  for (int a = 0; a < NCOL; ++a)
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) zt[a][pt] = zero4();
  for (int n0 = 0; n0 < pb.N; n0 += NS) {
    __syncthreads();
    st_b.store(s_bz, LDN);
    st_ds.template store_convert<T>(s_dsz, LDN);
    __syncthreads();
    if (n0 + NS < pb.N) {
      st_b.load(bc_row(Bg, n0 + NS));
      st_ds.load(ds_row(n0 + NS));
    }
    const int z = opaque_zero();
    const int wz = w + z;
#pragma unroll
    for (int a = 0; a < NCOL; ++a) {
      const int J = Cf::Split::col(wz, a);
#pragma unroll
      for (int pt = 0; pt < PT; ++pt)
        zt[a][pt] = tile_mma_kk<T>(zt[a][pt], s_dsz + z + 16 * pt * LDN, LDN, s_bz + z + 16 * J * LDN, LDN, 0, NS);
    }
  }

  // ---- phase C: dx, and per column the ddt parts and s_j
  const float Dh = pb.D ? pb.D[h] : 0.f;
#pragma unroll
  for (int a = 0; a < NCOL; ++a) {
    const int J = Cf::Split::col(w, a);
    const int j = 16 * J + r16, t = c * Q + j;
    const float dtj = s_dt[j], wj = s_w[j], eej = s_ee[j];
    float xz = 0.f;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      T outv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = 16 * pt + 4 * kg + r;
        const float dyv = Elem<T>::to_f(s_dyk[j * LDP + p]);
        const float xv = Elem<T>::to_f(s_xk[j * LDP + p]);
        outv[r] = Elem<T>::from_f(dtj * dxt[a][pt][r] + wj * zt[a][pt][r] + Dh * dyv);
        xz += xv * zt[a][pt][r];
      }
      if (t < pb.L) {
        T* dst = static_cast<T*>(pb.dx) + ((static_cast<int64_t>(b) * pb.L + t) * pb.H + h) * P + 16 * pt + 4 * kg;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[r] = outv[r];
      }
    }
    xz = sum_kgroups(xz);
    if (kg == 0) {
      s_ddtp[j] = ddti[a] + eej * xz;
      s_sj[j] = wj * xz;
    }
  }
  __syncthreads();

  // ---- phase D: da and its consumers
  if (tid < T16) {
    const int K = tid;
    float t1 = 0.f;
    for (int I = K + 1; I < T16; ++I)
      for (int J = 0; J < K; ++J) t1 += s_tot[causal_index(I, J)];
    s_t1[K] = t1;
  }
  if (tid < Q) {
    const int i = tid, K = i / 16, ii = i % 16;
    float rs2 = 0.f;
    for (int J = 0; J < K; ++J) rs2 += s_rs[causal_index(K, J) * 16 + ii];
    s_rs2[i] = rs2;
    float cs3 = 0.f;
    for (int I = K + 1; I < T16; ++I) cs3 += s_cs[causal_index(I, K) * 16 + ii];
    s_cs3[i] = cs3;
    s_dd[i] = s_ddacs[i] - s_sj[i];
  }
  float sum_s = 0.f;
  if (w == 0) {
    float v = 0.f;
#pragma unroll
    for (int e = 0; e < R; ++e) v += s_sj[l * R + e];
    sum_s = wave_sum(v);
  }
  float endd = 0.f;
  for (int nt = 0; nt < pb.ntg; ++nt) endd += pb.endd[bhc * pb.ntg + nt];
  __syncthreads();
  if (tid < Q) {
    const int k = tid, K = k / 16, kap = k % 16;
    float t2 = 0.f;
    for (int ii = 15; ii >= kap; --ii) t2 += s_rs2[16 * K + ii];
    float t3 = 0.f;
    for (int jj = 0; jj < kap; ++jj) t3 += s_cs3[16 * K + jj];
    float t4 = 0.f;
    for (int ii = kap; ii < 16; ++ii)
      for (int jj = 0; jj < kap; ++jj) t4 += s_vdiag[K * 256 + ii * 16 + jj];
    s_daint[k] = ((s_t1[K] + t2) + t3) + t4;
  }
  if (tid == 0) s_dd[Q - 1] += sum_s + Elem<T>::exp(acs_end) * endd;
  __syncthreads();
  if (w == 0) {
    // reverse in-chunk, in-segment cumulative sum of ddAcs (fixed order)
    float v[R], loc[R];
    int f[R];
#pragma unroll
    for (int e = 0; e < R; ++e) {
      const int i = l * R + e;
      v[e] = s_dd[i];
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
    float vl = run;
    int fl = any;
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
      const float vu = __shfl_down(vl, off, WAVE);
      const int fu = __shfl_down(fl, off, WAVE);
      if (l + off < WAVE) {
        if (!fl) vl = vl + vu;
        fl |= fu;
      }
    }
    float carry = __shfl_down(vl, 1, WAVE);
    if (l == WAVE - 1) carry = 0.f;
    int seen = 0;
    const float Ah = pb.A[h];
    float dap = 0.f;
#pragma unroll
    for (int e = R - 1; e >= 0; --e) {
      const int k = l * R + e;
      if (f[e]) seen = 1;
      const float rc = seen ? loc[e] : loc[e] + carry;
      const float da = s_daint[k] + rc;
      const float ddt = s_ddtp[k] + Ah * da;
      const int t = c * Q + k;
      if (t < pb.L) pb.ddt[(static_cast<int64_t>(b) * pb.L + t) * pb.H + h] = ddt;
      dap += s_dt[k] * da;
    }
    dap = wave_sum(dap);
    if (l == 0) {
      pb.slot_dA[bc * pb.H + h] = dap;
      float dd = 0.f;
      for (int k = 0; k < W; ++k) dd += s_red[k];
      pb.slot_dD[bc * pb.H + h] = dd;
    }
  }
}

template <typename T, int Q, int P>
static hipError_t launch_head_t(const Problem& pb, hipStream_t s) {
  using Cf = HeadCfg<T, Q, P>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_head_bwd<T, Q, P>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(Cf::LDS));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = static_cast<int64_t>(pb.B) * pb.H * pb.nc;
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
