// Group kernel: dB and dC of one (batch, group, chunk, dstate tile), the
// chunk_scan_bwd_dC / chunk_state_bwd_db rows of the page "Deterministic bwd
// kernel for mamba2" together with the intra-chunk dCB product.
//
// For the heads h of the group, in ascending order (the head sum lives in
// fp32 accumulator registers, so it needs no per-head slots and no atomics):
//   M_h     = dy_h x_h^T                                   (Q x Q causal, MFMA over P)
//   dCB    += W_h o M_h,  W_h[i,j] = exp(Acs_i - Acs_j) dt_j   (j <= i, same segment)
//   dC^off += exp(Acs_i) dy_h,i E_h,seg(i)                 (MFMA over P)
//   dB^st  += w_j dS_h^T x_h,j,  w_j = exp(Acs_end - Acs_j) dt_j (last segment)
// where E is the state entering a row's segment: Hin for a segment that
// continues the previous chunk's sequence, the sequence's initial state
// otherwise.  Then
//   dB = dB^st + dCB^T C     (register-direct MFMA: the dCB tiles feed the MFMA B operand)
//   dC = dC^off + dCB B      (dCB rows staged through LDS, half the chunk at a time)
// It also leaves, per head, the partial (over this dstate tile) of
//   offd_i = exp(Acs_i) dy_i . (E C_i)        (the off-diagonal ddA_cumsum term)
//   endd   = <dS, E_end>                      (the chunk-end ddA_cumsum term)
// for the head kernel, in slots owned by (batch, head, chunk, tile).
//
// Ownership inside the block (Q/32 waves): wave w holds the causal dCB tiles
// of column tiles {w, T-1-w}, the dB rows of those column tiles and the dC
// rows of row tiles {w, T-1-w} (T = Q/16 tiles per side).
#include "ssd_problem.h"
#include "ssd_tiles.h"

namespace ssd {

template <typename T, int Q, int P, int NTG>
struct GroupCfg {
  static constexpr int T16 = Q / 16;
  static constexpr int W = T16 / 2;
  static constexpr int NTHR = W * WAVE;
  static constexpr int NCT = NTG / 16;
  static constexpr int VEC = Vec16<T>::N;
  static constexpr int LDP = P + VEC;
  static constexpr int LDQ = Q + VEC;
  static constexpr int NOWN = T16 + 1;  // causal tiles per wave
  // LDS layout (bytes)
  static constexpr size_t R1 = (size_t(2) * Q * LDP > size_t(W) * 16 * LDQ ? size_t(2) * Q * LDP
                                                                           : size_t(W) * 16 * LDQ) * sizeof(T);
  static constexpr size_t R2 = size_t(NTG) * LDQ * sizeof(T);
  static constexpr size_t R3 = size_t(2) * NTG * LDP * sizeof(T);
  // acs, dt, w, eA (4 Q floats), seg (Q ints), segstart (Q + 1 ints), red (W + 8 floats)
  static constexpr size_t R4 = size_t(4) * Q * 4 + size_t(Q) * 4 + size_t(Q + 1) * 4 + size_t(W + 8) * 4;
  static constexpr size_t OFF_R2 = R1;
  static constexpr size_t OFF_R3 = OFF_R2 + R2;
  static constexpr size_t OFF_R4 = OFF_R3 + R3;
  static constexpr size_t LDS = OFF_R4 + R4;
  static_assert(R1 % 16 == 0 && R2 % 16 == 0 && R3 % 16 == 0, "alignment");
};

template <int T16>
__device__ __forceinline__ void owned_tile(int w, int k, int& I, int& J) {
  if (k < T16 - w) {
    J = w;
    I = w + k;
  } else {
    J = T16 - 1 - w;
    I = J + (k - (T16 - w));
  }
}

template <typename T, int Q, int P, int NTG>
__global__ __launch_bounds__((GroupCfg<T, Q, P, NTG>::NTHR)) void k_group_bwd(Problem pb) {
  using Cf = GroupCfg<T, Q, P, NTG>;
  constexpr int T16 = Cf::T16, W = Cf::W, NTHR = Cf::NTHR, NCT = Cf::NCT, VEC = Cf::VEC;
  constexpr int LDP = Cf::LDP, LDQ = Cf::LDQ;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* s_xk = reinterpret_cast<T*>(smem);                 // [Q][LDP] x rows
  T* s_dyk = s_xk + Q * LDP;                             // [Q][LDP] dy rows
  T* s_sb = reinterpret_cast<T*>(smem);                  // phase 3: [W*16][LDQ] dCB rows
  T* s_ct = reinterpret_cast<T*>(smem + Cf::OFF_R2);     // [NTG][LDQ] C^T (phase 3: B^T)
  T* s_et = reinterpret_cast<T*>(smem + Cf::OFF_R3);     // [NTG][LDP] E^T
  T* s_dst = s_et + NTG * LDP;                           // [NTG][LDP] dS^T
  float* s_acs = reinterpret_cast<float*>(smem + Cf::OFF_R4);
  float* s_dt = s_acs + Q;
  float* s_w = s_dt + Q;
  float* s_eA = s_w + Q;
  int* s_seg = reinterpret_cast<int*>(s_eA + Q);
  int* s_segstart = s_seg + Q;  // [Q + 1]
  float* s_red = reinterpret_cast<float*>(s_segstart + Q + 1);

  const int ntiles = pb.ntg;
  const int64_t total = static_cast<int64_t>(pb.B) * pb.G * pb.nc * ntiles;
  const int64_t lb = xcd_logical_block(blockIdx.x, total);
  const int ntile = static_cast<int>(lb % ntiles);
  int64_t rest = lb / ntiles;
  const int g = static_cast<int>(rest % pb.G);
  rest /= pb.G;
  const int c = static_cast<int>(rest % pb.nc);
  const int b = static_cast<int>(rest / pb.nc);
  const int n0 = ntile * NTG;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r16 = l & 15, kg = l >> 4;
  const int64_t bc = static_cast<int64_t>(b) * pb.nc + c;
  const T* xg = static_cast<const T*>(pb.x);
  const T* dyg = static_cast<const T*>(pb.dy);
  const T* Bg = static_cast<const T*>(pb.Bm);
  const T* Cg = static_cast<const T*>(pb.Cm);

  // chunk metadata and C^T (shared by all heads)
  const int nstart = pb.cinfo[bc * CINFO + 0];
  const int seqbase = pb.cinfo[bc * CINFO + 3];
  for (int i = tid; i < Q; i += NTHR) s_seg[i] = pb.segpos[bc * Q + i];
  for (int v = tid; v < Q * NTG / VEC; v += NTHR) {
    const int i = v / (NTG / VEC), nv = v % (NTG / VEC), t = c * Q + i;
    uint4 u = zero_u4();
    if (t < pb.L) u = ld_global16(Cg + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + n0 + nv * VEC);
#pragma unroll
    for (int e = 0; e < VEC; ++e) s_ct[(nv * VEC + e) * LDQ + i] = vraw<T>(u, e);
  }
  if (tid == 0) s_segstart[0] = 0;
  __syncthreads();
  const int start0 = seg_rank(s_seg[0]);
  const int nseg = nstart + 1 - start0;
  const int lolast = seg_lo(s_seg[Q - 1]);
  for (int i = tid; i < Q; i += NTHR)
    if (i > 0 && seg_lo(s_seg[i]) == i) s_segstart[seg_rank(s_seg[i]) - start0] = i;
  if (tid == 0) s_segstart[nseg] = Q;

  f32x4_t dcb[Cf::NOWN];
  f32x4_t dbt[2][NCT];
  f32x4_t dc[2][NCT];
#pragma unroll
  for (int k = 0; k < Cf::NOWN; ++k) dcb[k] = zero4();
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nt = 0; nt < NCT; ++nt) {
      dbt[a][nt] = zero4();
      dc[a][nt] = zero4();
    }
  const int own0 = w, own1 = T16 - 1 - w;

  for (int hh = 0; hh < pb.hpg; ++hh) {
    const int h = g * pb.hpg + hh;
    const int64_t bhc = (static_cast<int64_t>(b) * pb.H + h) * pb.nc + c;
    __syncthreads();  // previous head's LDS reads are done
    for (int i = tid; i < Q; i += NTHR) {
      s_acs[i] = pb.acs[bhc * Q + i];
      s_dt[i] = pb.dtc[bhc * Q + i];
    }
    // x, dy rows (K-major along p)
    for (int v = tid; v < Q * P / VEC; v += NTHR) {
      const int j = v / (P / VEC), pv = v % (P / VEC), t = c * Q + j;
      uint4 ux = zero_u4(), ud = zero_u4();
      if (t < pb.L) {
        const int64_t off = ((static_cast<int64_t>(b) * pb.L + t) * pb.H + h) * P + pv * VEC;
        ux = ld_global16(xg + off);
        ud = ld_global16(dyg + off);
      }
      *reinterpret_cast<uint4*>(s_xk + j * LDP + pv * VEC) = ux;
      *reinterpret_cast<uint4*>(s_dyk + j * LDP + pv * VEC) = ud;
    }
    // dS^T for this dstate tile
    for (int v = tid; v < P * NTG; v += NTHR) {
      const int p = v / NTG, n = v % NTG;
      s_dst[n * LDP + p] = Elem<T>::from_f(pb.dstate[(bhc * P + p) * pb.N + n0 + n]);
    }
    __syncthreads();
    const float acs_end = s_acs[Q - 1];
    for (int i = tid; i < Q; i += NTHR) {
      s_w[i] = (i >= lolast) ? expf(acs_end - s_acs[i]) * s_dt[i] : 0.f;
      s_eA[i] = expf(s_acs[i]);
    }

    // dCB += W o (dy x^T) over the owned causal tiles
#pragma unroll
    for (int k = 0; k < Cf::NOWN; ++k) {
      int I, J;
      owned_tile<T16>(w, k, I, J);
      const f32x4_t m = tile_mma_kk<T>(zero4(), s_dyk + 16 * I * LDP, LDP, s_xk + 16 * J * LDP, LDP, 0, P);
      const int j = 16 * J + r16;
      const int loj = seg_lo(s_seg[j]);
      const float aj = s_acs[j], dtj = s_dt[j];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * kg + r;
        const bool ok = (j <= i) && (seg_lo(s_seg[i]) == loj);
        const float wgt = ok ? expf(s_acs[i] - aj) * dtj : 0.f;
        dcb[k][r] += wgt * m[r];
      }
    }
    __syncthreads();  // s_w / s_eA visible
    // dB^st (as its transpose, [n][j]) += w_j dS^T x_j
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int J = a == 0 ? own0 : own1;
      const float wj = s_w[16 * J + r16];
#pragma unroll
      for (int nt = 0; nt < NCT; ++nt) {
        const f32x4_t u = tile_mma_kk<T>(zero4(), s_dst + 16 * nt * LDP, LDP, s_xk + 16 * J * LDP, LDP, 0, P);
#pragma unroll
        for (int r = 0; r < 4; ++r) dbt[a][nt][r] += wj * u[r];
      }
    }

    // dC^off and the offd / endd partials, one pass per distinct entering state
    float offp[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
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
      const bool is_last = (hi == Q);
      const bool want_end = is_last && (nstart == 0 || rank > 0);
      __syncthreads();  // previous pass finished reading s_et
      for (int v = tid; v < P * NTG; v += NTHR) {
        const int p = v / NTG, n = v % NTG;
        float e = 0.f;
        if (esrc) e = esrc[p * pb.N + n0 + n];
        s_et[n * LDP + p] = Elem<T>::from_f(e);
        if (want_end && esrc) endp += pb.dstate[(bhc * P + p) * pb.N + n0 + n] * e;
      }
      __syncthreads();
      if (!esrc) continue;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int I = a == 0 ? own0 : own1;
        if (16 * I + 15 < lo || 16 * I >= hi) continue;
#pragma unroll
        for (int nt = 0; nt < NCT; ++nt) {
          const f32x4_t y = tile_mma_kk<T>(zero4(), s_dyk + 16 * I * LDP, LDP, s_et + 16 * nt * LDP, LDP, 0, P);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * I + 4 * kg + r;
            if (i >= lo && i < hi) {
              const float yv = y[r] * s_eA[i];
              dc[a][nt][r] += yv;
              offp[a][r] += yv * Elem<T>::to_f(s_ct[(16 * nt + r16) * LDQ + i]);
            }
          }
        }
      }
    }
    // offd partial: sum over the 16 lanes holding one row's columns
    const int64_t offd_base = (bhc * pb.ntg + ntile) * Q;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int I = a == 0 ? own0 : own1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = sum16(offp[a][r]);
        if (r16 == 0) pb.offd[offd_base + 16 * I + 4 * kg + r] = v;
      }
    }
    // endd partial: fixed-order block reduction
    {
      const float v = wave_sum(endp);
      if (l == 0) s_red[w] = v;
      __syncthreads();
      if (tid == 0) {
        float s = 0.f;
        for (int k = 0; k < W; ++k) s += s_red[k];
        pb.endd[bhc * pb.ntg + ntile] = s;
      }
    }
  }
  __syncthreads();

  // dB = dB^st + dCB^T C  (register-direct; output tile layout [n][j])
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int J = a == 0 ? own0 : own1;
#pragma unroll
    for (int nt = 0; nt < NCT; ++nt) {
      f32x4_t acc = dbt[a][nt];
#pragma unroll
      for (int k = 0; k < Cf::NOWN; ++k) {
        int I, JJ;
        owned_tile<T16>(w, k, I, JJ);
        if (JJ != J) continue;
        float av[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) av[r] = Elem<T>::to_f(s_ct[(16 * nt + r16) * LDQ + 16 * I + 4 * kg + r]);
        acc = Mma<T>::mma_regdirect(av, dcb[k], acc);
      }
      const int j = 16 * J + r16, t = c * Q + j;
      if (t < pb.L) {
        T* dst = static_cast<T*>(pb.dB) + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + n0 + 16 * nt + 4 * kg;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[r] = Elem<T>::from_f(acc[r]);
      }
    }
  }
  __syncthreads();  // C^T reads done; region 2 becomes B^T
  T* s_bt = s_ct;
  for (int v = tid; v < Q * NTG / VEC; v += NTHR) {
    const int j = v / (NTG / VEC), nv = v % (NTG / VEC), t = c * Q + j;
    uint4 u = zero_u4();
    if (t < pb.L) u = ld_global16(Bg + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + n0 + nv * VEC);
#pragma unroll
    for (int e = 0; e < VEC; ++e) s_bt[(nv * VEC + e) * LDQ + j] = vraw<T>(u, e);
  }

  // dC = dC^off + dCB B: half of the dCB row tiles per round through LDS
  constexpr int KS = Mma<T>::KSTEP;
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int I_lo = rd * W;
#pragma unroll
    for (int k = 0; k < Cf::NOWN; ++k) {
      int I, J;
      owned_tile<T16>(w, k, I, J);
      if (I < I_lo || I >= I_lo + W) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        s_sb[((I - I_lo) * 16 + 4 * kg + r) * LDQ + 16 * J + r16] = Elem<T>::from_f(dcb[k][r]);
    }
    // zero the columns past the diagonal tile that the K loop still reads
    {
      const int I = rd == 0 ? own0 : own1;
      const int kend = ((16 * (I + 1) + KS - 1) / KS) * KS;
      for (int e = l; e < 16 * (kend - 16 * (I + 1)); e += WAVE) {
        const int wdt = kend - 16 * (I + 1);
        const int ii = e / wdt, jj = 16 * (I + 1) + e % wdt;
        s_sb[((I - I_lo) * 16 + ii) * LDQ + jj] = Elem<T>::from_f(0.f);
      }
    }
    __syncthreads();
    {
      const int I = rd == 0 ? own0 : own1;
      const int kend = ((16 * (I + 1) + KS - 1) / KS) * KS;
#pragma unroll
      for (int nt = 0; nt < NCT; ++nt)
        dc[rd][nt] = tile_mma_kk<T>(dc[rd][nt], s_sb + (I - I_lo) * 16 * LDQ, LDQ, s_bt + 16 * nt * LDQ, LDQ, 0, kend);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int I = a == 0 ? own0 : own1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * I + 4 * kg + r, t = c * Q + i;
      if (t >= pb.L) continue;
      T* dst = static_cast<T*>(pb.dC) + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + n0;
#pragma unroll
      for (int nt = 0; nt < NCT; ++nt) dst[16 * nt + r16] = Elem<T>::from_f(dc[a][nt][r]);
    }
  }
}

int group_ntile(int N, bool io_bf16) {
  (void)io_bf16;
  if (N % 64 == 0) return 64;
  if (N % 32 == 0) return 32;
  return 16;
}

template <typename T, int Q, int P, int NTG>
static hipError_t launch_group_t(const Problem& pb, hipStream_t s) {
  using Cf = GroupCfg<T, Q, P, NTG>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_group_bwd<T, Q, P, NTG>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(Cf::LDS));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = static_cast<int64_t>(pb.B) * pb.G * pb.nc * pb.ntg;
  hipLaunchKernelGGL((k_group_bwd<T, Q, P, NTG>), dim3(static_cast<unsigned>(blocks)), dim3(Cf::NTHR),
                     Cf::LDS, s, pb);
  return hipGetLastError();
}

template <typename T, int Q, int P>
static hipError_t launch_group_qp(const Problem& pb, hipStream_t s) {
  const int ntg_w = pb.N / pb.ntg;
  if (ntg_w == 64) return launch_group_t<T, Q, P, 64>(pb, s);
  if (ntg_w == 32) return launch_group_t<T, Q, P, 32>(pb, s);
  if (ntg_w == 16) return launch_group_t<T, Q, P, 16>(pb, s);
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_group_any(const Problem& pb, hipStream_t s) {
#define SSD_GROUP_CASE(QQ, PP) \
  if (pb.Q == QQ && pb.P == PP) return launch_group_qp<T, QQ, PP>(pb, s);
  if constexpr (sizeof(T) == 2) {
    SSD_BF16_SHAPES(SSD_GROUP_CASE)
  } else {
    SSD_F32_SHAPES(SSD_GROUP_CASE)
  }
#undef SSD_GROUP_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_group_bwd(const Problem& pb, bool io_bf16, hipStream_t s) {
  return io_bf16 ? launch_group_any<bf16_t>(pb, s) : launch_group_any<float>(pb, s);
}

// LDS bytes of the group kernel for a compiled shape; ~0 when not compiled.
size_t group_lds_bytes(int Q, int P, int NTG, bool bf16) {
#define SSD_GROUP_LDS_B(QQ, PP)                                         \
  if (bf16 && Q == QQ && P == PP) {                                     \
    if (NTG == 64) return GroupCfg<bf16_t, QQ, PP, 64>::LDS;            \
    if (NTG == 32) return GroupCfg<bf16_t, QQ, PP, 32>::LDS;            \
    if (NTG == 16) return GroupCfg<bf16_t, QQ, PP, 16>::LDS;            \
  }
#define SSD_GROUP_LDS_F(QQ, PP)                                         \
  if (!bf16 && Q == QQ && P == PP) {                                    \
    if (NTG == 64) return GroupCfg<float, QQ, PP, 64>::LDS;             \
    if (NTG == 32) return GroupCfg<float, QQ, PP, 32>::LDS;             \
    if (NTG == 16) return GroupCfg<float, QQ, PP, 16>::LDS;             \
  }
  SSD_BF16_SHAPES(SSD_GROUP_LDS_B)
  SSD_F32_SHAPES(SSD_GROUP_LDS_F)
#undef SSD_GROUP_LDS_B
#undef SSD_GROUP_LDS_F
  return ~size_t(0);
}

}  // namespace ssd
