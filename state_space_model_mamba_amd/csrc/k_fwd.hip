// Forward of the SSD layer: y and the sequences' final states, in the same
// chunked form as the backward (the page "Deterministic bwd kernel for
// mamba2" lists the forward kernels chunk_cumsum, chunk_state, state passing
// and chunk_scan beside their backward twins).  The chunk preparation (Acs)
// and the forward state walk (Hin, the state entering every chunk) are the
// backward's own kernels; this file adds
//
//   k_seqstart  first position of every sequence (from the chunk records)
//   k_cbf       C B^T of each (batch, group, chunk), as transposed causal
//               tiles in the output kernel's (wave, tile) order
//   k_y         y_i = sum_{j <= i, same segment} CB[i,j] exp(Acs_i - Acs_j) dt_j x_j
//                     + exp(Acs_i) C_i . E_seg(i)  +  D x_i
//               per (batch, head, chunk); E is the state entering row i's
//               segment: Hin_c when the segment continues the chunk's
//               sequence, h0[s] when it starts sequence s
//   k_final     the state after each sequence's last position,
//               exp(Acs_e) E + sum_{j in the segment, j <= e} exp(Acs_e - Acs_j) dt_j x_j (outer) B_j
//
// Every output element has one writer; no atomics.
#include "ssd_problem.h"
#include "ssd_tiles.h"

namespace ssd {

// ----------------------------------------------------------------------------
// k_seqstart: seqstart[s] = b L + t of sequence s's first position
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_seqstart(Problem pb) {
  const int c = blockIdx.x, b = blockIdx.y;
  const int64_t bc = static_cast<int64_t>(b) * pb.nc + c;
  const int seqbase = pb.cinfo[bc * CINFO + 3];
  for (int i = threadIdx.x; i < pb.Q; i += blockDim.x) {
    const int t = c * pb.Q + i;
    if (t >= pb.L) continue;
    const int v = pb.segpos[bc * pb.Q + i];
    const bool start = i > 0 ? seg_lo(v) == i : seg_rank(v) > 0;
    if (!start) continue;
    const int s = seqbase + seg_rank(v) - 1;
    if (s >= 0 && s < pb.nseqs) pb.seqstart[s] = b * pb.L + t;
  }
}

// ----------------------------------------------------------------------------
// Row split of the causal 16 x 16 tiles: wave w owns row tiles w and T-1-w.
// Its tiles are row w's off-diagonal tiles (J = 0 .. w-1), row T-1-w's
// (J = 0 .. T-2-w), then the two diagonal tiles; T+1 tiles per wave.
// ----------------------------------------------------------------------------
template <int T16>
struct RowSplit {
  static constexpr int NOWN = T16 + 1;
  static __device__ __forceinline__ int row(int w, int a) { return a ? T16 - 1 - w : w; }
  // tile k of wave w: row slot a, row tile I, column tile J
  static __device__ __forceinline__ void tile(int w, int k, int& a, int& I, int& J) {
    if (k == T16 - 1) {
      a = 0;
      I = J = w;
    } else if (k == T16) {
      a = 1;
      I = J = T16 - 1 - w;
    } else if (k < w) {
      a = 0;
      I = w;
      J = k;
    } else {
      a = 1;
      I = T16 - 1 - w;
      J = k - w;
    }
  }
  // position of tile (row slot a, column J) in the wave's order
  static __device__ __forceinline__ int pos(int w, int a, int J) {
    if (J == row(w, a)) return T16 - 1 + a;
    return a ? w + J : J;
  }
};

template <typename T, int Q>
struct CbfCfg {
  static constexpr int T16 = Q / 16;
  static constexpr int W = Q / 32;
  static constexpr int NTHR = W * WAVE;
  static constexpr int NS = sizeof(T) == 2 ? 32 : 16;   // dstate slab
  static constexpr int VEC = Vec16<T>::N;
  static constexpr int LDN = NS + VEC;
  using Split = RowSplit<T16>;
};

// CB^T tiles: tile (I, J) holds CB^T[j][i] = B_j . C_i in the accumulator
// layout (lane: rows j = 16 J + 4 (lane / 16) + r, column i = 16 I + lane % 16).
template <typename T, int Q>
__global__ __launch_bounds__((CbfCfg<T, Q>::NTHR)) void k_cbf(Problem pb) {
  using Cf = CbfCfg<T, Q>;
  constexpr int T16 = Cf::T16, W = Cf::W, NTHR = Cf::NTHR, NS = Cf::NS, LDN = Cf::LDN;
  __shared__ __attribute__((aligned(16))) T s_c[Q * LDN];
  __shared__ __attribute__((aligned(16))) T s_b[Q * LDN];
  const int64_t total = static_cast<int64_t>(pb.B) * pb.G * pb.nc;
  const int64_t lb = xcd_logical_block(blockIdx.x, total);
  const int c = static_cast<int>(lb % pb.nc);
  const int64_t bg = lb / pb.nc;
  const int g = static_cast<int>(bg % pb.G), b = static_cast<int>(bg / pb.G);
  const int w = wave_id_s(), l = lane_id();
  const T* Bg = static_cast<const T*>(pb.Bm);
  const T* Cg = static_cast<const T*>(pb.Cm);
  auto row_src = [&](const T* base, int n0) {
    return [=, &pb](int i) -> const T* {
      const int t = c * Q + i;
      return t < pb.L ? base + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + n0 : nullptr;
    };
  };
  f32x4_t acc[T16 + 1];
#pragma unroll
  for (int k = 0; k < T16 + 1; ++k) acc[k] = zero4();
  RowStage<T, Q, NS, NTHR> st_c, st_b;
  st_c.load(row_src(Cg, 0));
  st_b.load(row_src(Bg, 0));
  for (int n0 = 0; n0 < pb.N; n0 += NS) {
    __syncthreads();
    st_c.store(s_c, LDN);
    st_b.store(s_b, LDN);
    __syncthreads();
    if (n0 + NS < pb.N) {
      st_c.load(row_src(Cg, n0 + NS));
      st_b.load(row_src(Bg, n0 + NS));
    }
#pragma unroll
    for (int k = 0; k < T16 + 1; ++k) {
      int a, I, J;
      Cf::Split::tile(w, k, a, I, J);
      acc[k] = tile_mma_kk<T>(acc[k], s_b + 16 * J * LDN, LDN, s_c + 16 * I * LDN, LDN, 0, NS);
    }
  }
  const int64_t bgc = (static_cast<int64_t>(b) * pb.G + g) * pb.nc + c;
  float* dst = pb.cbt + (bgc * W + w) * (T16 + 1) * 256 + l * 4;
#pragma unroll
  for (int k = 0; k < T16 + 1; ++k) *reinterpret_cast<f32x4_t*>(dst + k * 256) = acc[k];
}

// ----------------------------------------------------------------------------
// k_y
// ----------------------------------------------------------------------------
template <typename T, int Q, int P>
struct YCfg {
  static constexpr int T16 = Q / 16;
  static constexpr int W = Q / 32;
  static constexpr int NTHR = W * WAVE;
  static constexpr int PT = P / 16;
  static constexpr int VEC = Vec16<T>::N;
  static constexpr int LDX = P + VEC;                   // dt-scaled x rows [j][p]
  static constexpr int NS = sizeof(T) == 2 ? 32 : 16;   // dstate slab of the state term (divides N)
  static constexpr int LDC = NS + VEC;                  // C rows [i][n] of one slab
  static constexpr int LDE = NS + VEC;                  // E rows [p][n] of one slab
  using Split = RowSplit<T16>;
  static constexpr size_t LDS =
      (size_t(Q) * LDX + size_t(Q) * LDC + size_t(P) * LDE) * sizeof(T) + size_t(5 * Q + 1) * 4;
};

template <typename T, int Q, int P>
__global__ __launch_bounds__((YCfg<T, Q, P>::NTHR)) void k_y(Problem pb) {
  using Cf = YCfg<T, Q, P>;
  constexpr int T16 = Cf::T16, W = Cf::W, NTHR = Cf::NTHR, PT = Cf::PT, VEC = Cf::VEC;
  constexpr int LDX = Cf::LDX, NS = Cf::NS, LDC = Cf::LDC, LDE = Cf::LDE;
  constexpr int KW = Mma<T>::KW, KS = Mma<T>::KSTEP;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* s_xs = reinterpret_cast<T*>(smem);
  T* s_c = s_xs + Q * LDX;
  T* s_e = s_c + Q * LDC;
  float* s_acs = reinterpret_cast<float*>(s_e + P * LDE);
  float* s_dt = s_acs + Q;
  float* s_ej = s_dt + Q;
  int* s_seg = reinterpret_cast<int*>(s_ej + Q);
  int* s_segstart = s_seg + Q;   // Q + 1 entries (only the chunk's segments are used)

  const int64_t total = static_cast<int64_t>(pb.B) * pb.H * pb.nc;
  const int64_t lb = xcd_logical_block(blockIdx.x, total);
  const int hh = static_cast<int>(lb % pb.hpg);
  int64_t rest = lb / pb.hpg;
  const int c = static_cast<int>(rest % pb.nc);
  rest /= pb.nc;
  const int g = static_cast<int>(rest % pb.G), b = static_cast<int>(rest / pb.G);
  const int h = g * pb.hpg + hh;
  const int tid = threadIdx.x, w = wave_id_s(), l = lane_id(), r16 = l & 15, kg = l >> 4;
  const int64_t bc = static_cast<int64_t>(b) * pb.nc + c;
  const int64_t bhc = (static_cast<int64_t>(b) * pb.H + h) * pb.nc + c;
  const int64_t bgc = (static_cast<int64_t>(b) * pb.G + g) * pb.nc + c;
  const T* xg = static_cast<const T*>(pb.x);
  const T* Cg = static_cast<const T*>(pb.Cm);

  // per-position metadata; ej_j = exp(Acs_{16 J + 15} - Acs_j) (j in tile J)
  if (tid < Q) {
    const float acs_i = pb.acs[bhc * Q + tid];
    s_acs[tid] = acs_i;
    s_dt[tid] = pb.dtc[bhc * Q + tid];
    const int seg_i = pb.segpos[bc * Q + tid];
    s_seg[tid] = seg_i;
    const float acs_ref = __shfl(acs_i, l | 15, WAVE);
    s_ej[tid] = Elem<T>::exp(acs_ref - acs_i);
    if (tid > 0 && seg_lo(seg_i) == tid) s_segstart[seg_rank(seg_i) - seg_rank(pb.segpos[bc * Q])] = tid;
  }
  const int nstart = pb.cinfo[bc * CINFO + 0];
  const int seqbase = pb.cinfo[bc * CINFO + 3];
  const int rank0 = seg_rank(pb.segpos[bc * Q]);   // 1 when a sequence starts at position 0
  const int nseg = nstart + 1 - rank0;
  const int lolast = seg_lo(pb.segpos[bc * Q + Q - 1]);
  const bool uniform = __builtin_amdgcn_readfirstlane(lolast) == 0;
  if (tid == 0) {
    s_segstart[0] = 0;
    s_segstart[nseg] = Q;
  }
  // x rows -> LDS scaled by dt (rows past L are zero)
  {
    RowStage<T, Q, P, NTHR> st_x;
    st_x.load([&](int i) -> const T* {
      const int t = c * Q + i;
      return t < pb.L ? xg + ((static_cast<int64_t>(b) * pb.L + t) * pb.H + h) * P : nullptr;
    });
    __syncthreads();   // s_dt
#pragma unroll
    for (int k = 0; k < st_x.IT; ++k) {
      const int v = tid + k * NTHR;
      if (v < st_x.NV) {
        const int i = v / st_x.CV, c0 = (v % st_x.CV) * VEC;
        const float d = s_dt[i];
        T o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = Elem<T>::from_f(vget<T>(st_x.buf[k], e) * d);
        *reinterpret_cast<uint4*>(s_xs + i * LDX + c0) = *reinterpret_cast<const uint4*>(o);
      }
    }
  }
  __syncthreads();

  // ---- intra-chunk term, row tile by row tile (slot a = 0: row w, 1: row T-1-w)
  f32x4_t y0[PT], y1[PT];   // y^T tiles of the two owned row tiles: [p][i]
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) y0[pt] = y1[pt] = zero4();
  const float* cbw = pb.cbt + (bgc * W + w) * (T16 + 1) * 256 + l * 4;
  auto tile = [&](int a, int I, int J, f32x4_t(&yt)[PT]) {
    const f32x4_t cbT = *reinterpret_cast<const f32x4_t*>(cbw + Cf::Split::pos(w, a, J) * 256);
    const int i = 16 * I + r16;
    const float ai = s_acs[i];
    f32x4_t e4;
    if (uniform && J < I) {
      const float ei = Elem<T>::exp(ai - s_acs[16 * J + 15]);
      const f32x4_t ej = *reinterpret_cast<const f32x4_t*>(s_ej + 16 * J + 4 * kg);
#pragma unroll
      for (int r = 0; r < 4; ++r) e4[r] = ei * ej[r];
    } else {
      const int loi = seg_lo(s_seg[i]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * J + 4 * kg + r;
        const bool ok = (j <= i) & (seg_lo(s_seg[j]) == loi);
        const float e = Elem<T>::exp(ok ? ai - s_acs[j] : 0.f);
        e4[r] = ok ? e : 0.f;
      }
    }
    f32x4_t gT;
#pragma unroll
    for (int r = 0; r < 4; ++r) gT[r] = cbT[r] * e4[r];
    const typename Mma<T>::rfrag gf = Mma<T>::rfrag_from_acc(gT);
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
      yt[pt] = Mma<T>::mma_rd(Mma<T>::rfrag_load_kn(s_xs + 16 * J * LDX + 16 * pt, LDX), gf, yt[pt]);
  };
  {
    const int I0 = Cf::Split::row(w, 0), I1 = Cf::Split::row(w, 1);
    for (int J = 0; J <= I0; ++J) tile(0, I0, J, y0);
    for (int J = 0; J <= I1; ++J) tile(1, I1, J, y1);
  }

  // ---- state term: exp(Acs_i) C_i . E_seg(i), segment by segment, dstate slab by slab
  f32x4_t z0[PT], z1[PT];
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) z0[pt] = z1[pt] = zero4();
  for (int m = 0; m < nseg; ++m) {
    const int lo = s_segstart[m], hi = s_segstart[m + 1];
    const int rank = seg_rank(s_seg[lo]);
    // entering state: Hin_c (I/O dtype) or h0[s] (fp32) or none
    const T* e_t = nullptr;
    const float* e_f = nullptr;
    if (rank == 0) {
      e_t = static_cast<const T*>(pb.hin) + bhc * P * pb.N;
    } else if (pb.h0) {
      const int s = clamp_seq(seqbase + rank - 1, pb.nseqs);
      e_f = pb.h0 + (static_cast<int64_t>(s) * pb.H + h) * P * pb.N;
    }
    if (!e_t && !e_f) continue;   // (uniform)
    for (int n0 = 0; n0 < pb.N; n0 += NS) {
      RowStage<T, Q, NS, NTHR> st_c;
      RowStage<T, P, NS, NTHR> st_e;
      st_c.load([&](int i) -> const T* {
        const int t = c * Q + i;
        return t < pb.L ? Cg + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + n0 : nullptr;
      });
      if (e_t)
        st_e.load([&](int p) -> const T* { return e_t + static_cast<int64_t>(p) * pb.N + n0; });
      else
        st_e.load_from_f32([&](int p) -> const float* { return e_f + static_cast<int64_t>(p) * pb.N + n0; });
      __syncthreads();   // the previous slab is read
      st_c.store(s_c, LDC);
      st_e.store(s_e, LDE);
      __syncthreads();
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int I = Cf::Split::row(w, a);
        if (16 * I + 15 < lo || 16 * I >= hi) continue;   // (uniform)
        const int i = 16 * I + r16;
        const bool in_seg = i >= lo && i < hi;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          f32x4_t v = a ? z1[pt] : z0[pt];
#pragma unroll
          for (int k0 = 0; k0 < NS; k0 += KS) {
            const auto af = Mma<T>::load_k(s_e + (16 * pt + r16) * LDE + kg * KW + k0);
            auto bf = Mma<T>::load_k(s_c + i * LDC + kg * KW + k0);
            if (!in_seg) bf = Mma<T>::zero();
            v = Mma<T>::mma(af, bf, v);
          }
          if (a) z1[pt] = v; else z0[pt] = v;
        }
      }
    }
  }

  // ---- epilogue: y = intra + exp(Acs_i) state + D x
  const float Dh = pb.D ? pb.D[h] : 0.f;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int I = Cf::Split::row(w, a);
    const int i = 16 * I + r16, t = c * Q + i;
    if (t >= pb.L) continue;
    const float ei = Elem<T>::exp(s_acs[i]);
    const int64_t row = ((static_cast<int64_t>(b) * pb.L + t) * pb.H + h) * P;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      const f32x4_t yv = a ? y1[pt] : y0[pt];
      const f32x4_t zv = a ? z1[pt] : z0[pt];
      const f32x4_t xv = load4f<T>(xg + row + 16 * pt + 4 * kg);
      f32x4_t o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = yv[r] + ei * zv[r] + Dh * xv[r];
      store4f<T>(static_cast<T*>(pb.y) + row + 16 * pt + 4 * kg, o);
    }
  }
}

// ----------------------------------------------------------------------------
// k_final: state after the last position of each sequence
// ----------------------------------------------------------------------------
template <typename T, int Q, int P, int NT>
struct FinalCfg {
  static constexpr int NTHR = 256;
  static constexpr int NW = NTHR / WAVE;
  static constexpr int VEC = Vec16<T>::N;
  using XTile = KnTile<T, P>;    // scaled x rows [j][p]
  using BTile = KnTile<T, NT>;   // B rows [j][n]
  static constexpr int PT = P / 16, NTT = NT / 16, NTILE = PT * NTT;
  static constexpr int TPW = (NTILE + NW - 1) / NW;
};

template <typename T, int Q, int P, int NT>
__global__ __launch_bounds__((FinalCfg<T, Q, P, NT>::NTHR)) void k_final(Problem pb) {
  using Cf = FinalCfg<T, Q, P, NT>;
  constexpr int NTHR = Cf::NTHR, VEC = Cf::VEC;
  __shared__ __attribute__((aligned(16))) T s_x[Q * Cf::XTile::LD];
  __shared__ __attribute__((aligned(16))) T s_b[Q * Cf::BTile::LD];
  __shared__ float s_w[Q];
  const int ntiles = pb.N / NT;
  const int ntile = blockIdx.x % ntiles;
  const int h = (blockIdx.x / ntiles) % pb.H;
  const int s = blockIdx.x / ntiles / pb.H;
  const int n0 = ntile * NT, g = h / pb.hpg;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r16 = l & 15, kg = l >> 4;
  float* out = pb.final + (static_cast<int64_t>(s) * pb.H + h) * P * pb.N + n0;

  // sequences that exist: the starts counted by the chunk records
  const int64_t lastbc = static_cast<int64_t>(pb.B) * pb.nc - 1;
  const int nseq = pb.cinfo[lastbc * CINFO + 3] + pb.cinfo[lastbc * CINFO + 0];
  if (s >= nseq) {   // (named by nseqs but absent from seq_idx): zeros
    for (int v = tid; v < P * NT; v += NTHR) out[static_cast<int64_t>(v / NT) * pb.N + v % NT] = 0.f;
    return;
  }
  const int st0 = pb.seqstart[s];
  const int b = st0 / pb.L;
  int tend = pb.L - 1;
  if (s + 1 < nseq && s + 1 < pb.nseqs) {
    const int st1 = pb.seqstart[s + 1];
    if (st1 / pb.L == b) tend = st1 % pb.L - 1;
  }
  const int ce = tend / Q, e = tend % Q;
  const int64_t bc = static_cast<int64_t>(b) * pb.nc + ce;
  const int64_t bhc = (static_cast<int64_t>(b) * pb.H + h) * pb.nc + ce;
  const int lo = seg_lo(pb.segpos[bc * Q + e]);
  const bool continues = lo == 0 && seg_rank(pb.segpos[bc * Q]) == 0;
  const float acs_e = pb.acs[bhc * Q + e];
  if (tid < Q) {
    const float acs_j = pb.acs[bhc * Q + tid];
    s_w[tid] = (tid >= lo && tid <= e) ? Elem<T>::exp(acs_e - acs_j) * pb.dtc[bhc * Q + tid] : 0.f;
  }
  __syncthreads();
  // x rows scaled by w, B rows of this state tile
  {
    const T* xg = static_cast<const T*>(pb.x);
    const T* Bg = static_cast<const T*>(pb.Bm);
    RowStage<T, Q, P, NTHR> st_x;
    RowStage<T, Q, NT, NTHR> st_b;
    st_x.load([&](int j) -> const T* {
      const int t = ce * Q + j;
      return t < pb.L ? xg + ((static_cast<int64_t>(b) * pb.L + t) * pb.H + h) * P : nullptr;
    });
    st_b.load([&](int j) -> const T* {
      const int t = ce * Q + j;
      return t < pb.L ? Bg + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + n0 : nullptr;
    });
#pragma unroll
    for (int k = 0; k < st_x.IT; ++k) {
      const int v = tid + k * NTHR;
      if (v < st_x.NV) {
        const int j = v / st_x.CV, c0 = (v % st_x.CV) * VEC;
        const float sc = s_w[j];
        T o[VEC];
#pragma unroll
        for (int q = 0; q < VEC; ++q) o[q] = Elem<T>::from_f(vget<T>(st_x.buf[k], q) * sc);
        *reinterpret_cast<uint4*>(s_x + Cf::XTile::at(j, c0)) = *reinterpret_cast<const uint4*>(o);
      }
    }
#pragma unroll
    for (int k = 0; k < st_b.IT; ++k) {
      const int v = tid + k * NTHR;
      if (v < st_b.NV) {
        const int j = v / st_b.CV, c0 = (v % st_b.CV) * VEC;
        *reinterpret_cast<uint4*>(s_b + Cf::BTile::at(j, c0)) = st_b.buf[k];
      }
    }
  }
  __syncthreads();
  // entering state of the segment: Hin (I/O dtype) or h0[s] (fp32) or none
  const T* e_t = continues ? static_cast<const T*>(pb.hin) + bhc * P * pb.N + n0 : nullptr;
  const float* e_f = (!continues && pb.h0) ? pb.h0 + (static_cast<int64_t>(s) * pb.H + h) * P * pb.N + n0 : nullptr;
  const float decay = Elem<T>::exp(acs_e);
  const int kb = (lo / Mma<T>::KSTEP) * Mma<T>::KSTEP;
#pragma unroll
  for (int k = 0; k < Cf::TPW; ++k) {
    const int tl = w + Cf::NW * k;
    if (tl >= Cf::NTILE) break;
    const int pt = tl / Cf::NTT, nt = tl % Cf::NTT;
    f32x4_t S = zero4();
    for (int k0 = kb; k0 <= e; k0 += Mma<T>::KSTEP)
      S = Mma<T>::mma(Cf::XTile::frag(s_x, pt * 16, k0), Cf::BTile::frag(s_b, nt * 16, k0), S);
    const int n = nt * 16 + r16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = pt * 16 + 4 * kg + r;
      float init = 0.f;
      if (e_t) init = Elem<T>::to_f(e_t[static_cast<int64_t>(p) * pb.N + n]);
      if (e_f) init = e_f[static_cast<int64_t>(p) * pb.N + n];
      out[static_cast<int64_t>(p) * pb.N + n] = S[r] + decay * init;
    }
  }
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------
template <typename T, int Q, int P>
static hipError_t launch_fwd_qp(const Problem& pb, hipStream_t s) {
  {
    const int64_t blocks = static_cast<int64_t>(pb.B) * pb.G * pb.nc;
    hipLaunchKernelGGL((k_cbf<T, Q>), dim3(static_cast<unsigned>(blocks)), dim3(CbfCfg<T, Q>::NTHR), 0, s, pb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    using Cf = YCfg<T, Q, P>;
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_y<T, Q, P>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(Cf::LDS));
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    const int64_t blocks = static_cast<int64_t>(pb.B) * pb.H * pb.nc;
    hipLaunchKernelGGL((k_y<T, Q, P>), dim3(static_cast<unsigned>(blocks)), dim3(Cf::NTHR), Cf::LDS, s, pb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (pb.final) {
    const int nt = pb.N % 64 == 0 ? 64 : (pb.N % 32 == 0 ? 32 : 16);
    const int64_t blocks = static_cast<int64_t>(pb.nseqs) * pb.H * (pb.N / nt);
    if (nt == 64)
      hipLaunchKernelGGL((k_final<T, Q, P, 64>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, pb);
    else if (nt == 32)
      hipLaunchKernelGGL((k_final<T, Q, P, 32>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, pb);
    else
      hipLaunchKernelGGL((k_final<T, Q, P, 16>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, pb);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename T>
static hipError_t launch_fwd_any(const Problem& pb, hipStream_t s) {
#define SSD_FWD_CASE(QQ, PP) \
  if (pb.Q == QQ && pb.P == PP) return launch_fwd_qp<T, QQ, PP>(pb, s);
  if constexpr (sizeof(T) == 2) {
    SSD_BF16_SHAPES(SSD_FWD_CASE)
  } else {
    SSD_F32_SHAPES(SSD_FWD_CASE)
  }
#undef SSD_FWD_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_seqstart(const Problem& pb, hipStream_t s) {
  hipLaunchKernelGGL(k_seqstart, dim3(pb.nc, pb.B), dim3(256), 0, s, pb);
  return hipGetLastError();
}

hipError_t launch_fwd_out(const Problem& pb, bool io_bf16, hipStream_t s) {
  return io_bf16 ? launch_fwd_any<bf16_t>(pb, s) : launch_fwd_any<float>(pb, s);
}

size_t fwd_lds_bytes(int Q, int P, bool bf16) {
#define SSD_Y_LDS_B(QQ, PP) \
  if (bf16 && Q == QQ && P == PP) return YCfg<bf16_t, QQ, PP>::LDS;
#define SSD_Y_LDS_F(QQ, PP) \
  if (!bf16 && Q == QQ && P == PP) return YCfg<float, QQ, PP>::LDS;
  SSD_BF16_SHAPES(SSD_Y_LDS_B)
  SSD_F32_SHAPES(SSD_Y_LDS_F)
#undef SSD_Y_LDS_B
#undef SSD_Y_LDS_F
  return ~size_t(0);
}

}  // namespace ssd
