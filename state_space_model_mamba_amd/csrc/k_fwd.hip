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
//               (times silu(z_i) with an output gate; in the backward's gate
//               pass it writes dout silu(z) and dz instead of y)
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

// sigmoid(z) of the gate.  With bf16 I/O from the hardware exponential and
// reciprocal (v_rcp_f32, 1 ulp): their error is far below the bf16 rounding
// of the gate's outputs, and an IEEE division costs about ten instructions
// per element.  With fp32 I/O the library expf and a correctly rounded division.
template <typename T>
__device__ __forceinline__ float gate_sigmoid(float z) {
  if constexpr (sizeof(T) == 2) return __builtin_amdgcn_rcpf(1.f + __expf(-z));
  else return 1.f / (1.f + expf(-z));
}

// The backward's gate pass for one 16-byte piece of dout (du), z (zu) and y
// (yu, rounded to the I/O dtype): the gated dy = dout silu(z) and
// dz = dout y sigmoid(z) (1 + z (1 - sigmoid(z))), rounded to the I/O dtype.
template <typename T>
__device__ __forceinline__ void gate_grads(uint4 du, uint4 zu, uint4 yu, T* dy_out, T* dz_out) {
  constexpr int VEC = Vec16<T>::N;
  T dyo[VEC], dzo[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const float zz = vget<T>(zu, e), sg = gate_sigmoid<T>(zz), dv = vget<T>(du, e);
    dyo[e] = Elem<T>::from_f(dv * zz * sg);
    dzo[e] = Elem<T>::from_f(dv * vget<T>(yu, e) * sg * (1.f + zz * (1.f - sg)));
  }
  *reinterpret_cast<uint4*>(dy_out) = *reinterpret_cast<const uint4*>(dyo);
  *reinterpret_cast<uint4*>(dz_out) = *reinterpret_cast<const uint4*>(dzo);
}

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

// One CB^T tile as a lane holds it between k_cbf and k_y: the accumulator's
// four values, as bf16 pairs on the bf16 path (the MFMA operand they scale
// is rounded to bf16 anyway) and as fp32 on the fp32 path.
template <typename T> struct CbPack;
template <> struct CbPack<bf16_t> {
  using type = uint2;
  static __device__ __forceinline__ type pack(f32x4_t v) {
    return uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
  static __device__ __forceinline__ f32x4_t unpack(type u) {
    return f32x4_t{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                   __uint_as_float(u.y & 0xffff0000u)};
  }
};
template <> struct CbPack<float> {
  using type = f32x4_t;
  static __device__ __forceinline__ type pack(f32x4_t v) { return v; }
  static __device__ __forceinline__ f32x4_t unpack(type v) { return v; }
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
// layout (lane: rows j = 16 J + 4 (lane / 16) + r, column i = 16 I + lane % 16),
// stored per lane in the CbPack format.
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
  using Pk = CbPack<T>;
  typename Pk::type* dst = reinterpret_cast<typename Pk::type*>(pb.cbt) + (bgc * W + w) * (T16 + 1) * WAVE + l;
#pragma unroll
  for (int k = 0; k < T16 + 1; ++k) dst[k * WAVE] = Pk::pack(acc[k]);
}

// ----------------------------------------------------------------------------
// k_y: one block per (batch, group, chunk, slice of the group's heads).  The
// group's C rows and C B^T tiles do not depend on the head, so the block
// stages them once (C in LDS when one dstate slab holds all of N, the wave's
// CB^T tiles in registers) and walks its heads, reading per head only x, the
// entering state and the per-position tables, and requesting the next head's
// while it computes the current one.
// ----------------------------------------------------------------------------
template <typename T, int Q, int P, int NS>
struct YCfg {
  static constexpr int T16 = Q / 16;
  static constexpr int W = Q / 32;
  static constexpr int NTHR = W * WAVE;
  static constexpr int PT = P / 16;
  static constexpr int VEC = Vec16<T>::N;
  static constexpr int LDX = P + VEC;    // x rows [j][p]
  static constexpr int LDC = NS + VEC;   // C rows [i][n] of one dstate slab
  static constexpr int LDE = NS + VEC;   // E rows [p][n] of one dstate slab
  static constexpr int NOWN = T16 + 1;
  using Split = RowSplit<T16>;
  // x, C, E; acs, dt, exp-table, segpos (Q each), segment starts (Q + 1) and
  // the head's per-channel D (P)
  static constexpr size_t LDS =
      (size_t(Q) * LDX + size_t(Q) * LDC + size_t(P) * LDE) * sizeof(T) + size_t(5 * Q + 4 + P) * 4;
};

// The intra-chunk term over the wave's tiles (row split order), added to the
// y^T tiles of the wave's two row tiles: ya (row w) and yb (row T-1-w).  The
// decay and dt_j multiply the CB^T tile before it becomes the MFMA operand:
// G^T[j][i] = CB[i,j] exp(Acs_i - Acs_j) dt_j.  Row w's off-diagonal tiles
// come first, then row T-1-w's, then the two diagonal tiles; which
// accumulator an early tile feeds is a wave-uniform branch around its MFMAs.
// UNI: the chunk has one segment, so an off-diagonal decay factors through the
// column table ejdt[j] = exp(Acs_{16J+15} - Acs_j) dt_j; the two versions keep
// the unrolled sequence free of branches on it.
template <typename T, int P, bool UNI>
struct YTileOps {   // a tile's LDS operands, requested one tile ahead
  float aref;        // UNI: Acs at the end of the column tile
  f32x4_t t0;        // UNI: ejdt of the lane's 4 columns; else their Acs
  f32x4_t dt4;       // (general) dt of the lane's 4 columns
  int4 sj;           // (general) segpos of the lane's 4 columns
  typename Mma<T>::rfrag xf[P / 16];
};

template <typename T, int Q, int P, int NS, bool UNI>
__device__ __forceinline__ void y_tiles(const typename CbPack<T>::type (&cb)[Q / 16 + 1], f32x4_t (&ya)[P / 16],
                                        f32x4_t (&yb)[P / 16], const T* s_x, const float* s_acs,
                                        const float* s_dt, const float* s_ejdt, const int* s_seg, int w, int l) {
  using Cf = YCfg<T, Q, P, NS>;
  constexpr int T16 = Cf::T16, PT = Cf::PT, LDX = Cf::LDX;
  const int r16 = l & 15, kg = l >> 4;
  // per-row values: Acs_i and (general) the segment start of i
  const int iw = 16 * Cf::Split::row(w, 0) + r16, iv = 16 * Cf::Split::row(w, 1) + r16;
  const float ai_w = s_acs[iw], ai_v = s_acs[iv];
  int lo_w = 0, lo_v = 0;
  if (!UNI) {
    lo_w = seg_lo(s_seg[iw]);
    lo_v = seg_lo(s_seg[iv]);
  }
  auto load_ops = [&](int k) {
    int a, I, J;
    Cf::Split::tile(w, k, a, I, J);
    const bool diag = k >= T16 - 1;
    YTileOps<T, P, UNI> o;
    if (UNI && !diag) {
      o.aref = s_acs[16 * J + 15];
      o.t0 = *reinterpret_cast<const f32x4_t*>(s_ejdt + 16 * J + 4 * kg);
    } else {
      o.t0 = *reinterpret_cast<const f32x4_t*>(s_acs + 16 * J + 4 * kg);
      o.dt4 = *reinterpret_cast<const f32x4_t*>(s_dt + 16 * J + 4 * kg);
      o.sj = *reinterpret_cast<const int4*>(s_seg + 16 * J + 4 * kg);
    }
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) o.xf[pt] = Mma<T>::rfrag_load_kn(s_x + 16 * J * LDX + 16 * pt, LDX);
    return o;
  };
  YTileOps<T, P, UNI> nxt = load_ops(0);
#pragma clang loop unroll(full)
  for (int k = 0; k < Cf::NOWN; ++k) {
    const YTileOps<T, P, UNI> cur = nxt;
    if (k + 1 < Cf::NOWN) nxt = load_ops(k + 1);
    int a, I, J;
    Cf::Split::tile(w, k, a, I, J);
    const bool diag = k >= T16 - 1;   // a constant once unrolled
    const float ai = a ? ai_v : ai_w;
    f32x4_t e4;
    if (UNI && !diag) {
      const float ei = Elem<T>::exp(ai - cur.aref);
#pragma unroll
      for (int r = 0; r < 4; ++r) e4[r] = ei * cur.t0[r];
    } else {
      // causal and same-segment mask
      const int i = 16 * I + r16;
      const int loi = UNI ? 0 : (a ? lo_v : lo_w);
      const int sjv[4] = {cur.sj.x, cur.sj.y, cur.sj.z, cur.sj.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * J + 4 * kg + r;
        const bool ok = (j <= i) & (UNI || seg_lo(sjv[r]) == loi);
        const float e = Elem<T>::exp(ok ? ai - cur.t0[r] : 0.f);
        e4[r] = ok ? e * cur.dt4[r] : 0.f;
      }
    }
    const f32x4_t cbk = CbPack<T>::unpack(cb[k]);
    f32x4_t gT;
#pragma unroll
    for (int r = 0; r < 4; ++r) gT[r] = cbk[r] * e4[r];
    const typename Mma<T>::rfrag gf = Mma<T>::rfrag_from_acc(gT);
    const bool row_w = k == T16 - 1 || (k < T16 / 2 && k < w);
    if (row_w) {
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) ya[pt] = Mma<T>::mma_rd(cur.xf[pt], gf, ya[pt]);
    } else {
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) yb[pt] = Mma<T>::mma_rd(cur.xf[pt], gf, yb[pt]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <typename T, int Q, int P, int NS, bool MULTI>
__global__ __launch_bounds__((YCfg<T, Q, P, NS>::NTHR)) void k_y(Problem pb) {
  using Cf = YCfg<T, Q, P, NS>;
  constexpr int T16 = Cf::T16, W = Cf::W, NTHR = Cf::NTHR, PT = Cf::PT;
  constexpr int LDX = Cf::LDX, LDC = Cf::LDC, LDE = Cf::LDE;
  constexpr int KW = Mma<T>::KW, KS = Mma<T>::KSTEP;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* const s_x0 = reinterpret_cast<T*>(smem);
  T* const s_c0 = s_x0 + Q * LDX;
  T* const s_e0 = s_c0 + Q * LDC;
  float* const s_acs0 = reinterpret_cast<float*>(s_e0 + P * LDE);
  float* const s_dt0 = s_acs0 + Q;
  float* const s_ejdt0 = s_dt0 + Q;
  int* const s_seg0 = reinterpret_cast<int*>(s_ejdt0 + Q);
  int* const s_segstart0 = s_seg0 + Q;   // Q + 1 entries (only the chunk's segments are used)
  float* const s_D = reinterpret_cast<float*>(s_segstart0 + Q + 4);   // per-channel D of the head (16-byte aligned)

  // block -> (batch, group, chunk, head slice); the slices of one (b, g, c)
  // are consecutive logical blocks and so share an XCD's L2
  const int64_t total = gridDim.x;
  const int nsplit = static_cast<int>(total / (static_cast<int64_t>(pb.B) * pb.G * pb.nc));
  const int64_t lb = xcd_logical_block(blockIdx.x, total);
  const int split = static_cast<int>(lb % nsplit);
  int64_t rest = lb / nsplit;
  const int c = static_cast<int>(rest % pb.nc);
  rest /= pb.nc;
  const int g = static_cast<int>(rest % pb.G), b = static_cast<int>(rest / pb.G);
  const int hper = (pb.hpg + nsplit - 1) / nsplit;
  const int h_begin = g * pb.hpg + split * hper;
  const int h_end = g * pb.hpg + min(pb.hpg, (split + 1) * hper);
  if (h_begin >= h_end) return;   // (uniform)
  const int tid = threadIdx.x, w0 = wave_id_s(), l0 = lane_id();
  const int64_t bc = static_cast<int64_t>(b) * pb.nc + c;
  const int64_t bgc = (static_cast<int64_t>(b) * pb.G + g) * pb.nc + c;
  const T* xg = static_cast<const T*>(pb.x);
  const T* Cg = static_cast<const T*>(pb.Cm);
  // MULTI: N spans several dstate slabs and C is restaged slab by slab for
  // every head; otherwise N == NS and C stays in LDS

  // chunk-wide segment structure
  const int nstart = pb.cinfo[bc * CINFO + 0];
  const int seqbase = pb.cinfo[bc * CINFO + 3];
  const int rank0 = seg_rank(pb.segpos[bc * Q]);   // 1 when a sequence starts at position 0
  const int nseg = nstart + 1 - rank0;
  const int lolast = seg_lo(pb.segpos[bc * Q + Q - 1]);
  const bool uniform = __builtin_amdgcn_readfirstlane(lolast) == 0;
  // entering state of segment m for head h: Hin_c (I/O dtype), h0[s] (fp32), or none
  auto e_src = [&](int h, int m, const T*& e_t, const float*& e_f) {
    e_t = nullptr;
    e_f = nullptr;
    const int rank = m == 0 ? rank0 : rank0 + m;
    if (rank == 0) {
      e_t = static_cast<const T*>(pb.hin) + ((static_cast<int64_t>(b) * pb.H + h) * pb.nc + c) * P * pb.N;
    } else if (pb.h0) {
      const int s = clamp_seq(seqbase + rank - 1, pb.nseqs);
      e_f = pb.h0 + (static_cast<int64_t>(s) * pb.H + h) * P * pb.N;
    }
  };
  auto c_row = [&](int n0) {
    return [=, &pb](int i) -> const T* {
      const int t = c * Q + i;
      return t < pb.L ? Cg + ((static_cast<int64_t>(b) * pb.L + t) * pb.G + g) * pb.N + n0 : nullptr;
    };
  };
  auto load_e = [&](RowStage<T, P, NS, NTHR>& st, const T* e_t, const float* e_f, int n0) {
    if (e_t)
      st.load([=, &pb](int p) -> const T* { return e_t + static_cast<int64_t>(p) * pb.N + n0; });
    else if (e_f)
      st.load_from_f32([=, &pb](int p) -> const float* { return e_f + static_cast<int64_t>(p) * pb.N + n0; });
  };
  // segment 0 continues the chunk's sequence: its entering state Hin_c comes
  // with the head's prefetch (any other entering state is staged in the state
  // loop; a single load path keeps the prefetch free of waits)
  const bool e0_hin = rank0 == 0;

  // the per-head inputs, requested one head ahead
  float pf_acs = 0.f, pf_dt = 0.f;
  RowStage<T, Q, P, NTHR> st_x;
  RowStage<T, P, NS, NTHR> st_e;
  auto prefetch = [&](int h) {
    const int64_t bhc = (static_cast<int64_t>(b) * pb.H + h) * pb.nc + c;
    if (tid < Q) {
      pf_acs = pb.acs[bhc * Q + tid];
      pf_dt = pb.dtc[bhc * Q + tid];
    }
    st_x.load([&](int i) -> const T* {
      const int t = c * Q + i;
      return t < pb.L ? xg + ((static_cast<int64_t>(b) * pb.L + t) * pb.H + h) * P : nullptr;
    });
    if (e0_hin) {
      const T* e_t = static_cast<const T*>(pb.hin) + bhc * P * pb.N;
      st_e.load([=, &pb](int p) -> const T* { return e_t + static_cast<int64_t>(p) * pb.N; });
    }
  };

  // head-independent inputs: the wave's CB^T tiles, C (one slab), segments
  typename CbPack<T>::type cb[T16 + 1];
  {
    const auto* cbw = reinterpret_cast<const typename CbPack<T>::type*>(pb.cbt) + (bgc * W + w0) * (T16 + 1) * WAVE + l0;
#pragma unroll
    for (int k = 0; k < T16 + 1; ++k) cb[k] = cbw[k * WAVE];
  }
  RowStage<T, Q, NS, NTHR> st_c;
  if (!MULTI) st_c.load(c_row(0));
  prefetch(h_begin);
  if (tid < Q) {
    const int v = pb.segpos[bc * Q + tid];
    s_seg0[tid] = v;
    if (tid > 0 && seg_lo(v) == tid) s_segstart0[seg_rank(v) - rank0] = tid;
  }
  if (tid == 0) {
    s_segstart0[0] = 0;
    s_segstart0[nseg] = Q;
  }
  if (!MULTI) st_c.store(s_c0, LDC);

  for (int h = h_begin; h < h_end; ++h) {
    // per-iteration LDS bases keep the compiler from hoisting per-tile
    // addresses and masks out of the head loop (they would hold registers)
    const int oz = opaque_zero();
    T* const s_x = s_x0 + oz;
    T* const s_c = s_c0 + oz;
    T* const s_e = s_e0 + oz;
    float* const s_acs = s_acs0 + oz;
    float* const s_dt = s_dt0 + oz;
    float* const s_ejdt = s_ejdt0 + oz;
    int* const s_seg = s_seg0 + oz;
    int* const s_segstart = s_segstart0 + oz;
    const int w = w0 + oz, l = l0 + oz, r16 = l & 15, kg = l >> 4;
#pragma unroll
    for (int k = 0; k < T16 + 1; ++k) asm volatile("" : "+v"(cb[k]));   // (nor their unpacked values)
    __syncthreads();   // the previous head is done with the per-head LDS
    if (tid < Q) {
      s_acs[tid] = pf_acs;
      s_dt[tid] = pf_dt;
      const float acs_ref = __shfl(pf_acs, l | 15, WAVE);   // Acs at the end of the 16-row tile
      s_ejdt[tid] = Elem<T>::exp(acs_ref - pf_acs) * pf_dt;
    }
    st_x.store(s_x, LDX);
    if (e0_hin) st_e.store(s_e, LDE);
    if (tid < P) s_D[tid] = pb.D ? pb.D[pb.d_hp ? h * P + tid : h] : 0.f;   // D per channel (or repeated)
    __syncthreads();
    if (h + 1 < h_end) prefetch(h + 1);

    // ---- state term, exp(Acs_i) C_i . E_seg(i), segment by segment and
    // dstate slab by slab, into the y^T tiles of the wave's rows (ya: row w,
    // yb: row T-1-w)
    f32x4_t ya[PT], yb[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) ya[pt] = yb[pt] = zero4();
    for (int m = 0; m < nseg; ++m) {
      const int lo = s_segstart[m], hi = s_segstart[m + 1];
      const T* e_t;
      const float* e_f;
      e_src(h, m, e_t, e_f);
      if (!e_t && !e_f) continue;   // (uniform) no entering state
      for (int n0 = 0; n0 < pb.N; n0 += NS) {
        const bool stage_e = m > 0 || n0 > 0 || !e0_hin;   // (Hin's first slab came with the head)
        if (MULTI || stage_e) {
          RowStage<T, P, NS, NTHR> st_e2;
          if (MULTI) st_c.load(c_row(n0));
          if (stage_e) load_e(st_e2, e_t, e_f, n0);
          __syncthreads();   // the previous slab is read
          if (MULTI) st_c.store(s_c, LDC);
          if (stage_e) st_e2.store(s_e, LDE);
          __syncthreads();
        }
        // rows outside the segment take zero C operands (a row tile wholly
        // outside it adds nothing)
        const int iw = 16 * Cf::Split::row(w, 0) + r16, iv = 16 * Cf::Split::row(w, 1) + r16;
        const bool in_w = iw >= lo && iw < hi, in_v = iv >= lo && iv < hi;
#pragma unroll
        for (int k0 = 0; k0 < NS; k0 += KS) {
          typename Mma<T>::frag af[PT];
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) af[pt] = Mma<T>::load_k(s_e + (16 * pt + r16) * LDE + kg * KW + k0);
          auto bw = Mma<T>::load_k(s_c + iw * LDC + kg * KW + k0);
          auto bv = Mma<T>::load_k(s_c + iv * LDC + kg * KW + k0);
          if (!in_w) bw = Mma<T>::zero();
          if (!in_v) bv = Mma<T>::zero();
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) {
            ya[pt] = Mma<T>::mma(af[pt], bw, ya[pt]);
            yb[pt] = Mma<T>::mma(af[pt], bv, yb[pt]);
          }
        }
      }
    }
    {
      // a lane's accumulator values share one row i = 16 I + lane % 16
      const float e_w = Elem<T>::exp(s_acs[16 * Cf::Split::row(w, 0) + r16]);
      const float e_v = Elem<T>::exp(s_acs[16 * Cf::Split::row(w, 1) + r16]);
#pragma unroll
      for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ya[pt][r] *= e_w;
          yb[pt][r] *= e_v;
        }
    }

    // ---- intra-chunk term
    if (uniform)
      y_tiles<T, Q, P, NS, true>(cb, ya, yb, s_x, s_acs, s_dt, s_ejdt, s_seg, w, l);
    else
      y_tiles<T, Q, P, NS, false>(cb, ya, yb, s_x, s_acs, s_dt, s_ejdt, s_seg, w, l);

    // ---- epilogue: y = intra + state + D x, then the output gate if any:
    // forward, y silu(z); gate pass (dz given), the gated dy = dout silu(z)
    // into y's place and dz = dout y silu'(z).  y goes through the wave's own
    // x rows in LDS (every wave has finished reading x) so that the rows
    // leave, and dout / z arrive, as whole 16-byte pieces per lane.
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int i = 16 * Cf::Split::row(w, a) + r16;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const f32x4_t yv = a ? yb[pt] : ya[pt];
        T* px = s_x + i * LDX + 16 * pt + 4 * kg;
        const f32x4_t xv = load4f<T>(px);
        const f32x4_t D4 = *reinterpret_cast<const f32x4_t*>(s_D + 16 * pt + 4 * kg);
        f32x4_t o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = yv[r] + D4[r] * xv[r];
        store4f<T>(px, o);   // (each element is read and rewritten by the same lane)
      }
    }
    constexpr int VEC = Cf::VEC, CV = P / VEC, RV = 16 * CV / WAVE;   // 16-byte pieces per lane and row tile
    static_assert((16 * CV) % WAVE == 0, "whole pieces per lane");
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int I = Cf::Split::row(w, a);
#pragma unroll
      for (int q = 0; q < RV; ++q) {
        const int v = l + WAVE * q, i = 16 * I + v / CV, cv = v % CV, t = c * Q + i;
        if (t >= pb.L) continue;
        const uint4 yu = *reinterpret_cast<const uint4*>(s_x + i * LDX + cv * VEC);
        const int64_t off = ((static_cast<int64_t>(b) * pb.L + t) * pb.H + h) * P + cv * VEC;
        if (!pb.z) {   // (uniform)
          *reinterpret_cast<uint4*>(static_cast<T*>(pb.y) + off) = yu;
          continue;
        }
        const uint4 zu = ld_global16(static_cast<const T*>(pb.z) + off);
        if (!pb.dz) {
          T o[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float zz = vget<T>(zu, e), sg = gate_sigmoid<T>(zz);
            o[e] = Elem<T>::from_f(vget<T>(yu, e) * zz * sg);
          }
          *reinterpret_cast<uint4*>(static_cast<T*>(pb.y) + off) = *reinterpret_cast<const uint4*>(o);
          if (pb.ypre) *reinterpret_cast<uint4*>(static_cast<T*>(pb.ypre) + off) = yu;   // (uniform)
        } else {
          const uint4 du = ld_global16(static_cast<const T*>(pb.dout) + off);
          gate_grads<T>(du, zu, yu, static_cast<T*>(pb.y) + off, static_cast<T*>(pb.dz) + off);
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// k_gate_bwd: the backward's gate pass from the y the forward saved
// ----------------------------------------------------------------------------
// One thread per 16-byte piece of (B, L, H, P): the gated dy into dx's place
// and dz, from dout, z and the saved y (the same arithmetic as the output
// kernel's gate pass, so the same bits).
template <typename T>
__global__ __launch_bounds__(256) void k_gate_bwd(Problem pb, int64_t npiece) {
  constexpr int VEC = Vec16<T>::N;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= npiece) return;
  const int64_t off = i * VEC;
  const uint4 du = ld_global16(static_cast<const T*>(pb.dout) + off);
  const uint4 zu = ld_global16(static_cast<const T*>(pb.z) + off);
  const uint4 yu = ld_global16(static_cast<const T*>(pb.ypre) + off);
  gate_grads<T>(du, zu, yu, static_cast<T*>(pb.y) + off, static_cast<T*>(pb.dz) + off);
}

hipError_t launch_gate_bwd(const Problem& pb, bool io_bf16, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(pb.B) * pb.L * pb.H * pb.P;
  const int64_t npiece = n / (io_bf16 ? Vec16<bf16_t>::N : Vec16<float>::N);
  const dim3 grid(static_cast<unsigned>((npiece + 255) / 256));
  if (io_bf16)
    hipLaunchKernelGGL((k_gate_bwd<bf16_t>), grid, dim3(256), 0, s, pb, npiece);
  else
    hipLaunchKernelGGL((k_gate_bwd<float>), grid, dim3(256), 0, s, pb, npiece);
  return hipGetLastError();
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
template <typename T, int Q, int P, int NS, bool MULTI>
static hipError_t launch_y(const Problem& pb, hipStream_t s) {
  using Cf = YCfg<T, Q, P, NS>;
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&k_y<T, Q, P, NS, MULTI>), Cf::LDS);
  if (e != hipSuccess) return e;
  // heads per block: as many as keep about 1024 blocks (four per CU of an
  // MI355X) in the grid -- a function of the shape only -- or the test
  // override; every head's arithmetic is the same whatever the split
  const int64_t bgc = static_cast<int64_t>(pb.B) * pb.G * pb.nc;
  const int64_t want = 4 * static_cast<int64_t>(kHeadBlocks);
  int nsplit = static_cast<int>(std::min<int64_t>(pb.hpg, (want + bgc - 1) / bgc));
  int hper = (pb.hpg + nsplit - 1) / nsplit;
  const int ov = fwd_heads_per_block_override();
  if (ov > 0) hper = std::min(ov, pb.hpg);
  nsplit = (pb.hpg + hper - 1) / hper;
  hipLaunchKernelGGL((k_y<T, Q, P, NS, MULTI>), dim3(static_cast<unsigned>(bgc * nsplit)), dim3(Cf::NTHR), Cf::LDS, s, pb);
  return hipGetLastError();
}

template <typename T, int Q, int P>
static hipError_t launch_fwd_qp(const Problem& pb, hipStream_t s) {
  {
    const int64_t blocks = static_cast<int64_t>(pb.B) * pb.G * pb.nc;
    hipLaunchKernelGGL((k_cbf<T, Q>), dim3(static_cast<unsigned>(blocks)), dim3(CbfCfg<T, Q>::NTHR), 0, s, pb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    // all of N in one dstate slab up to 128 (bf16) / 64 (fp32) columns, else
    // slabs of 64 / 32 columns (or 32 / 16 when those do not divide N)
    constexpr int S = sizeof(T) == 2 ? 32 : 16;
    hipError_t e = pb.N == 4 * S   ? launch_y<T, Q, P, 4 * S, false>(pb, s)
                   : pb.N == 2 * S ? launch_y<T, Q, P, 2 * S, false>(pb, s)
                   : pb.N % (2 * S) == 0 ? launch_y<T, Q, P, 2 * S, true>(pb, s)
                                         : launch_y<T, Q, P, S, true>(pb, s);
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
  if (bf16 && Q == QQ && P == PP) return YCfg<bf16_t, QQ, PP, 128>::LDS;
#define SSD_Y_LDS_F(QQ, PP) \
  if (!bf16 && Q == QQ && P == PP) return YCfg<float, QQ, PP, 64>::LDS;
  SSD_BF16_SHAPES(SSD_Y_LDS_B)
  SSD_F32_SHAPES(SSD_Y_LDS_F)
#undef SSD_Y_LDS_B
#undef SSD_Y_LDS_F
  return ~size_t(0);
}

}  // namespace ssd
