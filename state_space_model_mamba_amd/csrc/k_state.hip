// Chunk-state forward recompute + state passing, and the state-passing
// backward (the inter-chunk half of the SSD backward whose intra-chunk
// kernels the page "Deterministic bwd kernel for mamba2" lists).
//
// Both kernels own one (batch, head, dstate tile) and walk the chunks in
// order, so every state element is produced by exactly one thread in a fixed
// order.  The chunk rows are double-buffered in LDS: while chunk c is
// multiplied from one buffer, the next chunk's rows (requested one chunk
// earlier) are staged into the other and the rows after it are requested.
//
// Forward, chunk c (positions j of the chunk's last segment, Acs restarted at
// that segment's start):
//   S_c        = sum_j exp(Acs_end - Acs_j) dt_j x_j (outer) B_j      (P x N, MFMA over j)
//   Hin_{c+1}  = exp(Acs_end) Hin_c + S_c                 if no sequence starts in chunk c
//              = S_c + exp(Acs_end) h0[s_last]            otherwise (h0 term only if given)
// Backward, chunk c from the last down (dOut = gradient w.r.t. the state at
// the end of chunk c through later positions; zero for the last chunk):
//   R_m        = sum_{i in segment m} exp(Acs_i) dy_i (outer) C_i  (MFMA over i)
//   d_h0[s_m]  = R_m (+ exp(Acs_end) dOut if m is the chunk's last segment)   segments that start s_m
//   dOut_{c-1} = R_0 + exp(Acs_end) dOut                if no sequence starts in chunk c
//              = R_0 (segment 0 continues) or 0          otherwise
#include "ssd_problem.h"
#include "ssd_tiles.h"

namespace ssd {

template <typename T, int Q, int P, int NT>
struct StateCfg {
  static constexpr int VEC = Vec16<T>::N;
  using XTile = KnTile<T, P>;                  // x / dy chunk rows [j][p]
  using BTile = KnTile<T, NT>;                 // B / C tile rows [j][n]
  static constexpr int NTHR = NT * 16;         // 8 waves for 32 state columns, 16 for 64
  static constexpr int NW = NTHR / WAVE;
  static constexpr int XV = Q * P / VEC;       // 16-byte vectors of one x/dy chunk
  static constexpr int NXV = (XV + NTHR - 1) / NTHR;
  static constexpr int BV = Q * NT / VEC;      // vectors of one B/C chunk tile
  static constexpr int NBV = (BV + NTHR - 1) / NTHR;
  static constexpr int PT = P / 16, NTT = NT / 16;
  // The chunk product is register-blocked: wave w < NBLK forms a BNB x BPB
  // block of 16 x 16 tiles (state columns x state rows), so each operand
  // fragment read from LDS serves two tiles and the LDS reads of a chunk are
  // half those of one tile per wave; the other waves only stage rows.
  static constexpr int BPB = PT % 2 == 0 ? 2 : 1, BNB = NTT % 2 == 0 ? 2 : 1;
  static constexpr int NBN = NTT / BNB, NBLK = (PT / BPB) * NBN;
  static_assert(NBLK <= NW, "a wave per block");
  static_assert(NTHR >= Q, "one thread per chunk position");
  static_assert(P % 16 == 0 && NT % 16 == 0 && Q % Mma<T>::KSTEP == 0, "tile shape");
};

// Forward walk.  The chunk rows are double-buffered in LDS: chunk c's
// product reads one buffer while chunk c+1's rows, which arrived in registers
// during chunk c-1, are staged into the other, and chunk c+2's rows and
// metadata are requested; one barrier per chunk.  Each thread scales the x
// rows it stages with w_j = exp(Acs_end - Acs_j) dt_j from its own loads.
// Every load is unconditional (row indices past L are clamped and the values
// zeroed when staged), so the requests never wait on a branch join.
template <typename T, int Q, int P, int NT>
struct StateFwdCfg {
  using Cf = StateCfg<T, Q, P, NT>;
  static constexpr int XSZ = Q * Cf::XTile::LD;   // elements of one x buffer
  static constexpr int BSZ = Q * Cf::BTile::LD;
  static constexpr size_t LDS_ROWS = 2 * static_cast<size_t>(XSZ + BSZ) * sizeof(T);
  // Hin leaves through LDS when it fits: each chunk's state tile [P][NT] is
  // written there (two buffers, taking turns) and stored during the next
  // chunk as whole rows, 16 bytes per lane
  static constexpr int LDH = NT + Cf::VEC;          // row pitch of a staged state tile
  static constexpr int HSZ = P * LDH;
  static constexpr bool HSTAGE = LDS_ROWS + 2 * static_cast<size_t>(HSZ) * sizeof(T) <= 160 * 1024;
  static constexpr size_t LDS = LDS_ROWS + (HSTAGE ? 2 * static_cast<size_t>(HSZ) * sizeof(T) : 0);
  static constexpr int HV = P * NT / Cf::VEC;       // 16-byte vectors of one state tile
};

// What a chunk's staging needs, as loaded (nothing derived, so nothing waits
// for it before the staging itself)
template <int NXV>
struct FwdRaw {
  float acs_end;
  int seg_last, nstart, seqbase;
  float acs[NXV], dt[NXV];   // of the rows this thread stages
};

template <typename T, int Q, int P, int NT>
__global__ __launch_bounds__((StateCfg<T, Q, P, NT>::NTHR)) void k_state_fwd(Problem pb) {
  using Cf = StateCfg<T, Q, P, NT>;
  using Fc = StateFwdCfg<T, Q, P, NT>;
  constexpr int VEC = Cf::VEC, NTHR = Cf::NTHR, NXV = Cf::NXV, NBV = Cf::NBV;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* const s_x0 = reinterpret_cast<T*>(smem);
  T* const s_b0 = s_x0 + 2 * Fc::XSZ;
  T* const s_h0 = s_b0 + 2 * Fc::BSZ;   // (HSTAGE) the two staged state tiles

  const int ntiles = pb.N / NT;
  const int64_t total = static_cast<int64_t>(pb.B) * pb.H * ntiles;
  const int64_t lb = xcd_logical_block(blockIdx.x, total);
  const int ntile = static_cast<int>(lb % ntiles);
  const int64_t bh = lb / ntiles;
  const int h = static_cast<int>(bh % pb.H), b = static_cast<int>(bh / pb.H);
  const int g = h / pb.hpg, n0 = ntile * NT;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r16 = l & 15, kg = l >> 4;
  const T* xs = static_cast<const T*>(pb.x);
  const T* bs = static_cast<const T*>(pb.Bm);
  // (HSTAGE) the staged state tile of chunk c (buffer c & 1) -> Hin_c, whole rows
  auto store_staged = [&](int c) {
    const T* sh = s_h0 + (c & 1) * Fc::HSZ;
    T* hc = static_cast<T*>(pb.hin) + ((static_cast<int64_t>(b) * pb.H + h) * pb.nc + c) * P * pb.N + n0;
    for (int v = tid; v < Fc::HV; v += NTHR) {
      const int p = v / (NT / VEC), q = (v % (NT / VEC)) * VEC;
      *reinterpret_cast<uint4*>(hc + p * pb.N + q) = *reinterpret_cast<const uint4*>(sh + p * Fc::LDH + q);
    }
  };

  // the thread's staged vectors: x vector k is row xrow(k), B vector k row
  // brow(k); on small shapes some threads have fewer vectors than others
  auto xrow = [&](int k) { return min((tid + NTHR * k) / (P / VEC), Q - 1); };
  auto brow = [&](int k) { return min((tid + NTHR * k) / (NT / VEC), Q - 1); };
  auto xhas = [&](int k) { return Cf::XV % NTHR == 0 || tid + NTHR * k < Cf::XV; };
  auto bhas = [&](int k) { return Cf::BV % NTHR == 0 || tid + NTHR * k < Cf::BV; };

  // Addresses: wave-uniform bases per chunk plus per-lane 32-bit offsets
  // fixed for the whole walk (recomputed only for a chunk that passes L).
  const int vz = vgpr_zero();
  const float* acs_bh = pb.acs + (static_cast<int64_t>(b) * pb.H + h) * pb.nc * Q;
  const float* dt_bh = pb.dtc + (static_cast<int64_t>(b) * pb.H + h) * pb.nc * Q;
  const int* seg_b = pb.segpos + static_cast<int64_t>(b) * pb.nc * Q;
  const int* ci_b = pb.cinfo + static_cast<int64_t>(b) * pb.nc * CINFO;
  const T* x_bh = xs + (static_cast<int64_t>(b) * pb.L * pb.H + h) * P;       // + t H P
  const T* b_bg = bs + (static_cast<int64_t>(b) * pb.L * pb.G + g) * pb.N + n0;  // + t G N
  const uint32_t xrb = static_cast<uint32_t>(pb.H * P * sizeof(T)), brb = static_cast<uint32_t>(pb.G * pb.N * sizeof(T));
  auto xoff = [&](int k, int j) { return static_cast<uint32_t>(j) * xrb + ((tid + NTHR * k) % (P / VEC)) * 16u; };
  auto boff = [&](int k, int j) { return static_cast<uint32_t>(j) * brb + ((tid + NTHR * k) % (NT / VEC)) * 16u; };
  uint32_t xo[NXV], bo[NBV];
#pragma unroll
  for (int k = 0; k < NXV; ++k) xo[k] = xoff(k, xrow(k));
#pragma unroll
  for (int k = 0; k < NBV; ++k) bo[k] = boff(k, brow(k));

  uint4 xr[NXV], br[NBV];
  FwdRaw<NXV> raw;
  auto request = [&](int c) {
    c = min(c, pb.nc - 1);   // (past the last chunk: a harmless reload)
    const float* ac = acs_bh + c * Q;
    const float* dc = dt_bh + c * Q;
    raw.acs_end = ac[Q - 1 + vz];
    raw.seg_last = seg_b[c * Q + Q - 1 + vz];
    raw.nstart = ci_b[c * CINFO + 0 + vz];
    raw.seqbase = ci_b[c * CINFO + 3 + vz];
    const int lastrow = pb.L - 1 - c * Q;   // rows past it are clamped (uniform)
    const T* xc = x_bh + static_cast<int64_t>(c) * Q * pb.H * P;
    const T* bc = b_bg + static_cast<int64_t>(c) * Q * pb.G * pb.N;
#pragma unroll
    for (int k = 0; k < NXV; ++k) {
      raw.acs[k] = ac[xrow(k)];
      raw.dt[k] = dc[xrow(k)];
      uint32_t o = xo[k];
      if (lastrow < Q - 1) o = xoff(k, min(xrow(k), lastrow));
      if (xhas(k)) xr[k] = ld_global16_at(xc, o);
    }
#pragma unroll
    for (int k = 0; k < NBV; ++k) {
      uint32_t o = bo[k];
      if (lastrow < Q - 1) o = boff(k, min(brow(k), lastrow));
      if (bhas(k)) br[k] = ld_global16_at(bc, o);
    }
  };
  // per-chunk values the state update needs
  struct Upd {
    float decay;
    int nstart, s_last;
  };
  // stage chunk c's rows (arrived in xr / br) into buffer c & 1; returns its update values
  auto stage = [&](int c) {
    T* sx = s_x0 + (c & 1) * Fc::XSZ;
    T* sb = s_b0 + (c & 1) * Fc::BSZ;
    const int lolast = seg_lo(raw.seg_last);
#pragma unroll
    for (int k = 0; k < NXV; ++k) {
      const int j = xrow(k), pv = (tid + NTHR * k) % (P / VEC);
      const bool ok = j >= lolast && c * Q + j < pb.L;
      const float sc = ok ? Elem<T>::exp(raw.acs_end - raw.acs[k]) * raw.dt[k] : 0.f;
      uint4 o;
      if constexpr (sizeof(T) == 2) {
        uint32_t u[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(vget<T>(xr[k], 2 * e) * sc, vget<T>(xr[k], 2 * e + 1) * sc);
        o = uint4{u[0], u[1], u[2], u[3]};
      } else {
        f32x4_t f;
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = vget<T>(xr[k], e) * sc;
        o = __builtin_bit_cast(uint4, f);
      }
      if (xhas(k)) *reinterpret_cast<uint4*>(sx + Cf::XTile::at(j, pv * VEC)) = o;
    }
#pragma unroll
    for (int k = 0; k < NBV; ++k) {
      const int j = brow(k), nv = (tid + NTHR * k) % (NT / VEC);
      if (bhas(k)) *reinterpret_cast<uint4*>(sb + Cf::BTile::at(j, nv * VEC)) = c * Q + j < pb.L ? br[k] : zero_u4();
    }
    Upd u;
    u.decay = Elem<T>::exp(raw.acs_end);
    u.nstart = raw.nstart;
    u.s_last = clamp_seq(raw.seqbase + raw.nstart - 1, pb.nseqs);
    return u;
  };

  constexpr int BPB = Cf::BPB, BNB = Cf::BNB, NBN = Cf::NBN, NBLK = Cf::NBLK;
  f32x4_t st[BNB][BPB];   // (waves w < NBLK) the state of this wave's tiles
#pragma unroll
  for (int i = 0; i < BNB; ++i)
#pragma unroll
    for (int j = 0; j < BPB; ++j) st[i][j] = zero4();
  const int bp = w / NBN, bn = w % NBN;
  request(0);
  Upd cur = stage(0);
  request(1);
  __syncthreads();
  for (int c = 0; c < pb.nc; ++c) {
    const int64_t bhc = (static_cast<int64_t>(b) * pb.H + h) * pb.nc + c;
    Upd nxt = cur;
    if (c + 1 < pb.nc) nxt = stage(c + 1);   // (uniform)
    request(c + 2);
    if constexpr (Fc::HSTAGE) {
      if (c > 0) store_staged(c - 1);   // (staged before the last barrier)
    }
    const T* sx = s_x0 + (c & 1) * Fc::XSZ;
    const T* sb = s_b0 + (c & 1) * Fc::BSZ;
    if (w < NBLK) {   // (wave-uniform)
      // S^T (the B tiles as the A operand): for tile (i, j) this lane holds
      // state row p = 16 pt + lane % 16 and the four columns n .. n + 3,
      // n = n0 + 16 nt + 4 (lane / 16), with pt = BPB bp + j, nt = BNB bn + i
      f32x4_t S[BNB][BPB];
#pragma unroll
      for (int i = 0; i < BNB; ++i)
#pragma unroll
        for (int j = 0; j < BPB; ++j) S[i][j] = zero4();
#pragma unroll
      for (int k0 = 0; k0 < Q; k0 += Mma<T>::KSTEP) {
        typename Mma<T>::frag af[BNB], bfr[BPB];
#pragma unroll
        for (int i = 0; i < BNB; ++i) af[i] = Cf::BTile::frag(sb, (BNB * bn + i) * 16, k0);
#pragma unroll
        for (int j = 0; j < BPB; ++j) bfr[j] = Cf::XTile::frag(sx, (BPB * bp + j) * 16, k0);
#pragma unroll
        for (int i = 0; i < BNB; ++i)
#pragma unroll
          for (int j = 0; j < BPB; ++j) S[i][j] = Mma<T>::mma(af[i], bfr[j], S[i][j]);
      }
#pragma unroll
      for (int i = 0; i < BNB; ++i)
#pragma unroll
        for (int j = 0; j < BPB; ++j) {
          const int pt = BPB * bp + j, nt = BNB * bn + i;
          const int p = pt * 16 + r16, n = n0 + nt * 16 + 4 * kg;
          if constexpr (Fc::HSTAGE)
            store4f<T>(s_h0 + (c & 1) * Fc::HSZ + p * Fc::LDH + nt * 16 + 4 * kg, st[i][j]);
          else
            store4f<T>(static_cast<T*>(pb.hin) + (bhc * P + p) * pb.N + n, st[i][j]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (cur.nstart == 0) {
              st[i][j][r] = cur.decay * st[i][j][r] + S[i][j][r];
            } else {
              float init = 0.f;
              if (pb.h0) init = cur.decay * pb.h0[((static_cast<int64_t>(cur.s_last) * pb.H + h) * P + p) * pb.N + n + r];
              st[i][j][r] = S[i][j][r] + init;
            }
          }
        }
    }
    __syncthreads();
    cur = nxt;
  }
  if constexpr (Fc::HSTAGE) store_staged(pb.nc - 1);
}

// Backward walk, chunks from the last down, with the forward walk's
// pipeline: chunk rows double-buffered in LDS with their segment tables, each
// thread scaling the dy rows it stages by exp(Acs_i) from its own loads,
// unconditional requests, one barrier per chunk.
template <typename T, int Q, int P, int NT>
struct StateBwdCfg {
  using Cf = StateCfg<T, Q, P, NT>;
  static constexpr int XSZ = Q * Cf::XTile::LD;
  static constexpr int BSZ = Q * Cf::BTile::LD;
  static constexpr int TSZ = 2 * Q + 1;   // segpos[Q], segment starts[Q + 1]
  static constexpr size_t LDS_ROWS = 2 * static_cast<size_t>(XSZ + BSZ) * sizeof(T) + 2 * TSZ * sizeof(int);
  // dS leaves through LDS as whole rows when it fits (as Hin in the forward walk)
  static constexpr int LDH = NT + Cf::VEC;
  static constexpr int HSZ = P * LDH;
  static constexpr size_t OFF_H = (LDS_ROWS + 15) / 16 * 16;   // the staged tiles (16-byte aligned)
  static constexpr bool HSTAGE = OFF_H + 2 * static_cast<size_t>(HSZ) * sizeof(T) <= 160 * 1024;
  static constexpr size_t LDS = HSTAGE ? OFF_H + 2 * static_cast<size_t>(HSZ) * sizeof(T) : LDS_ROWS;
  static constexpr int HV = P * NT / Cf::VEC;
};

template <int NXV>
struct BwdRaw {
  float acs_end;
  int nstart, seqbase, seg0, seg_own;
  float acs[NXV];   // of the rows this thread stages
};

template <typename T, int Q, int P, int NT>
__global__ __launch_bounds__((StateCfg<T, Q, P, NT>::NTHR)) void k_state_bwd(Problem pb) {
  using Cf = StateCfg<T, Q, P, NT>;
  using Bc = StateBwdCfg<T, Q, P, NT>;
  constexpr int VEC = Cf::VEC, NTHR = Cf::NTHR, NXV = Cf::NXV, NBV = Cf::NBV;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* const s_x0 = reinterpret_cast<T*>(smem);
  T* const s_b0 = s_x0 + 2 * Bc::XSZ;
  int* const s_t0 = reinterpret_cast<int*>(s_b0 + 2 * Bc::BSZ);

  const int ntiles = pb.N / NT;
  const int64_t total = static_cast<int64_t>(pb.B) * pb.H * ntiles;
  const int64_t lb = xcd_logical_block(blockIdx.x, total);
  const int ntile = static_cast<int>(lb % ntiles);
  const int64_t bh = lb / ntiles;
  const int h = static_cast<int>(bh % pb.H), b = static_cast<int>(bh / pb.H);
  const int g = h / pb.hpg, n0 = ntile * NT;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), r16 = l & 15, kg = l >> 4;
  const T* ys = static_cast<const T*>(pb.dy);
  const T* cs = static_cast<const T*>(pb.Cm);

  auto xrow = [&](int k) { return min((tid + NTHR * k) / (P / VEC), Q - 1); };
  auto brow = [&](int k) { return min((tid + NTHR * k) / (NT / VEC), Q - 1); };
  auto xhas = [&](int k) { return Cf::XV % NTHR == 0 || tid + NTHR * k < Cf::XV; };
  auto bhas = [&](int k) { return Cf::BV % NTHR == 0 || tid + NTHR * k < Cf::BV; };

  // Addresses as in the forward walk: wave-uniform bases plus per-lane
  // 32-bit offsets fixed for the whole walk.
  const int vz = vgpr_zero();
  const float* acs_bh = pb.acs + (static_cast<int64_t>(b) * pb.H + h) * pb.nc * Q;
  const int* seg_b = pb.segpos + static_cast<int64_t>(b) * pb.nc * Q;
  const int* ci_b = pb.cinfo + static_cast<int64_t>(b) * pb.nc * CINFO;
  const T* y_bh = ys + (static_cast<int64_t>(b) * pb.L * pb.H + h) * P;       // + t H P
  const T* c_bg = cs + (static_cast<int64_t>(b) * pb.L * pb.G + g) * pb.N + n0;  // + t G N
  const uint32_t xrb = static_cast<uint32_t>(pb.H * P * sizeof(T)), brb = static_cast<uint32_t>(pb.G * pb.N * sizeof(T));
  auto xoff = [&](int k, int j) { return static_cast<uint32_t>(j) * xrb + ((tid + NTHR * k) % (P / VEC)) * 16u; };
  auto boff = [&](int k, int j) { return static_cast<uint32_t>(j) * brb + ((tid + NTHR * k) % (NT / VEC)) * 16u; };
  uint32_t xo[NXV], bo[NBV];
#pragma unroll
  for (int k = 0; k < NXV; ++k) xo[k] = xoff(k, xrow(k));
#pragma unroll
  for (int k = 0; k < NBV; ++k) bo[k] = boff(k, brow(k));
  const int own = min(tid, Q - 1);

  uint4 xr[NXV], br[NBV];
  BwdRaw<NXV> raw;
  auto request = [&](int c) {
    c = max(c, 0);   // (before the first chunk: a harmless reload)
    const float* ac = acs_bh + c * Q;
    const int* sg = seg_b + c * Q;
    raw.acs_end = ac[Q - 1 + vz];
    raw.nstart = ci_b[c * CINFO + 0 + vz];
    raw.seqbase = ci_b[c * CINFO + 3 + vz];
    raw.seg0 = sg[vz];
    raw.seg_own = sg[own];
    const int lastrow = pb.L - 1 - c * Q;   // rows past it are clamped (uniform)
    const T* yc = y_bh + static_cast<int64_t>(c) * Q * pb.H * P;
    const T* cc = c_bg + static_cast<int64_t>(c) * Q * pb.G * pb.N;
#pragma unroll
    for (int k = 0; k < NXV; ++k) {
      raw.acs[k] = ac[xrow(k)];
      uint32_t o = xo[k];
      if (lastrow < Q - 1) o = xoff(k, min(xrow(k), lastrow));
      if (xhas(k)) xr[k] = ld_global16_at(yc, o);
    }
#pragma unroll
    for (int k = 0; k < NBV; ++k) {
      uint32_t o = bo[k];
      if (lastrow < Q - 1) o = boff(k, min(brow(k), lastrow));
      if (bhas(k)) br[k] = ld_global16_at(cc, o);
    }
  };
  struct Upd {
    float decay;
    int nstart, nseg, seqbase;
  };
  // stage chunk c (buffer par) from xr / br / raw
  auto stage = [&](int c, int par) {
    T* sx = s_x0 + par * Bc::XSZ;
    T* sb = s_b0 + par * Bc::BSZ;
    int* s_seg = s_t0 + par * Bc::TSZ;
    int* s_segstart = s_seg + Q;
#pragma unroll
    for (int k = 0; k < NXV; ++k) {
      const int j = xrow(k), pv = (tid + NTHR * k) % (P / VEC);
      const float sc = c * Q + j < pb.L ? Elem<T>::exp(raw.acs[k]) : 0.f;
      uint4 o;
      if constexpr (sizeof(T) == 2) {
        uint32_t u[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(vget<T>(xr[k], 2 * e) * sc, vget<T>(xr[k], 2 * e + 1) * sc);
        o = uint4{u[0], u[1], u[2], u[3]};
      } else {
        f32x4_t f;
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = vget<T>(xr[k], e) * sc;
        o = __builtin_bit_cast(uint4, f);
      }
      if (xhas(k)) *reinterpret_cast<uint4*>(sx + Cf::XTile::at(j, pv * VEC)) = o;
    }
#pragma unroll
    for (int k = 0; k < NBV; ++k) {
      const int j = brow(k), nv = (tid + NTHR * k) % (NT / VEC);
      if (bhas(k)) *reinterpret_cast<uint4*>(sb + Cf::BTile::at(j, nv * VEC)) = c * Q + j < pb.L ? br[k] : zero_u4();
    }
    const int start0 = seg_rank(raw.seg0);   // 1 when a sequence starts at position 0
    Upd u;
    u.decay = Elem<T>::exp(raw.acs_end);
    u.nstart = raw.nstart;
    u.nseg = raw.nstart + 1 - start0;
    u.seqbase = raw.seqbase;
    if (tid < Q) {
      s_seg[tid] = raw.seg_own;
      if (tid > 0 && seg_lo(raw.seg_own) == tid) s_segstart[seg_rank(raw.seg_own) - start0] = tid;
    }
    if (tid == 0) {
      s_segstart[0] = 0;
      s_segstart[u.nseg] = Q;
    }
    return u;
  };

  // the gradient at the end of the last chunk: zero, or the one handed in for the
  // state after the row's last position (padded positions leave the state unchanged)
  // (as in the forward walk, for tile (i, j) of its block this lane holds
  // state row p = 16 pt + lane % 16 and columns n0 + 16 nt + 4 (lane / 16) + r,
  // pt = BPB bp + j, nt = BNB bn + i)
  constexpr int BPB = Cf::BPB, BNB = Cf::BNB, NBN = Cf::NBN, NBLK = Cf::NBLK;
  const int bp = w / NBN, bn = w % NBN;
  f32x4_t dout[BNB][BPB];
#pragma unroll
  for (int i = 0; i < BNB; ++i)
#pragma unroll
    for (int j = 0; j < BPB; ++j) {
      dout[i][j] = zero4();
      const int pt = BPB * bp + j, nt = BNB * bn + i;
      if (pb.dlast && w < NBLK) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dout[i][j][r] = pb.dlast[((static_cast<int64_t>(b) * pb.H + h) * P + pt * 16 + r16) * pb.N + n0 +
                                   nt * 16 + 4 * kg + r];
      }
    }
  T* const dst_bh = static_cast<T*>(pb.dstate) + (static_cast<int64_t>(b) * pb.H + h) * pb.nc * P * pb.N;
  // (HSTAGE) the two staged state-gradient tiles, after the segment tables
  T* const s_h0 = reinterpret_cast<T*>(smem + Bc::OFF_H);
  auto store_staged = [&](int c, int buf) {
    const T* sh = s_h0 + buf * Bc::HSZ;
    T* dc = dst_bh + static_cast<int64_t>(c) * P * pb.N + n0;
    for (int v = tid; v < Bc::HV; v += NTHR) {
      const int p = v / (NT / VEC), q = (v % (NT / VEC)) * VEC;
      *reinterpret_cast<uint4*>(dc + p * pb.N + q) = *reinterpret_cast<const uint4*>(sh + p * Bc::LDH + q);
    }
  };
  request(pb.nc - 1);
  Upd cur = stage(pb.nc - 1, 0);
  request(pb.nc - 2);
  __syncthreads();
  for (int c = pb.nc - 1, it = 0; c >= 0; --c, ++it) {
    const int par = it & 1;
    Upd nxt = cur;
    if (c > 0) nxt = stage(c - 1, par ^ 1);   // (uniform)
    request(c - 2);
    if constexpr (Bc::HSTAGE) {
      if (c < pb.nc - 1) store_staged(c + 1, par ^ 1);   // (staged before the last barrier)
    }
    T* const dc = dst_bh + static_cast<int64_t>(c) * P * pb.N;   // this chunk's [P][N] state gradient
    const T* s_dyt = s_x0 + par * Bc::XSZ;
    const T* s_ct = s_b0 + par * Bc::BSZ;
    const int* s_seg = s_t0 + par * Bc::TSZ;
    const int* s_segstart = s_seg + Q;
    if (w < NBLK) {   // (wave-uniform)
#pragma unroll
      for (int i = 0; i < BNB; ++i)
#pragma unroll
        for (int j = 0; j < BPB; ++j) {
          const int pt = BPB * bp + j, nt = BNB * bn + i;
          const int p = pt * 16 + r16, n = n0 + nt * 16 + 4 * kg;
          if constexpr (Bc::HSTAGE)
            store4f<T>(s_h0 + par * Bc::HSZ + p * Bc::LDH + nt * 16 + 4 * kg, dout[i][j]);
          else
            store4f<T>(dc + p * pb.N + n, dout[i][j]);
        }
      if (cur.nstart == 0) {
        f32x4_t R[BNB][BPB];
#pragma unroll
        for (int i = 0; i < BNB; ++i)
#pragma unroll
          for (int j = 0; j < BPB; ++j) R[i][j] = zero4();
#pragma unroll
        for (int k0 = 0; k0 < Q; k0 += Mma<T>::KSTEP) {
          typename Mma<T>::frag af[BNB], bfr[BPB];
#pragma unroll
          for (int i = 0; i < BNB; ++i) af[i] = Cf::BTile::frag(s_ct, (BNB * bn + i) * 16, k0);
#pragma unroll
          for (int j = 0; j < BPB; ++j) bfr[j] = Cf::XTile::frag(s_dyt, (BPB * bp + j) * 16, k0);
#pragma unroll
          for (int i = 0; i < BNB; ++i)
#pragma unroll
            for (int j = 0; j < BPB; ++j) R[i][j] = Mma<T>::mma(af[i], bfr[j], R[i][j]);
        }
#pragma unroll
        for (int i = 0; i < BNB; ++i)
#pragma unroll
          for (int j = 0; j < BPB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) dout[i][j][r] = R[i][j][r] + cur.decay * dout[i][j][r];
      } else {
        // A chunk with a sequence start: per segment the same blocked product
        // over the segment's positions (the rows outside it masked), each
        // tile's products in ascending position order.  The segments go last
        // first: the last one's d_init term takes the incoming dOut, and the
        // segment that continues the previous chunk's sequence (segment 0, if
        // any) becomes the outgoing dOut after all of them.
        bool cont = false;
        for (int m = cur.nseg - 1; m >= 0; --m) {
          const int lo = __builtin_amdgcn_readfirstlane(s_segstart[m]);
          const int hi = __builtin_amdgcn_readfirstlane(s_segstart[m + 1]);
          f32x4_t R[BNB][BPB];
#pragma unroll
          for (int i = 0; i < BNB; ++i)
#pragma unroll
            for (int j = 0; j < BPB; ++j) R[i][j] = zero4();
#pragma unroll 1
          for (int k0 = (lo / Mma<T>::KSTEP) * Mma<T>::KSTEP; k0 < hi; k0 += Mma<T>::KSTEP) {
            typename Mma<T>::frag af[BNB], bfr[BPB];
#pragma unroll
            for (int i = 0; i < BNB; ++i) af[i] = Cf::BTile::frag(s_ct, (BNB * bn + i) * 16, k0);
#pragma unroll
            for (int j = 0; j < BPB; ++j) bfr[j] = mask_k<T>(Cf::XTile::frag(s_dyt, (BPB * bp + j) * 16, k0), k0, lo, hi);
#pragma unroll
            for (int i = 0; i < BNB; ++i)
#pragma unroll
              for (int j = 0; j < BPB; ++j) R[i][j] = Mma<T>::mma(af[i], bfr[j], R[i][j]);
          }
          const int rank = __builtin_amdgcn_readfirstlane(seg_rank(s_seg[lo]));
          if (rank == 0) {
#pragma unroll
            for (int i = 0; i < BNB; ++i)
#pragma unroll
              for (int j = 0; j < BPB; ++j) dout[i][j] = R[i][j];
            cont = true;
          } else if (pb.dinit) {
            const int s = clamp_seq(cur.seqbase + rank - 1, pb.nseqs);
#pragma unroll
            for (int i = 0; i < BNB; ++i)
#pragma unroll
              for (int j = 0; j < BPB; ++j) {
                const int pt = BPB * bp + j, nt = BNB * bn + i;
                const int p = pt * 16 + r16, n = n0 + nt * 16 + 4 * kg;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  float v = R[i][j][r];
                  if (hi == Q) v += cur.decay * dout[i][j][r];
                  pb.dinit[((static_cast<int64_t>(s) * pb.H + h) * P + p) * pb.N + n + r] = v;
                }
              }
          }
        }
        if (!cont) {
#pragma unroll
          for (int i = 0; i < BNB; ++i)
#pragma unroll
            for (int j = 0; j < BPB; ++j) dout[i][j] = zero4();
        }
      }
    }
    __syncthreads();
    cur = nxt;
  }
  if constexpr (Bc::HSTAGE) store_staged(0, (pb.nc - 1) & 1);
}

// N-tile width of the state kernels.
static int state_nt(int N, bool bf16) {
  (void)bf16;
  return (N % 64 == 0) ? 64 : (N % 32 == 0) ? 32 : 16;
}

template <typename T, int Q, int P, int NT>
static hipError_t launch_state_t(const Problem& pb, bool fwd, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(pb.B) * pb.H * (pb.N / NT);
  if (fwd) {
    constexpr size_t lds = StateFwdCfg<T, Q, P, NT>::LDS;
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&k_state_fwd<T, Q, P, NT>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_state_fwd<T, Q, P, NT>), dim3(static_cast<unsigned>(blocks)), dim3(StateCfg<T, Q, P, NT>::NTHR), lds, s, pb);
  } else {
    constexpr size_t lds = StateBwdCfg<T, Q, P, NT>::LDS;
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&k_state_bwd<T, Q, P, NT>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_state_bwd<T, Q, P, NT>), dim3(static_cast<unsigned>(blocks)), dim3(StateCfg<T, Q, P, NT>::NTHR), lds, s, pb);
  }
  return hipGetLastError();
}

template <typename T, int Q, int P>
static hipError_t launch_state_qp(const Problem& pb, bool fwd, hipStream_t s) {
  const int nt = state_nt(pb.N, sizeof(T) == 2);
  if (nt == 64) return launch_state_t<T, Q, P, 64>(pb, fwd, s);
  if (nt == 32) return launch_state_t<T, Q, P, 32>(pb, fwd, s);
  if constexpr (Q <= 128) return launch_state_t<T, Q, P, 16>(pb, fwd, s);
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_state_any(const Problem& pb, bool fwd, hipStream_t s) {
#define SSD_STATE_CASE(QQ, PP) \
  if (pb.Q == QQ && pb.P == PP) return launch_state_qp<T, QQ, PP>(pb, fwd, s);
  if constexpr (sizeof(T) == 2) {
    SSD_BF16_SHAPES(SSD_STATE_CASE)
  } else {
    SSD_F32_SHAPES(SSD_STATE_CASE)
  }
#undef SSD_STATE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_state_fwd(const Problem& pb, bool io_bf16, hipStream_t s) {
  return io_bf16 ? launch_state_any<bf16_t>(pb, true, s) : launch_state_any<float>(pb, true, s);
}

hipError_t launch_state_bwd(const Problem& pb, bool io_bf16, hipStream_t s) {
  return io_bf16 ? launch_state_any<bf16_t>(pb, false, s) : launch_state_any<float>(pb, false, s);
}

}  // namespace ssd
