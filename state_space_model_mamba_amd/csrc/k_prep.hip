// Chunk preparation, sequence numbering and the final fixed-order reduction.
//
// k_prep (the forward half of chunk_cumsum named on the page "Deterministic
// bwd kernel for mamba2"): per (batch, chunk) it finds the sequence starts,
// records each position's segment, and for every head writes
//   Acs_i = sum of dt_k * A_h over k from the start of i's segment to i,
// restarted at the chunk start and at every sequence start.  Every kernel
// downstream takes exp(Acs_i - Acs_j) from these values, and gradients such
// as dA add many such terms with heavy cancellation, so Acs is scanned in
// double and rounded to float once.  The scan order is fixed by the chunk
// size alone: the chunk is scanned as Q/64 runs of 64 positions, each with a
// 64-lane segmented scan in DPP steps (row shifts by 1, 2, 4 and 8 lanes, then
// the row-broadcast steps across rows) that starts from the previous run's
// last value.
// A block handles PREP_HEADS (4) heads of one (batch, chunk), one per wave.  That page
// reports that a cumsum whose result changes with the block shape broke
// run-to-run reproducibility; here the result does not depend on how many
// heads a block handles or on the launch shape.
#include "ssd_device.h"
#include "ssd_problem.h"

namespace ssd {

constexpr int PREP_HEADS = 4;    // heads per block of k_prep

// The double that the DPP control CTRL reads from another lane (rows ROWS;
// +0.0 where it reads none), both halves moved the same way.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u)), CTRL, ROWS, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u >> 32)), CTRL, ROWS, 0xF, false));
  return __builtin_bit_cast(double, static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
}

// One step of the segmented inclusive scan over the wave's lanes (a lane
// whose flag is set starts a segment)
template <int CTRL, int ROWS>
__device__ __forceinline__ void seg_step_f64(double& v, int& f) {
  const double tv = dpp_f64<CTRL, ROWS>(v);
  const int tf = __builtin_amdgcn_update_dpp(0, f, CTRL, ROWS, 0xF, false);
  v = f ? v : tv + v;
  f |= tf;
}

template <int Q>
__global__ __launch_bounds__(256) void k_prep(Problem pb) {
  static_assert(Q % WAVE == 0 && Q <= 256, "chunk size");
  constexpr int R = Q / WAVE;
  constexpr int LDD = PREP_HEADS + 1;   // dt rows in LDS, padded
  const int c = blockIdx.x, b = blockIdx.y, h0 = blockIdx.z * PREP_HEADS;
  const int tid = threadIdx.x;
  __shared__ int s_flag[Q], s_lo[Q], s_rank[Q];
  __shared__ float s_dt[Q * LDD];
  __shared__ float s_dfe[Q * LDD];   // (with a dt front-end) its derivative

  // this block's heads of the chunk's dt rows, coalesced (zeros past L and past H)
  // (through the dt front-end when one is given; zeros stay zeros)
  for (int v = tid; v < Q * PREP_HEADS; v += 256) {
    const int i = v / PREP_HEADS, hh = v % PREP_HEADS, t = c * Q + i;
    float d = 0.f, dfdu = 0.f;
    if (t < pb.L && h0 + hh < pb.H) {
      d = pb.dt[(static_cast<int64_t>(b) * pb.L + t) * pb.H + h0 + hh];
      if (pb.fe) d = dt_frontend(pb, d, h0 + hh, &dfdu);
    }
    s_dt[i * LDD + hh] = d;
    if (pb.fe) s_dfe[i * LDD + hh] = dfdu;
  }
  if (tid < Q) {
    const int t = c * Q + tid;
    int st = 0;
    if (t < pb.L) {
      st = (t == 0);
      if (!st && pb.seq_idx) {
        const int64_t base = static_cast<int64_t>(b) * pb.L + t;
        st = pb.seq_idx[base] != pb.seq_idx[base - 1];
      }
    }
    s_flag[tid] = st;
    s_lo[tid] = st ? tid : 0;
    s_rank[tid] = st;
  }
  __syncthreads();
  const int64_t bc = static_cast<int64_t>(b) * pb.nc + c;
  if (blockIdx.z == 0) {   // (uniform) the chunk's segment table, written by its first block of heads
    // integer inclusive scans (max for the segment start, sum for the rank)
    for (int off = 1; off < Q; off <<= 1) {
      int lo = 0, rk = 0;
      const bool act = tid < Q && tid >= off;
      if (act) {
        lo = s_lo[tid - off];
        rk = s_rank[tid - off];
      }
      __syncthreads();
      if (act) {
        s_lo[tid] = max(s_lo[tid], lo);
        s_rank[tid] += rk;
      }
      __syncthreads();
    }
    if (tid < Q) pb.segpos[bc * Q + tid] = s_lo[tid] | (s_rank[tid] << 16);
    if (tid == 0) {
      pb.cinfo[bc * CINFO + 0] = s_rank[Q - 1];
      pb.cinfo[bc * CINFO + 1] = 0;
      pb.cinfo[bc * CINFO + 2] = 0;
    }
  }

  // Segmented inclusive cumsum of a = dt A over the chunk, per head, in one
  // order fixed by Q alone: the chunk is cut into R runs of 64 positions
  // (lane l holds position 64 e + l); each run is scanned across the wave
  // with a segmented scan in DPP steps (a doubling scan within each row of
  // 16 lanes, then row 0's total into row 1 and row 2's into row 3, then the
  // first half's total into rows 2 and 3), and each run starts from the
  // carry of the previous one.
  const int w = wave_id(), l = lane_id();
  for (int hh = w; hh < PREP_HEADS && h0 + hh < pb.H; hh += 4) {
    const int h = h0 + hh;
    const double Ah = pb.A[h];
    const int64_t out = ((static_cast<int64_t>(b) * pb.H + h) * pb.nc + c) * Q;
    double carry = 0.0;
#pragma unroll
    for (int e = 0; e < R; ++e) {
      const int i = 64 * e + l;
      const float d = s_dt[i * LDD + hh];
      int fl = (i == 0) || s_flag[i];
      double v = static_cast<double>(d) * Ah;
      seg_step_f64<0x111, 0xF>(v, fl);   // row_shr:1
      seg_step_f64<0x112, 0xF>(v, fl);   // row_shr:2
      seg_step_f64<0x114, 0xF>(v, fl);   // row_shr:4
      seg_step_f64<0x118, 0xF>(v, fl);   // row_shr:8
      seg_step_f64<0x142, 0xA>(v, fl);   // row_bcast:15 into rows 1 and 3
      seg_step_f64<0x143, 0xC>(v, fl);   // row_bcast:31 into rows 2 and 3
      // positions not preceded by a start within this run continue the carry
      const double acs = fl ? v : carry + v;
      pb.acs[out + i] = static_cast<float>(acs);
      pb.dtc[out + i] = d;
      if (pb.fe) pb.dfe[out + i] = s_dfe[i * LDD + hh];
      const uint64_t cu = __builtin_bit_cast(uint64_t, acs);   // lane 63's value, to every lane
      carry = __builtin_bit_cast(double, static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(cu)), WAVE - 1))) |
                                             (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(cu >> 32)), WAVE - 1))) << 32));
    }
  }
}

// Global numbering of sequence starts: exclusive prefix sum of the per-chunk
// start counts in row-major (batch, chunk) order.  One wave; integer only:
// 64 counts at a time, each batch a DPP inclusive scan over the lanes (a
// doubling scan within each row of 16, then row 0's total into row 1 and row
// 2's into row 3, then the first half's into rows 2 and 3) plus the running
// total of the batches before.
template <int CTRL, int ROWS>
__device__ __forceinline__ int scan_step_i32(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}

__global__ __launch_bounds__(64) void k_seqbase(Problem pb) {
  const int l = threadIdx.x;
  const int total = pb.B * pb.nc;
  int run = 0;
  for (int base = 0; base < total; base += WAVE) {
    const int idx = base + l;
    const int v = idx < total ? pb.cinfo[static_cast<int64_t>(idx) * CINFO] : 0;
    int incl = v;
    incl = scan_step_i32<0x111, 0xF>(incl);   // row_shr:1
    incl = scan_step_i32<0x112, 0xF>(incl);   // row_shr:2
    incl = scan_step_i32<0x114, 0xF>(incl);   // row_shr:4
    incl = scan_step_i32<0x118, 0xF>(incl);   // row_shr:8
    incl = scan_step_i32<0x142, 0xA>(incl);   // row_bcast:15 into rows 1 and 3
    incl = scan_step_i32<0x143, 0xC>(incl);   // row_bcast:31 into rows 2 and 3
    if (idx < total) pb.cinfo[static_cast<int64_t>(idx) * CINFO + 3] = run + incl - v;
    run += __builtin_amdgcn_readlane(incl, WAVE - 1);
  }
}

// dA_h = sum over (b, c) of slot_dA[b, c, h], dD likewise.  The slots of a
// head can cancel heavily, so they are added in double and rounded once:
// lane l sums the slots l, l + 64, ... in ascending order, then the 64 lane
// sums meet in a fixed xor butterfly (offsets 32, 16, ..., 1).  The double
// sum's own error is at most about n 2^-53 times the slots' absolute sum,
// far below the rounding already in each float slot.  One wave per head.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, WAVE);
  return v;
}

__global__ __launch_bounds__(256) void k_reduce(Problem pb) {
  const int h = blockIdx.x * 4 + wave_id();
  if (h >= pb.H) return;
  const int l = lane_id();
  const int n = pb.B * pb.nc;
  double a = 0.0, d = 0.0, e = 0.0;
  for (int k = l; k < n; k += WAVE) {
    a += static_cast<double>(pb.slot_dA[static_cast<int64_t>(k) * pb.H + h]);
    d += static_cast<double>(pb.slot_dD[static_cast<int64_t>(k) * pb.H + h]);
    if (pb.ddt_bias) e += static_cast<double>(pb.slot_ddtb[static_cast<int64_t>(k) * pb.H + h]);
  }
  a = wave_sum_f64(a);
  d = wave_sum_f64(d);
  e = wave_sum_f64(e);
  if (l == 0) {
    pb.dA[h] = static_cast<float>(a);
    if (pb.dD && !pb.d_hp) pb.dD[h] = static_cast<float>(d);
    if (pb.ddt_bias) pb.ddt_bias[h] = static_cast<float>(e);
  }
}

// Per-channel dD: one thread per (h, p), the (b, c) slots in order, in double.
__global__ __launch_bounds__(256) void k_reduce_dp(Problem pb) {
  const int hp = blockIdx.x * 256 + threadIdx.x;
  if (hp >= pb.H * pb.P) return;
  const int n = pb.B * pb.nc;
  double d = 0.0;
  for (int k = 0; k < n; ++k) d += static_cast<double>(pb.slot_dDp[static_cast<int64_t>(k) * pb.H * pb.P + hp]);
  pb.dD[hp] = static_cast<float>(d);
}

hipError_t launch_prep(const Problem& pb, hipStream_t s) {
  const dim3 grid(pb.nc, pb.B, (pb.H + PREP_HEADS - 1) / PREP_HEADS);
  switch (pb.Q) {
    case 64: hipLaunchKernelGGL(k_prep<64>, grid, dim3(256), 0, s, pb); break;
    case 128: hipLaunchKernelGGL(k_prep<128>, grid, dim3(256), 0, s, pb); break;
    case 256: hipLaunchKernelGGL(k_prep<256>, grid, dim3(256), 0, s, pb); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_seqbase, dim3(1), dim3(WAVE), 0, s, pb);
  return hipGetLastError();
}

hipError_t launch_reduce(const Problem& pb, hipStream_t s) {
  hipLaunchKernelGGL(k_reduce, dim3((pb.H + 3) / 4), dim3(256), 0, s, pb);
  if (pb.d_hp && pb.dD) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_reduce_dp, dim3((pb.H * pb.P + 255) / 256), dim3(256), 0, s, pb);
  }
  return hipGetLastError();
}

}  // namespace ssd
