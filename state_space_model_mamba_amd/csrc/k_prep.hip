// Chunk preparation, sequence numbering and the final fixed-order reduction.
//
// k_prep (the forward half of chunk_cumsum named on the page "Deterministic
// bwd kernel for mamba2"): per (batch, chunk) it finds the sequence starts,
// records each position's segment, and for every head writes
//   Acs_i = sum of dt_k * A_h over k from the start of i's segment to i,
// restarted at the chunk start and at every sequence start.  The scan order
// is fixed by the chunk size alone: each lane adds its Q/64 consecutive
// elements in order, then a 64-lane Hillis-Steele segmented scan over lane
// totals (shuffle offsets 1, 2, ..., 32) supplies the carry.  That page
// reports that a cumsum whose result changes with the block shape broke
// run-to-run reproducibility; here the result does not depend on how many
// heads a block handles or on the launch shape.
#include "ssd_device.h"
#include "ssd_problem.h"

namespace ssd {

template <int Q>
__global__ __launch_bounds__(256) void k_prep(Problem pb) {
  static_assert(Q % WAVE == 0 && Q <= 256, "chunk size");
  constexpr int R = Q / WAVE;
  const int c = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ int s_flag[Q], s_lo[Q], s_rank[Q];

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
  const int64_t bc = static_cast<int64_t>(b) * pb.nc + c;
  if (tid < Q) pb.segpos[bc * Q + tid] = s_lo[tid] | (s_rank[tid] << 16);
  if (tid == 0) {
    pb.cinfo[bc * CINFO + 0] = s_rank[Q - 1];
    pb.cinfo[bc * CINFO + 1] = 0;
    pb.cinfo[bc * CINFO + 2] = 0;
  }

  const int w = wave_id(), l = lane_id(), nw = blockDim.x / WAVE;
  for (int h = w; h < pb.H; h += nw) {
    const float Ah = pb.A[h];
    float loc[R], d[R];
    int f[R];
#pragma unroll
    for (int e = 0; e < R; ++e) {
      const int i = l * R + e, t = c * Q + i;
      d[e] = (t < pb.L) ? pb.dt[(static_cast<int64_t>(b) * pb.L + t) * pb.H + h] : 0.f;
      f[e] = (i == 0) || s_flag[i];
    }
    float run = 0.f;
    int any = 0;
#pragma unroll
    for (int e = 0; e < R; ++e) {
      const float a = d[e] * Ah;
      if (f[e]) {
        run = a;
        any = 1;
      } else {
        run += a;
      }
      loc[e] = run;
    }
    float v = run;
    int fl = any;
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
      const float vu = __shfl_up(v, off, WAVE);
      const int fu = __shfl_up(fl, off, WAVE);
      if (l >= off) {
        if (!fl) v = vu + v;
        fl |= fu;
      }
    }
    float carry = __shfl_up(v, 1, WAVE);
    if (l == 0) carry = 0.f;
    int seen = 0;
    const int64_t out = ((static_cast<int64_t>(b) * pb.H + h) * pb.nc + c) * Q;
#pragma unroll
    for (int e = 0; e < R; ++e) {
      const int i = l * R + e;
      if (f[e]) seen = 1;
      pb.acs[out + i] = seen ? loc[e] : loc[e] + carry;
      pb.dtc[out + i] = d[e];
    }
  }
}

// Global numbering of sequence starts: exclusive prefix sum of the per-chunk
// start counts in row-major (batch, chunk) order.  One block; integer only.
__global__ __launch_bounds__(256) void k_seqbase(Problem pb) {
  __shared__ int s[256];
  __shared__ int s_run;
  const int tid = threadIdx.x;
  const int total = pb.B * pb.nc;
  if (tid == 0) s_run = 0;
  __syncthreads();
  for (int base = 0; base < total; base += 256) {
    const int idx = base + tid;
    const int v = idx < total ? pb.cinfo[static_cast<int64_t>(idx) * CINFO] : 0;
    s[tid] = v;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int u = tid >= off ? s[tid - off] : 0;
      __syncthreads();
      s[tid] += u;
      __syncthreads();
    }
    if (idx < total) pb.cinfo[static_cast<int64_t>(idx) * CINFO + 3] = s_run + s[tid] - v;
    __syncthreads();
    if (tid == 255) s_run += s[255];
    __syncthreads();
  }
}

// dA_h = sum over (b, c) of slot_dA[b, c, h], dD likewise: one thread per
// head, summing in ascending (b, c) order.
__global__ __launch_bounds__(256) void k_reduce(Problem pb) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= pb.H) return;
  float a = 0.f, d = 0.f;
  for (int b = 0; b < pb.B; ++b)
    for (int c = 0; c < pb.nc; ++c) {
      const int64_t k = (static_cast<int64_t>(b) * pb.nc + c) * pb.H + h;
      a += pb.slot_dA[k];
      d += pb.slot_dD[k];
    }
  pb.dA[h] = a;
  if (pb.dD) pb.dD[h] = d;
}

hipError_t launch_prep(const Problem& pb, hipStream_t s) {
  const dim3 grid(pb.nc, pb.B);
  switch (pb.Q) {
    case 64: hipLaunchKernelGGL(k_prep<64>, grid, dim3(256), 0, s, pb); break;
    case 128: hipLaunchKernelGGL(k_prep<128>, grid, dim3(256), 0, s, pb); break;
    case 256: hipLaunchKernelGGL(k_prep<256>, grid, dim3(256), 0, s, pb); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_seqbase, dim3(1), dim3(256), 0, s, pb);
  return hipGetLastError();
}

hipError_t launch_reduce(const Problem& pb, hipStream_t s) {
  hipLaunchKernelGGL(k_reduce, dim3((pb.H + 255) / 256), dim3(256), 0, s, pb);
  return hipGetLastError();
}

}  // namespace ssd
