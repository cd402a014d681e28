// Depthwise causal convolution of the Mamba-2 block (forward and its
// deterministic backward) for gfx950.  The operation and its gradients are
// written out in include/causal_conv1d.h; the page "Deterministic bwd kernel
// for mamba2" (state-spaces/mamba PR 827, "Atomic add non-determinism") is
// why the filter gradient here is a fixed-order sum and not an atomic one.
//
// The op is bound by HBM (x and dout read once, out or dx written once; the
// filter has W <= 4 taps), so the kernels are streaming walks, not
// contractions:
//
// * A lane owns 16 bytes (forward) or 8 bytes (backward) of channels, a
//   wave 64 lanes side by side, so every row load or store of a wave is one
//   contiguous 1 KiB or 512-byte piece of a channels-last row.
// * Each wave walks TT consecutive rows, keeping the last W input rows (and,
//   in the backward, the last W values of g = dout * act'(pre)) in registers,
//   with DEPTH rows of loads in flight ahead of the row it computes.  The
//   W-1 rows before its first row are read once more as a halo.
// * Each staged row's sequence key (the number of sequence starts in the
//   block's rows up to it) is staged in LDS.  A window of W rows that lies in
//   one sequence (nearly all of them) takes the unmasked path; a window
//   across a sequence start, the first row or the end of the input takes the
//   masked one.  Both tests are wave-uniform.
// * Backward: the filter and bias gradients of the block's NWAVE * TT rows are
//   summed in registers (row order), then over the block's 4 waves in wave
//   order through LDS, and parked in the block's own slot of the workspace;
//   k_conv_reduce adds the slots in slot order in double.  No atomics.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "causal_conv1d.h"
#include "ssd_device.h"

namespace conv {

using ssd::bf16_t;
using ssd::pack_bf16x2;

constexpr int WAVE = 64;
constexpr int NWAVE = 4;          // waves per block, one run of rows each
constexpr int NTHR = NWAVE * WAVE;
// sequence ids of the rows before the first and past the last (never in the same sequence as a real row)
constexpr int BEFORE_START = INT32_MIN, PAST_END = INT32_MIN + 1;

// Rows per wave, bytes per lane and rows requested ahead (DEPTH) of each walk,
// from a sweep at L = 16384 and 10240 bf16 channels.  The backward carries
// more state per lane (the g ring and the gradient sums): with 8 bytes per
// lane it keeps 3 waves per SIMD, and its longer runs amortise the halo rows
// and the per-block slot.  NTL / NTS: the walk's row loads / stores carry the
// nontemporal hint (every byte is touched once; measured per walk).
template <bool BWD> struct Walk {
  static constexpr int TT = BWD ? 128 : 32;
  static constexpr int NB = BWD ? 8 : 16;
  static constexpr int DEPTH = BWD ? 4 : 8;
  static constexpr int RB = NWAVE * TT;   // rows per block
  static constexpr bool NTL = BWD, NTS = true;
};

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <int NWD> struct RawT;
template <> struct RawT<2> { using type = u32x2_t; };
template <> struct RawT<4> { using type = u32x4_t; };

// A lane's NB bytes of one row: load, store, and conversion to and from fp32
template <typename T, int NB, bool NTL = false, bool NTS = false> struct Io {
  static constexpr int VEC = NB / static_cast<int>(sizeof(T)), NWD = NB / 4;
  using raw = typename RawT<NWD>::type;
  static __device__ __forceinline__ raw load(const T* p) {
    if constexpr (NTL) return __builtin_nontemporal_load(reinterpret_cast<const raw*>(p));
    else return *reinterpret_cast<const raw*>(p);
  }
  static __device__ __forceinline__ void store(T* p, raw r) {
    if constexpr (NTS) __builtin_nontemporal_store(r, reinterpret_cast<raw*>(p));
    else *reinterpret_cast<raw*>(p) = r;
  }
  static __device__ __forceinline__ void unpack(raw u, float (&f)[VEC]) {
#pragma unroll
    for (int i = 0; i < NWD; ++i) {
      if constexpr (sizeof(T) == 2) {
        f[2 * i] = __uint_as_float(u[i] << 16);
        f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
      } else {
        f[i] = __uint_as_float(u[i]);
      }
    }
  }
  static __device__ __forceinline__ raw pack(const float (&f)[VEC]) {
    raw r;
#pragma unroll
    for (int i = 0; i < NWD; ++i) r[i] = sizeof(T) == 2 ? pack_bf16x2(f[2 * i], f[2 * i + 1]) : __float_as_uint(f[i]);
    return r;
  }
};

struct Args {
  const void* x;
  const float* w;
  const float* bias;
  const int32_t* seq;
  const void* dout;
  void* y;        // out (forward) or dx (backward)
  float* part;    // backward: per-block partials, (slots, W + 1, C)
  int64_t L, C;
  int ntb;        // row blocks per batch row
};

// SiLU and its derivative from one exponential and one hardware reciprocal
// (v_rcp_f32, 1 ulp; an IEEE division would cost about ten instructions per element)
__device__ __forceinline__ float sigmoid(float p) { return __builtin_amdgcn_rcpf(1.f + __expf(-p)); }

template <typename T, int W, bool SILU, bool BWD>
__global__ __launch_bounds__(NTHR) void k_conv(Args a) {
  using IO = Io<T, Walk<BWD>::NB, Walk<BWD>::NTL, Walk<BWD>::NTS>;
  constexpr int TT = Walk<BWD>::TT, RB = Walk<BWD>::RB, DEPTH = Walk<BWD>::DEPTH;
  constexpr int VEC = IO::VEC, CB = WAVE * VEC;
  constexpr int NSTEP = BWD ? (TT + W - 1 + DEPTH - 1) / DEPTH * DEPTH : TT;
  // rows tb0-(W-1) .. up to the last wave's last step
  constexpr int SEQN = (NWAVE - 1) * TT + NSTEP + W - 1;
  __shared__ int s_seq[SEQN];
  __shared__ float s_part[BWD ? NWAVE * (W + 1) * CB : 1];

  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int64_t b = blockIdx.z, L = a.L, C = a.C;
  const int64_t tb0 = static_cast<int64_t>(blockIdx.y) * RB;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * CB + lane * VEC;
  const bool cok = c0 < C;
  const int64_t cl = cok ? c0 : C - VEC;                 // loads stay in bounds for idle lanes

  // Sequence key of each staged row: a sequence starts at row t when t == 0
  // or seq_idx changes at t, and a real row's key counts the starts among
  // the staged rows up to it, so two rows less than W apart have equal keys
  // exactly when no sequence starts between them.  Rows before the first and
  // past the last get the sentinels.  (Start flags first, then one wave's
  // prefix sum over the window.)
  for (int i = tid; i < SEQN; i += NTHR) {
    const int64_t t = tb0 - (W - 1) + i;
    int st = 0;
    if (t >= 0 && t < L) st = (t == 0) || (a.seq && a.seq[b * L + t] != a.seq[b * L + t - 1]);
    s_seq[i] = st;
  }
  float wt[W][VEC], bi[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
#pragma unroll
    for (int k = 0; k < W; ++k) wt[k][e] = a.w[(cl + e) * W + k];
    bi[e] = a.bias ? a.bias[cl + e] : 0.f;
  }
  __syncthreads();
  if (wv == 0) {
    constexpr int PER = (SEQN + WAVE - 1) / WAVE;   // consecutive entries per lane
    int loc[PER], run = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = lane * PER + e;
      run += i < SEQN ? s_seq[i] : 0;
      loc[e] = run;
    }
    int incl = run;   // inclusive scan of the lanes' totals
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
      const int u = __shfl_up(incl, off, WAVE);
      if (lane >= off) incl += u;
    }
    const int base = incl - run;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = lane * PER + e;
      if (i < SEQN) {
        const int64_t t = tb0 - (W - 1) + i;
        s_seq[i] = t < 0 ? BEFORE_START : t >= L ? PAST_END : base + loc[e];
      }
    }
  }
  __syncthreads();

  const int64_t t0 = tb0 + wv * TT;                      // this wave's first row
  const T* xb = static_cast<const T*>(a.x) + b * L * C + cl;
  const T* db = BWD ? static_cast<const T*>(a.dout) + b * L * C + cl : nullptr;
  T* yb = static_cast<T*>(a.y) + b * L * C + c0;
  auto row = [&](int64_t t) { return min(max(t, static_cast<int64_t>(0)), L - 1) * C; };
  // seq id of row t (wave-uniform, kept in a scalar register)
  auto seq_of = [&](int64_t t) { return __builtin_amdgcn_readfirstlane(s_seq[t - tb0 + (W - 1)]); };

  // rings: xr[k] = x[t - (W-1) + k], gr[k] = g[t - (W-1) + k], sr[k] their sequence ids
  float xr[W][VEC], gr[W][VEC];
  int sr[W];
#pragma unroll
  for (int k = 1; k < W; ++k) {
    const int64_t t = t0 - W + k;
    IO::unpack(IO::load(xb + row(t)), xr[k]);
    sr[k] = seq_of(t);
#pragma unroll
    for (int e = 0; e < VEC; ++e) gr[k][e] = 0.f;
  }
  float dwa[W][VEC], dba[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    dba[e] = 0.f;
#pragma unroll
    for (int k = 0; k < W; ++k) dwa[k][e] = 0.f;
  }

  typename IO::raw rx[DEPTH], rd[DEPTH];
#pragma unroll
  for (int u = 0; u < DEPTH; ++u) {
    rx[u] = IO::load(xb + row(t0 + u));
    if constexpr (BWD) rd[u] = IO::load(db + row(t0 + u));
  }

  // next rows to request, and the last row (requests past the end reload it)
  const T* nx = xb + (t0 + DEPTH) * C;
  const T* nd = BWD ? db + (t0 + DEPTH) * C : nullptr;
  // the last row this wave reads (its run, plus W-1 rows of g for the backward); requests
  // past it reload that row instead, which is already in the cache, rather than pull the
  // next run's rows from HBM ahead of the wave that reads them
  const int64_t tend = min(L, t0 + (BWD ? TT + W - 1 : TT)) - 1;
  const T* xlast = xb + tend * C;
  const T* dlast = BWD ? db + tend * C : nullptr;
  for (int s0 = 0; s0 < NSTEP; s0 += DEPTH) {
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const int s = s0 + u;
      const int64_t t = t0 + s;                          // the row this step reads
#pragma unroll
      for (int k = 0; k < W - 1; ++k) {
        sr[k] = sr[k + 1];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          xr[k][e] = xr[k + 1][e];
          gr[k][e] = gr[k + 1][e];
        }
      }
      IO::unpack(rx[u], xr[W - 1]);
      float dv[VEC];
      if constexpr (BWD) IO::unpack(rd[u], dv);
      sr[W - 1] = seq_of(t);
      // next request into the slot just consumed (past the run: a reload of its last row)
      // (kept after the unpacks above, so that the request can reuse their registers:
      // a request issued before them would leave a copy, and a wait, at the loop's end)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        asm volatile("" : "+v"(xr[W - 1][e]));
        if constexpr (BWD) asm volatile("" : "+v"(dv[e]));
      }
      __builtin_amdgcn_sched_barrier(0);
      const bool in = t + DEPTH <= tend;
      rx[u] = IO::load(in ? nx : xlast);
      if constexpr (BWD) rd[u] = IO::load(in ? nd : dlast);
      nx += C;
      if constexpr (BWD) nd += C;

      bool uni = true;
#pragma unroll
      for (int k = 0; k < W - 1; ++k) uni = uni && sr[k] == sr[W - 1];
      // pre-activation of row t: taps from rows of t's own sequence
      float keep[W];
#pragma unroll
      for (int k = 0; k < W; ++k) keep[k] = (uni || sr[k] == sr[W - 1]) ? 1.f : 0.f;
      float pre[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float acc = bi[e];
        if (uni) {
#pragma unroll
          for (int k = 0; k < W; ++k) acc = fmaf(wt[k][e], xr[k][e], acc);
        } else {
#pragma unroll
          for (int k = 0; k < W; ++k) acc = fmaf(wt[k][e] * keep[k], xr[k][e], acc);
        }
        pre[e] = acc;
      }
      if constexpr (!BWD) {
        if (t < t0 + TT && t < L && cok) {
          float o[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) o[e] = SILU ? pre[e] * sigmoid(pre[e]) : pre[e];
          IO::store(yb + t * C, IO::pack(o));
        }
      } else {
        const bool live = t < L;                         // g past the end is zero
        float g[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float d = 1.f;
          if (SILU) {
            const float sg = sigmoid(pre[e]);
            d = sg * fmaf(pre[e], 1.f - sg, 1.f);
          }
          g[e] = live ? dv[e] * d : 0.f;
        }
        if (s < TT && live) {                            // row t is one of this wave's rows
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            dba[e] += g[e];
            if (uni) {
#pragma unroll
              for (int k = 0; k < W; ++k) dwa[k][e] = fmaf(g[e], xr[k][e], dwa[k][e]);
            } else {
#pragma unroll
              for (int k = 0; k < W; ++k) dwa[k][e] = fmaf(g[e] * keep[k], xr[k][e], dwa[k][e]);
            }
          }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) gr[W - 1][e] = g[e];
        // dx of row t - (W-1): taps to rows of its own sequence
        const int64_t tx = t - (W - 1);
        if (s >= W - 1 && s < TT + W - 1 && tx < L && cok) {
          float o[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            float acc = 0.f;
            if (uni) {
#pragma unroll
              for (int k = 0; k < W; ++k) acc = fmaf(wt[k][e], gr[W - 1 - k][e], acc);
            } else {
#pragma unroll
              for (int k = 0; k < W; ++k) {
                const float m = sr[W - 1 - k] == sr[0] ? 1.f : 0.f;
                acc = fmaf(wt[k][e] * m, gr[W - 1 - k][e], acc);
              }
            }
            o[e] = acc;
          }
          IO::store(yb + tx * C, IO::pack(o));
        }
      }
    }
  }

  if constexpr (BWD) {
    // the block's partials: waves summed in wave order, then one slot per block
#pragma unroll
    for (int k = 0; k <= W; ++k) {
      float* dst = s_part + (wv * (W + 1) + k) * CB + lane * VEC;
#pragma unroll
      for (int e = 0; e < VEC; ++e) dst[e] = k < W ? dwa[k][e] : dba[e];
    }
    __syncthreads();
    const int64_t slot = b * a.ntb + blockIdx.y;
    const int64_t cb0 = static_cast<int64_t>(blockIdx.x) * CB;
    for (int i = tid; i < (W + 1) * CB; i += NTHR) {
      const int k = i / CB, cc = i % CB;
      float sum = s_part[k * CB + cc];
#pragma unroll
      for (int v = 1; v < NWAVE; ++v) sum += s_part[(v * (W + 1) + k) * CB + cc];
      if (cb0 + cc < C) a.part[(slot * (W + 1) + k) * C + cb0 + cc] = sum;
    }
  }
}

// dweight[c][k] and dbias[c]: the slots added in slot order, in double.  Small
// blocks spread the (W + 1) * C sums over every CU; the slot loads are issued
// 32 (then 8) at a time ahead of their (ordered) adds.
constexpr int RED_THR = 64;
__global__ __launch_bounds__(RED_THR) void k_conv_reduce(const float* part, int64_t nslot, int64_t C, int W,
                                                         float* dw, float* dbias) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= (W + 1) * C) return;
  const int64_t k = i / C, c = i % C;
  const int64_t stride = (W + 1) * C;
  const float* p = part + k * C + c;
  double acc = 0.0;
  int64_t s = 0;
  for (; s + 32 <= nslot; s += 32) {
    float v[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = p[(s + j) * stride];
#pragma unroll
    for (int j = 0; j < 32; ++j) acc += static_cast<double>(v[j]);
  }
  for (; s + 8 <= nslot; s += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = p[(s + j) * stride];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += static_cast<double>(v[j]);
  }
  for (; s < nslot; ++s) acc += static_cast<double>(p[s * stride]);
  if (k < W) {
    dw[c * W + k] = static_cast<float>(acc);
  } else if (dbias) {
    dbias[c] = static_cast<float>(acc);
  }
}

template <bool BWD>
int64_t row_blocks(const conv1d_shape& s) { return (s.seqlen + Walk<BWD>::RB - 1) / Walk<BWD>::RB; }

int check(const conv1d_shape* s) {
  if (!s || s->reserved != 0) return SSD_ERR_INVALID_ARG;
  if (s->batch < 1 || s->seqlen < 1 || s->channels < 1) return SSD_ERR_UNSUPPORTED_SHAPE;
  if (s->width < 2 || s->width > 4) return SSD_ERR_UNSUPPORTED_SHAPE;
  if (s->activation != CONV1D_ACT_NONE && s->activation != CONV1D_ACT_SILU) return SSD_ERR_UNSUPPORTED_SHAPE;
  if (s->io_dtype != SSD_IO_BF16 && s->io_dtype != SSD_IO_F32) return SSD_ERR_UNSUPPORTED_SHAPE;
  const int vec = s->io_dtype == SSD_IO_BF16 ? 8 : 4;
  if (s->channels % vec != 0) return SSD_ERR_UNSUPPORTED_SHAPE;
  if (s->batch > 65535 || row_blocks<false>(*s) > 65535) return SSD_ERR_UNSUPPORTED_SHAPE;
  return SSD_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename T, int W, bool SILU, bool BWD>
void launch(const conv1d_shape& s, const Args& a, hipStream_t st) {
  constexpr int CB = WAVE * Io<T, Walk<BWD>::NB>::VEC;
  const dim3 grid(static_cast<unsigned>((s.channels + CB - 1) / CB), static_cast<unsigned>(row_blocks<BWD>(s)),
                  static_cast<unsigned>(s.batch));
  hipLaunchKernelGGL((k_conv<T, W, SILU, BWD>), grid, dim3(NTHR), 0, st, a);
}

template <typename T, bool BWD>
void dispatch(const conv1d_shape& s, const Args& a, hipStream_t st) {
  const bool silu = s.activation == CONV1D_ACT_SILU;
  switch (s.width) {
    case 2: silu ? launch<T, 2, true, BWD>(s, a, st) : launch<T, 2, false, BWD>(s, a, st); break;
    case 3: silu ? launch<T, 3, true, BWD>(s, a, st) : launch<T, 3, false, BWD>(s, a, st); break;
    default: silu ? launch<T, 4, true, BWD>(s, a, st) : launch<T, 4, false, BWD>(s, a, st); break;
  }
}

}  // namespace conv

extern "C" {

int conv1d_bwd_workspace_size(const conv1d_shape* shape, size_t* bytes) {
  const int rc = conv::check(shape);
  if (rc != SSD_OK) return rc;
  if (!bytes) return SSD_ERR_INVALID_ARG;
  *bytes = static_cast<size_t>(shape->batch * conv::row_blocks<true>(*shape)) * (shape->width + 1) *
           static_cast<size_t>(shape->channels) * sizeof(float);
  return SSD_OK;
}

int conv1d_fwd(const conv1d_shape* shape, const void* x, const float* weight, const float* bias,
               const int32_t* seq_idx, void* out, void* stream) {
  const int rc = conv::check(shape);
  if (rc != SSD_OK) return rc;
  if (!x || !weight || !out) return SSD_ERR_INVALID_ARG;
  if (!conv::aligned16(x) || !conv::aligned16(out)) return SSD_ERR_MISALIGNED;
  if (out == x) return SSD_ERR_INVALID_ARG;
  conv::Args a{x, weight, bias, seq_idx, nullptr, out, nullptr, shape->seqlen, shape->channels,
               static_cast<int>(conv::row_blocks<false>(*shape))};
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (shape->io_dtype == SSD_IO_BF16) {
    conv::dispatch<ssd::bf16_t, false>(*shape, a, st);
  } else {
    conv::dispatch<float, false>(*shape, a, st);
  }
  return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

int conv1d_bwd(const conv1d_shape* shape, const void* x, const float* weight, const float* bias,
               const int32_t* seq_idx, const void* dout, void* dx, float* dweight, float* dbias,
               void* workspace, size_t workspace_bytes, void* stream) {
  size_t need = 0;
  const int rc = conv1d_bwd_workspace_size(shape, &need);
  if (rc != SSD_OK) return rc;
  if (!x || !weight || !dout || !dx || !dweight || !workspace) return SSD_ERR_INVALID_ARG;
  if (workspace_bytes < need) return SSD_ERR_WORKSPACE_TOO_SMALL;
  if (!conv::aligned16(x) || !conv::aligned16(dout) || !conv::aligned16(dx) || !conv::aligned16(workspace))
    return SSD_ERR_MISALIGNED;
  if (dx == x || dx == dout) return SSD_ERR_INVALID_ARG;
  const int64_t ntb = conv::row_blocks<true>(*shape);
  conv::Args a{x, weight, bias, seq_idx, dout, dx, static_cast<float*>(workspace), shape->seqlen,
               shape->channels, static_cast<int>(ntb)};
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (shape->io_dtype == SSD_IO_BF16) {
    conv::dispatch<ssd::bf16_t, true>(*shape, a, st);
  } else {
    conv::dispatch<float, true>(*shape, a, st);
  }
  const int64_t n = (shape->width + 1) * shape->channels;
  hipLaunchKernelGGL(conv::k_conv_reduce, dim3(static_cast<unsigned>((n + conv::RED_THR - 1) / conv::RED_THR)),
                     dim3(conv::RED_THR), 0, st,
                     static_cast<const float*>(workspace), shape->batch * ntb, shape->channels, shape->width,
                     dweight, dbias);
  return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // extern "C"
