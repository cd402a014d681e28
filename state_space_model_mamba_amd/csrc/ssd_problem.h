// Problem descriptor shared by the host code and the kernels of the SSD
// backward, plus the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// Per-(batch, chunk) integer record in the workspace.
//   [0] number of sequence starts inside the chunk
//   [1] unused
//   [2] unused
//   [3] global index of the first sequence that starts in the chunk
constexpr int CINFO = 4;

// segpos entry of chunk position i: low 16 bits = first position of i's
// segment inside the chunk, high 16 bits = number of sequence starts at
// positions <= i inside the chunk (0: the segment continues the previous
// chunk's sequence).
__host__ __device__ inline int seg_lo(int v) { return v & 0xffff; }
__host__ __device__ inline int seg_rank(int v) { return v >> 16; }

struct Problem {
  int B, L, H, P, G, N, Q, nc, hpg, nseqs;
  int ntg;  // number of dstate tiles of the group kernel (dC, dB, offd, endd)
  // inputs
  const void* x;
  const float* dt;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* D;
  const void* dy;
  const float* h0;
  const int32_t* seq_idx;
  // outputs
  void* dx;
  float* ddt;
  float* dA;
  void* dB;
  void* dC;
  float* dD;
  float* dinit;
  // dt front-end (fe = 0: dt is used as given)
  int fe;                // nonzero when any of the three below applies
  const float* dt_bias;  // (H) or nullptr
  const float* dlast;    // (B, H, P, N) gradient of each row's state after position L-1, or nullptr
  int dt_softplus;
  float dt_min, dt_max;
  float* ddt_bias;       // (H) output, nullable
  int d_hp;              // nonzero: D and dD are (H, P)
  // output gate (nullable): out = y silu(z); the backward's gate pass reads
  // dout and writes the gated dy into y's place (the dx buffer) and dz
  const void* z;     // (B, L, H, P), I/O dtype
  const void* dout;  // gate pass only: the gradient of the gated output
  void* dz;          // gate pass only
  // forward outputs
  void* y;           // (B, L, H, P), I/O dtype
  void* ypre;        // (B, L, H, P), I/O dtype, nullable: y before the output gate (forward writes,
                     // the backward's elementwise gate pass reads)
  float* final;      // (nseqs, H, P, N) fp32, nullable
  // workspace
  int32_t* segpos;   // (B, nc, Q)
  int32_t* cinfo;    // (B, nc, CINFO)
  float* acs;        // (B, H, nc, Q)
  float* dtc;        // (B, H, nc, Q)
  float* dfe;        // (B, H, nc, Q): d dtc / d raw dt (written and read only with a dt front-end)
  void* hin;         // (B, H, nc, P, N), I/O dtype
  void* dstate;      // (B, H, nc, P, N), I/O dtype
  void* dcb;         // (B, G, nc, Q, Q) io dtype: head-summed intra-chunk dCB (split group path)
  void* dcbt;        // (B, G, nc, Q, Q) io dtype: its transpose (split group path)
  int nslice;        // head slices of the split group path's dCB kernel (1: one block per (b, g, c))
  float* dcbp;       // (B, G, nc, nslice, causal tiles, 256) fp32: the slices' dCB sums (nslice > 1)
  int nslice_bd;     // head slices of the split path's dC / dB kernels (1: one block per (b, g, c, tile))
  float* dcp;        // (B, G, nc, ntg, nslice_bd, Q, N / ntg) fp32: the slices' dC rows (nslice_bd > 1)
  float* dbp;        // the same for dB
  float* cbt;        // (B, G, nc, Q(Q+16)/512 tiles, 256): C B^T causal tiles, fp32, in the
                     // causal split's (wave, tile) order and accumulator lane layout
  float* offd;       // (B, H, nc, ntg, Q)
  float* endd;       // (B, H, nc, ntg)
  float* slot_dA;    // (B, nc, H)
  float* slot_dD;    // (B, nc, H)
  float* slot_ddtb;  // (B, nc, H): dt_bias gradient partials
  float* slot_dDp;   // (B, nc, H, P): per-channel dD partials
  int32_t* seqstart; // (nseqs): b * L + t of each sequence's first position (forward)
};

// The dt front-end of one raw value of head h: the activated, clamped dt and
// (if dfdu) its derivative with respect to the raw value.  softplus(u) =
// ln(1 + e^u), taken as u above 20, where the two agree to float precision.
__device__ inline float dt_frontend(const Problem& pb, float raw, int h, float* dfdu) {
  const float u = raw + (pb.dt_bias ? pb.dt_bias[h] : 0.f);
  float v = u, d = 1.f;
  if (pb.dt_softplus && u <= 20.f) {
    v = log1pf(expf(u));
    d = 1.f / (1.f + expf(-u));
  }
  const bool in = v >= pb.dt_min && v <= pb.dt_max;
  if (dfdu) *dfdu = in ? d : 0.f;
  return fminf(fmaxf(v, pb.dt_min), pb.dt_max);
}

// Raises `kernel`'s dynamic-LDS limit to `bytes` once per device (the
// device current on the calling thread); thread-safe.  Every launcher calls
// it before launching a kernel that needs more than the default.
hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes);

// Launch geometry that is not fixed by the problem shape alone, as
// overridden through ssd_set_launch_geometry (0: the shape-derived default).
// The results do not depend on either value.
int head_blocks_override();
int fwd_heads_per_block_override();

// Persistent blocks of the head kernel: a constant (the CU count of one
// MI355X), so the grid is a function of the problem shape only.
constexpr int kHeadBlocks = 256;

// Launchers (defined next to their kernels).  Return hipSuccess or the
// launch error.  io_bf16 selects the bf16 (true) or fp32 instantiation.
hipError_t launch_prep(const Problem& pb, hipStream_t s);
hipError_t launch_state_fwd(const Problem& pb, bool io_bf16, hipStream_t s);
hipError_t launch_state_bwd(const Problem& pb, bool io_bf16, hipStream_t s);
// the group stage, split: dCB and C B^T tiles (k_dcb), then dC (k_dc) and dB (k_db)
hipError_t launch_dcb(const Problem& pb, bool io_bf16, hipStream_t s);
hipError_t launch_dbdc(const Problem& pb, bool io_bf16, hipStream_t s);
// the group stage, fused: C B^T tiles (k_cb), then dCB, dC and dB per 64-row slab (k_grp)
hipError_t launch_cb(const Problem& pb, bool io_bf16, hipStream_t s);
hipError_t launch_grp(const Problem& pb, bool io_bf16, hipStream_t s);
hipError_t launch_head_bwd(const Problem& pb, bool io_bf16, hipStream_t s);
hipError_t launch_reduce(const Problem& pb, hipStream_t s);
// forward: sequence start table, then C B^T tiles, y and (if requested) the
// sequences' final states
hipError_t launch_seqstart(const Problem& pb, hipStream_t s);
hipError_t launch_fwd_out(const Problem& pb, bool io_bf16, hipStream_t s);
hipError_t launch_gate_bwd(const Problem& pb, bool io_bf16, hipStream_t s);

// The (chunk_size, headdim) pairs compiled for each io dtype.  bf16 needs
// headdim % 32 == 0 (one MFMA k-step over P); fp32 stops at chunk 128 so that
// its LDS tiles fit one workgroup.
#define SSD_BF16_SHAPES(X) X(64, 32) X(64, 64) X(128, 32) X(128, 64) X(256, 32) X(256, 64)
#define SSD_F32_SHAPES(X) X(64, 16) X(64, 32) X(64, 64) X(128, 16) X(128, 32) X(128, 64)

// Shape support (host side): true when kernels exist for this combination
// and fit the LDS of one workgroup.
int group_ntile(int N, bool io_bf16);   // dstate tile of k_dc / k_db
int grp_ntile(int N, bool io_bf16);     // dstate tile of k_grp
// Which group path a shape takes (0: by shape, 1: fused, 2: split), as
// overridden through ssd_set_group_path.
int group_path_override();
size_t dcb_lds_bytes(int Q, int P, bool io_bf16);
size_t dbdc_lds_bytes(int Q, int P, int NTG, bool io_bf16);
size_t grp_lds_bytes(int Q, int P, int NTG, bool io_bf16);
size_t head_lds_bytes(int Q, int P, bool io_bf16);
size_t fwd_lds_bytes(int Q, int P, bool io_bf16);

}  // namespace ssd
