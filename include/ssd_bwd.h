/*
 * ssd_bwd.h -- C ABI of libssd_bwd.so: the deterministic backward of the
 * Mamba-2 SSD (state space duality) chunked scan on AMD Instinct MI355X
 * (gfx950).
 *
 * The operation.  The page "Deterministic bwd kernel for mamba2"
 * (state-spaces/mamba PR 827, its per-kernel breakdown table) lists the
 * kernels of this backward -- chunk_cumsum_bwd, chunk_state_bwd_dx/db/ddAcs,
 * chunk_scan_bwd_dC/dx and combined_bwd_dx -- and makes them free of
 * floating-point atomics; the page "Fix Incorrect Gradients and Illegal
 * Memory Access Error in Mamba2" (PR 537) discusses the ddA_cumsum ("stable")
 * kernel.  Neither page writes the equations; the layer is the SSD
 * recurrence
 *
 *     a_t = dt_t * A_h
 *     h_t = exp(a_t) * h_{t-1} + dt_t * x_t (outer) B_t        (P x N per head)
 *     y_t = h_t C_t + D_h * x_t
 *
 * per batch row and head, restarted at every sequence start with
 * h_{t0-1} = initial_states[s] (zeros when not given).  ssd_bwd returns the
 * gradients of  l = sum_t dy_t . y_t  with respect to x, dt, A, B, C, D and
 * the initial states.  It recomputes the forward chunk states internally;
 * nothing from a forward pass is needed.
 *
 * Determinism.  Every output element and every workspace element is written
 * by exactly one thread; cross-head and cross-chunk sums are formed in a
 * fixed order that depends only on the problem shape (partials parked in
 * per-(batch, chunk, head) slots, then summed in index order), the in-chunk
 * cumulative sums use one fixed scan order that depends only on chunk_size,
 * and no floating-point atomics are used.  For the same inputs, shape and
 * library build the output bytes are identical on every call, in every
 * process, on any stream.
 *
 * Layouts (row-major, contiguous, element counts):
 *   x, dy, dx            (batch, seqlen, nheads, headdim)      io dtype
 *   dt, ddt              (batch, seqlen, nheads)               float32
 *   A, D, dA, dD         (nheads)                              float32
 *   B, C, dB, dC         (batch, seqlen, ngroups, dstate)      io dtype
 *   initial_states,
 *   d_initial_states     (nseqs, nheads, headdim, dstate)      float32
 *   seq_idx              (batch, seqlen)                       int32
 * Head h uses group h / (nheads / ngroups).  dt is the already-activated
 * (positive) step.  A sequence starts at (b, t) when t == 0 or
 * seq_idx[b, t] != seq_idx[b, t-1]; starts are numbered 0..nseqs-1 in
 * row-major (b, t) order.  With seq_idx == NULL every batch row is one
 * sequence (nseqs == batch).
 *
 * Ownership and calling convention.  All tensor pointers are device
 * pointers owned by the caller, 16-byte aligned.  Inputs are read-only;
 * outputs are fully overwritten (never accumulated into).  The library never
 * allocates or frees: it uses the caller's workspace, whose contents on entry
 * do not affect the results.  ssd_bwd only enqueues work on `stream`
 * (a hipStream_t; NULL = the default stream) and returns without host
 * synchronisation; argument errors are reported before anything is enqueued.
 * Concurrent calls must use distinct workspaces and outputs.
 */
#ifndef SSD_BWD_H
#define SSD_BWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype of x, B, C, dy and of the outputs dx, dB, dC */
typedef enum { SSD_IO_BF16 = 0, SSD_IO_F32 = 1 } ssd_io_dtype;

typedef struct {
  int64_t batch;      /* >= 1 */
  int64_t seqlen;     /* >= 1; need not be a multiple of chunk_size (tail masked) */
  int64_t nheads;     /* >= 1, multiple of ngroups */
  int64_t headdim;    /* P: 16/32/64 (f32 io) or 32/64 (bf16 io) */
  int64_t ngroups;    /* >= 1 */
  int64_t dstate;     /* N: multiple of 16 (f32) or 32 (bf16), <= 256 */
  int64_t chunk_size; /* Q: 64, 128 or 256 */
  int64_t nseqs;      /* number of sequence starts (see above); == batch without seq_idx */
                      /* also: chunk_size * nheads * headdim and chunk_size * ngroups * dstate
                         elements of the io dtype span at most 2^31 bytes */
  int32_t io_dtype;   /* ssd_io_dtype */
  int32_t reserved;   /* must be 0 */
} ssd_shape;

/* Status codes.  Negative = error; nothing was enqueued. */
enum {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARG = -1,         /* NULL pointer where one is required, bad field */
  SSD_ERR_UNSUPPORTED_SHAPE = -2,   /* shape outside the supported set above */
  SSD_ERR_WORKSPACE_TOO_SMALL = -3, /* workspace_bytes < ssd_bwd_workspace_size() */
  SSD_ERR_MISALIGNED = -4,          /* a pointer is not 16-byte aligned */
  SSD_ERR_HIP = -5                  /* a HIP launch failed (see hipGetLastError) */
};

/* Bytes of device workspace ssd_bwd needs for this shape (written to *bytes).
 * Pure host computation. */
int ssd_bwd_workspace_size(const ssd_shape* shape, size_t* bytes);

/*
 * The backward.  Required: x, dt, A, B, C, dy, dx, ddt, dA, dB, dC, workspace.
 * Optional (NULL allowed):
 *   D                 -- treated as zeros; then dD must be NULL too
 *   dD                -- dD_h = sum over (b, t) of dy . x; needs D
 *   initial_states    -- zeros when NULL
 *   seq_idx           -- one sequence per batch row when NULL
 *   d_initial_states  -- not computed when NULL (computed even when
 *                        initial_states is NULL)
 * nseqs must equal the number of sequence starts seq_idx describes whenever
 * initial_states or d_initial_states is given (it sizes those tensors); the
 * device code clamps sequence indices into [0, nseqs) so a wrong nseqs cannot
 * cause out-of-bounds accesses, but the results are then meaningless.
 * Returns SSD_OK or a negative status.
 */
int ssd_bwd(const ssd_shape* shape, const void* x, const float* dt, const float* A,
            const void* B, const void* C, const float* D, const void* dy,
            const float* initial_states, const int32_t* seq_idx,
            void* dx, float* ddt, float* dA, void* dB, void* dC, float* dD,
            float* d_initial_states, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The forward of the same layer (the kernels chunk_cumsum, chunk_state, state
 * passing and chunk_scan named on the page "Deterministic bwd kernel for
 * mamba2", whose backward twins are above), for callers that pair it with
 * ssd_bwd (an autograd function, a training step):
 *   y_t = h_t C_t + D_h x_t,  h_t = exp(dt_t A_h) h_{t-1} + dt_t x_t (outer) B_t
 * with h entering each sequence as its initial state (zeros when
 * initial_states is NULL).  Output y (B, L, H, P) in the I/O dtype.
 * final_states (nseqs, H, P, N) fp32, optional: the state after each
 * sequence's last position (sequences numbered as for ssd_bwd).
 * Required: x, dt, A, B, C, y, workspace.  Optional: D (zeros),
 * initial_states, seq_idx, final_states.  nseqs must be right whenever
 * initial_states or final_states is given (same clamping as ssd_bwd).
 * The workspace is sized by ssd_bwd_workspace_size; its contents on entry do
 * not matter.  Asynchronous on `stream`; deterministic like ssd_bwd.
 * Returns SSD_OK or a negative status.
 */
int ssd_fwd(const ssd_shape* shape, const void* x, const float* dt, const float* A,
            const void* B, const void* C, const float* D, const float* initial_states,
            const int32_t* seq_idx, void* y, float* final_states,
            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Optional dt front-end of the layer, applied per (position, head) before the
 * recurrence: with u = dt[b, t, h] + dt_bias[h] (dt_bias NULL: no bias),
 *   v      = softplus(u) = ln(1 + e^u) for u <= 20, u above   (dt_softplus != 0)
 *          = u                                               (dt_softplus == 0)
 *   dt_eff = min(max(v, dt_min), dt_max)
 * and dt_eff takes the place of dt in the recurrence stated above.  Pass
 * dt_min = -INFINITY, dt_max = INFINITY for no clamp; dt_min <= dt_max, no NaN.
 * The page "Deterministic bwd kernel for mamba2" times chunk_cumsum_bwd (its
 * "Per-kernel breakdown" tables), the step's own backward, but no page states
 * the activation; this is the usual parameterisation of the step in Mamba-2
 * layers, and the synthetic workloads draw dt through it.
 * Its gradient: d dt_eff / du = [dt_min <= v <= dt_max] * (dt_softplus ?
 * sigmoid(u), or 1 for u > 20 : 1).
 */
typedef struct {
  const float* dt_bias;  /* (nheads) fp32 device pointer, or NULL */
  int32_t dt_softplus;   /* nonzero: softplus after the bias */
  float dt_min, dt_max;  /* clamp of the activated value */
  int32_t d_per_channel; /* nonzero: D and dD are (nheads, headdim): y += D[h, p] x[.., h, p] */
  /* (batch, nheads, headdim, dstate) fp32 device pointer, or NULL; read by ssd_bwd_ex only:
   * the gradient arriving for the state after position seqlen-1 of each batch row (the final
   * state of the row's last sequence).  The loss becomes l + sum_b <d_last_states[b], h_{L-1}>. */
  const float* d_last_states;
  /* (batch, seqlen, nheads, headdim) in the I/O dtype, or NULL; used only with an output
   * gate z.  ssd_fwd_ex writes y before the gate there (the value it multiplies by silu(z),
   * rounded to the I/O dtype); ssd_bwd_ex reads it back instead of recomputing y, so that its
   * gate pass is one elementwise pass over dy, z and this array.  The results are the same
   * bits either way.  It may alias none of the other arrays of the call. */
  void* y_pre_gate;
} ssd_options;

/*
 * ssd_fwd and ssd_bwd extended with the options above (`opt` NULL: none of
 * them) and an output gate (`z` NULL: none).  With a dt front-end, `dt` is
 * the raw input and `ddt` the gradient with respect to it; `ddt_bias`
 * (nheads, fp32, nullable; requires opt->dt_bias) receives the gradient with
 * respect to dt_bias, summed over batch and positions in a fixed order.
 * With d_per_channel, D (nullable) and dD are (nheads, headdim) fp32, dD
 * summed over batch and positions in a fixed order.
 *
 * The gate z (batch, seqlen, nheads, headdim) in the I/O dtype multiplies
 * the layer's output by silu(z) = z sigmoid(z):  out = y * silu(z), y as
 * above (D term included).  ssd_bwd_ex then takes `dy` as the gradient of
 * `out` and writes `dz` (same shape and dtype as z; required with z):
 *   dz = dy * y * sigmoid(z) (1 + z (1 - sigmoid(z))),
 * and the gradients of everything else through dy * silu(z).  y is
 * recomputed from the inputs, or read from opt->y_pre_gate when the forward
 * saved it there.  The gated dy is held, rounded to the I/O dtype, in the dx
 * buffer until dx overwrites it.
 *
 * The gate is not on the pages either: it is the output gate of the usual
 * Mamba-2 layer, which sits around the scan as the dt front-end does.
 *
 * d_last_states is what a split of the sequence axis needs (a stretch of a
 * sequence on one device, the rest on the next): the later stretch starts
 * from this stretch's last states (initial_states) and hands back their
 * gradient (its d_initial_states), which enters here; chained that way the
 * stretches' gradients are those of the whole sequence.  No page describes
 * the hand-off; it follows from the recurrence above (the adjoint of the
 * state after the stretch's last position).
 * Everything else is as for ssd_fwd / ssd_bwd, including the workspace size.
 */
int ssd_fwd_ex(const ssd_shape* shape, const ssd_options* opt, const void* x, const float* dt,
               const float* A, const void* B, const void* C, const float* D, const void* z,
               const float* initial_states, const int32_t* seq_idx, void* y, float* final_states,
               void* workspace, size_t workspace_bytes, void* stream);
int ssd_bwd_ex(const ssd_shape* shape, const ssd_options* opt, const void* x, const float* dt,
               const float* A, const void* B, const void* C, const float* D, const void* z, const void* dy,
               const float* initial_states, const int32_t* seq_idx,
               void* dx, float* ddt, float* dA, void* dB, void* dC, float* dD,
               float* d_initial_states, float* ddt_bias, void* dz, void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * ssd_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and the same output bytes as ssd_bwd, with no workspace
 * argument.  Its workspace is a fixed array of SSD_NOALLOC_SCRATCH_BYTES
 * (64 MiB) in the library's device memory: one copy per GPU, whose address is
 * looked up on the first call on that device and which that GPU holds until
 * the process ends.  The call makes no hipMalloc/hipFree and no other
 * allocating call.
 *   - Shapes whose ssd_bwd_workspace_size exceeds SSD_NOALLOC_SCRATCH_BYTES
 *     are rejected with SSD_ERR_WORKSPACE_TOO_SMALL before anything is
 *     enqueued (the 2048-token, 128-head, dstate-128 layer needs 61 MiB).
 *   - Every call on one GPU shares that GPU's array and leaves its values in
 *     it; the next call's results do not depend on them.  Calls that overlap
 *     on one GPU (two streams, two host threads) race on the array: the
 *     caller serialises them.
 * Arguments, layouts and return codes are those of ssd_bwd.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ssd_bwd_noalloc(const ssd_shape* shape, const void* x, const float* dt, const float* A,
                    const void* B, const void* C, const float* D, const void* dy,
                    const float* initial_states, const int32_t* seq_idx,
                    void* dx, float* ddt, float* dA, void* dB, void* dC, float* dD,
                    float* d_initial_states, void* stream);

/* Static description of a status code (never NULL). */
const char* ssd_status_string(int status);

/*
 * Workspace regions, for inspecting intermediate results after a call
 * (tests, profiling).  Offsets are in bytes from the workspace start.
 *   SSD_WS_ACS    float32 (batch, nheads, nchunks, Q): in-chunk inclusive cumsum of
 *                 dt*A, restarted at chunk and sequence starts
 *   SSD_WS_HIN    I/O dtype (batch, nheads, nchunks, P, N): state entering each chunk
 *   SSD_WS_DSTATE I/O dtype (batch, nheads, nchunks, P, N): gradient w.r.t. the state at
 *                 the end of each chunk, through later positions only
 *                 (both are carried in fp32 and rounded once when stored)
 * Returns SSD_OK and fills offset/bytes, or a negative status.
 */
enum { SSD_WS_ACS = 0, SSD_WS_HIN = 1, SSD_WS_DSTATE = 2 };
int ssd_bwd_workspace_region(const ssd_shape* shape, int region, size_t* offset, size_t* bytes);

/*
 * Profiling twin of ssd_bwd: the same computation, plus a hipEvent_t recorded
 * on `stream` before the first stage and after every stage, so that a caller
 * can time the stages (kernels) of the backward inside its own timed region
 * without synchronising.  `events` points to ssd_bwd_stage_count() + 1
 * hipEvent_t handles, created (with timing enabled) and owned by the caller;
 * none may be NULL.  Stage i runs between events[i] and events[i + 1].
 */
int ssd_bwd_profiled(const ssd_shape* shape, const void* x, const float* dt, const float* A,
                     const void* B, const void* C, const float* D, const void* dy,
                     const float* initial_states, const int32_t* seq_idx,
                     void* dx, float* ddt, float* dA, void* dB, void* dC, float* dD,
                     float* d_initial_states, void* workspace, size_t workspace_bytes,
                     void* stream, void* const* events);

/* Number of stages of the backward and the name of stage i ("prep",
 * "state_fwd", "state_bwd", "dcb", "dbdc", "head_bwd", "reduce"); NULL for
 * an index out of range. */
int ssd_bwd_stage_count(void);
const char* ssd_bwd_stage_name(int stage);

/*
 * Launch geometry that the problem shape does not fix by itself, for tests of
 * the determinism contract.  The page "Deterministic bwd kernel for mamba2"
 * (its "Autotuner / kernel-shape non-determinism" section) reports results
 * that changed with the kernels' block shape; here no result depends on the
 * launch geometry, and this hook lets a test show it:
 *   head_blocks          persistent blocks of the backward's per-head kernel
 *                        (0: the default, 256, capped by the number of
 *                        (batch, head, chunk) items)
 *   fwd_heads_per_block  heads of one group handled by one block of the
 *                        forward's output kernel (0: the default, chosen from
 *                        the shape alone; capped by the heads per group)
 * Process-wide; takes effect for calls made after it returns.  Outputs are
 * byte-identical for every setting.  Returns SSD_OK, or SSD_ERR_INVALID_ARG
 * for a negative value.
 */
int ssd_set_launch_geometry(int head_blocks, int fwd_heads_per_block);

/*
 * Which of the two implementations of the group stage (the head-summed dCB
 * and dC, dB; stages "dcb" and "dbdc") the calls made after this one use,
 * for tests that cover both:
 *   0  by shape (the default): split kernels when their grid has at least
 *      256 blocks, else the fused slab kernel, which has Q / 64 times more
 *   1  fused: per (batch, group, chunk, 64-row slab, dstate tile), dCB, dC
 *      and dB in one pass over the group's heads
 *   2  split: dCB per (batch, group, chunk), then dC and dB per (batch,
 *      group, chunk, dstate tile)
 * Both sum the same terms in fixed orders, so each is deterministic; they
 * add in different orders, so they agree to rounding, not bit for bit.
 * The choice also changes the workspace size.  Process-wide.  Returns
 * SSD_OK, or SSD_ERR_INVALID_ARG for another value.
 */
int ssd_set_group_path(int path);

/* Library version, (major << 16) | minor. */
int ssd_bwd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_BWD_H */
