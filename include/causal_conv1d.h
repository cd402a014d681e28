/*
 * causal_conv1d.h -- C ABI (in libssd_bwd.so) of the depthwise causal
 * convolution of the Mamba-2 block and its deterministic backward, on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation.  The page "Deterministic bwd kernel for mamba2"
 * (state-spaces/mamba PR 827, section "Atomic add non-determinism") names
 * causal-conv1d's backward, next to the SSD kernels, as a source of
 * run-to-run differences, because it sums the filter gradient with atomics.
 * The page does not write the operation out; it is the short convolution of
 * the Mamba-2 block, applied per channel c of a channels-last input before
 * the SSD:
 *
 *     pre[b,t,c] = bias[c] + sum_{k<W} w[c,k] * x[b, t-(W-1)+k, c] * m(t, t-(W-1)+k)
 *     out[b,t,c] = pre[b,t,c]                        (CONV1D_ACT_NONE)
 *                = pre[b,t,c] * sigmoid(pre[b,t,c])  (CONV1D_ACT_SILU)
 *
 * with m(t, s) = 1 when s >= 0 and rows s and t are in the same sequence,
 * else 0.  As for ssd_bwd, a sequence starts at row r when r == 0 or
 * seq_idx[b, r] != seq_idx[b, r-1], so rows s <= t share a sequence when no
 * sequence starts in (s, t]; with seq_idx NULL every row is one sequence.  conv1d_bwd returns the gradients of l = sum dout * out:
 * dx (like x), dweight (like w) and dbias (like bias), recomputing pre from
 * x; nothing from the forward is needed.
 *
 * Determinism.  Every dx element has one writer.  dweight and dbias are sums
 * over all (b, t): each block forms its partial over its rows in a fixed
 * order into its own workspace slot, and a second kernel adds the slots in
 * slot order in double precision.  No floating-point atomics; the output
 * bytes depend only on the inputs, the shape and the library build.
 *
 * Layouts (row-major, contiguous):
 *   x, out, dout, dx   (batch, seqlen, channels)   io dtype (ssd_io_dtype)
 *   weight, dweight    (channels, width)           float32
 *   bias, dbias        (channels)                  float32
 *   seq_idx            (batch, seqlen)             int32
 *
 * Ownership and calling convention: as for ssd_bwd.  Device pointers owned
 * by the caller, x/out/dout/dx 16-byte aligned; outputs fully overwritten;
 * the library never allocates; work is only enqueued on `stream`
 * (hipStream_t, NULL = default stream); argument errors are returned before
 * anything is enqueued, as the SSD_* status codes of ssd_bwd.h.
 */
#ifndef CAUSAL_CONV1D_H
#define CAUSAL_CONV1D_H

#include <stddef.h>
#include <stdint.h>

#include "ssd_bwd.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { CONV1D_ACT_NONE = 0, CONV1D_ACT_SILU = 1 };

typedef struct {
  int64_t batch;      /* >= 1 */
  int64_t seqlen;     /* >= 1 */
  int64_t channels;   /* >= 1, multiple of 8 (bf16 io) or 4 (f32 io) */
  int32_t width;      /* W: 2, 3 or 4 */
  int32_t activation; /* CONV1D_ACT_NONE or CONV1D_ACT_SILU */
  int32_t io_dtype;   /* SSD_IO_BF16 or SSD_IO_F32 */
  int32_t reserved;   /* must be 0 */
} conv1d_shape;

/*
 * out = act(pre) as above.  bias and seq_idx may be NULL (no bias; one
 * sequence per batch row).  Returns SSD_OK or a negative status.
 */
int conv1d_fwd(const conv1d_shape* shape, const void* x, const float* weight, const float* bias,
               const int32_t* seq_idx, void* out, void* stream);

/* Workspace bytes conv1d_bwd needs for `shape` (the per-block partials of dweight and dbias). */
int conv1d_bwd_workspace_size(const conv1d_shape* shape, size_t* bytes);

/*
 * dx, dweight, dbias of l = sum dout * out.  bias and seq_idx may be NULL;
 * dbias may be NULL (not computed).  dx must not alias x or dout.  The
 * workspace's contents on entry do not matter.  Returns SSD_OK or a negative
 * status.
 */
int conv1d_bwd(const conv1d_shape* shape, const void* x, const float* weight, const float* bias,
               const int32_t* seq_idx, const void* dout, void* dx, float* dweight, float* dbias,
               void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CAUSAL_CONV1D_H */
