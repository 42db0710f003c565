/*
 * ssm_conv1d.h -- C ABI of the causal depthwise conv1d + SiLU in libssmscan.so
 * (MI355X, gfx950): the short convolution that feeds the selective scan.
 *
 * Source of the operation: the rustytorch commit log, page
 * "crates/training/rtx-transformers/tests":
 *   - the commit replacing the MambaBlock stub with a real S6 forward runs
 *     in_proj, then a causal depthwise conv1d, then SiLU, then x_proj and the scan;
 *   - the commit adding the hand-written VJP returns gradients for
 *     conv1d_weight and conv1d_bias (summed over the batch);
 *   - the commit introducing MambaRecurrence::step carries a conv ring next to
 *     the scan state, one token at a time.
 * The pages give neither the kernel width nor the tap order.  Read as PyTorch's
 * Conv1d(groups = d_inner, padding = d_conv - 1) truncated to the first seqlen
 * outputs, with the widths Mamba blocks use (d_conv <= 4):
 *
 *     pre[b,t,d] = bias[d] + sum_{k=0}^{K-1} w[d,k] * v[b, t-(K-1)+k, d]
 *     y[b,t,d]   = silu(pre[b,t,d]) = pre * sigmoid(pre)
 *
 * with v = x for times >= 0 and, for the K-1 times before the sequence, the
 * caller's ring (zero when no ring is passed).  The sum starts at the bias and
 * adds taps in increasing k in the forward and in the step, so stepping
 * reproduces the forward bit for bit.
 *
 * Conventions (as in ssm_scan.h): DEVICE pointers, dense row-major, 16-byte
 * aligned, caller-owned; nothing is allocated, copied to the host or
 * synchronised; work is ordered on `stream`; arguments are checked on the host
 * before any launch; optional ssm_timing logs each launch.
 *   - Layouts (Bt = batch, L = seqlen, D = d_inner, K = d_conv):
 *       x, y, dx, dy                  : [Bt, L, D]     io dtype (f32 or bf16)
 *       w, dw                         : [D, K]         f32 (PyTorch's [D, 1, K])
 *       bias, dbias                   : [D]            f32
 *       ring0, ring_last, dring0, ring: [Bt, D, K-1]   f32, oldest input first
 *   - bf16 outputs are rounded to nearest even; all arithmetic is f32.
 *   - Nullable: bias (0), ring0 (zero context), ring_last, dring0.  With K = 1
 *     the rings are empty and every ring pointer is ignored.
 *   - 1 <= d_conv <= 4 (larger: SSM_E_UNSUPPORTED); batch <= 65535.
 *   - seqlen may be 0: the forward copies ring0 (or zeros) to ring_last; the
 *     backward writes zero dw, dbias and dring0.
 */
#ifndef SSM_CONV1D_H
#define SSM_CONV1D_H

#include "ssm_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int64_t batch;
    int64_t seqlen;
    int64_t d_inner;
    int64_t d_conv;   /* kernel width K */
    int32_t io_dtype; /* ssm_dtype */
} ssm_conv_dims;

/* Bytes of workspace ssm_conv1d_bwd needs (per-tile dw/dbias partials); 0 for
 * invalid dims or seqlen 0. */
size_t ssm_conv1d_bwd_workspace_bytes(const ssm_conv_dims *dims);

/* Forward: y = silu(causal depthwise conv of x).  ring0 (nullable) supplies the
 * K-1 inputs before the sequence; ring_last (nullable) receives the last K-1
 * inputs of ring0 ++ x, i.e. the ring a following ssm_conv1d_step or forward
 * continues from.  ring_last must not alias ring0 or x. */
ssm_status ssm_conv1d_fwd(const ssm_conv_dims *dims, const void *x, const float *w,
                          const float *bias, const float *ring0, void *y, float *ring_last,
                          hipStream_t stream, ssm_timing *timing);

/* Backward of ssm_conv1d_fwd for the upstream gradient dy.  Writes dx; dw and
 * dbias are OVERWRITTEN with the sums over batch and time (fixed order:
 * bitwise deterministic); dring0 (nullable) receives the gradient w.r.t. ring0
 * (w.r.t. the zero context when ring0 is NULL).  bias may be NULL (then its
 * gradient is still written to dbias, which must not be NULL). */
ssm_status ssm_conv1d_bwd(const ssm_conv_dims *dims, const void *x, const float *w,
                          const float *bias, const float *ring0, const void *dy, void *dx,
                          float *dw, float *dbias, float *dring0, void *ws, size_t ws_bytes,
                          hipStream_t stream, ssm_timing *timing);

/* ssm_conv1d_bwd for callers that cannot allocate device memory: code under
 * HIP graph capture, allocation-free serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results (bit for bit) as
 * ssm_conv1d_bwd, except that its per-tile dw/dbias partials go to a static
 * device buffer of SSM_CONV1D_SCRATCH_BYTES that the library owns instead of a
 * caller workspace: it calls no hipMalloc, hipFree or allocating routine.
 *   - Limit: ssm_conv1d_bwd_workspace_bytes(dims) <= SSM_CONV1D_SCRATCH_BYTES
 *     (16 MiB; the batch 4 x 8192 x 5120, width 4 backward needs 13.1 MB), else
 *     SSM_E_WORKSPACE and nothing is launched.
 *   - The buffer lives on the device current on the calling thread when the
 *     call is made (which must be the stream's device); each GPU holds its own
 *     copy until the process ends.  Its address is looked up once per device
 *     (SSM_E_LAUNCH if that lookup fails).
 *   - Every call on a GPU shares that GPU's buffer and leaves its partials in
 *     it: calls that overlap on one GPU (streams not ordered with each other)
 *     race.  Order them on one stream or with events.  Nothing in the buffer
 *     needs to start at zero: each call writes every partial it reads. */
#define SSM_CONV1D_SCRATCH_BYTES ((size_t)16 << 20)
ssm_status ssm_conv1d_bwd_noalloc(const ssm_conv_dims *dims, const void *x, const float *w,
                                  const float *bias, const float *ring0, const void *dy, void *dx,
                                  float *dw, float *dbias, float *dring0, hipStream_t stream,
                                  ssm_timing *timing);

/* One token: y = silu(bias + sum_{k<K-1} w[k]*ring[k] + w[K-1]*x), then the ring
 * drops its oldest entry and appends x (in place).  x, y: [Bt, D] io dtype;
 * ring: [Bt, D, K-1] f32 (may be NULL when K = 1). */
ssm_status ssm_conv1d_step(int64_t batch, int64_t d_inner, int64_t d_conv, int32_t io_dtype,
                           float *ring, const void *x, const float *w, const float *bias,
                           void *y, hipStream_t stream, ssm_timing *timing);

#ifdef __cplusplus
}
#endif

#endif /* SSM_CONV1D_H */
