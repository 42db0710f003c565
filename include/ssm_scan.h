/*
 * ssm_scan.h -- C ABI of libssmscan.so, the MI355X (gfx950) Mamba S6 selective scan.
 *
 * Source of the operation: the rustytorch commit log, page
 * "crates/training/rtx-transformers/tests":
 *   - the commit replacing the MambaBlock stub with a real S6 forward defines
 *       delta = softplus(dt + dt_bias), A = -exp(A_log),
 *       h_t = exp(delta*A) (.) h_{t-1} + delta*B_t*x_t,
 *       y_t = (sum_n C_t[n]*h_t[n] + D*x_t) * silu(z_t),
 *     with B_t, C_t emitted per token by x_proj (2*d_state values per token,
 *     shared by every channel);
 *   - the commit adding the hand-written VJP defines the backward as the
 *     reverse-time recurrence over the state trajectory, covering A_log through
 *     dA_log = dA*A, dt_bias and D, with parameter gradients summed over batch;
 *   - the commit introducing MambaRecurrence::step defines the single-token
 *     update of a carried state, which must reproduce the full forward;
 *   - the commit adding the CUDA backward records the failure modes this ABI
 *     is shaped against: host round trips of device tensors and silently
 *     ignored strides.  Hence: device pointers only, dense row-major layouts,
 *     no host copies, no synchronisation.
 * The discretised input term is read as delta*B_t*x_t (Euler form).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers on the current HIP device, dense,
 *     row-major (last index fastest), 16-byte aligned.  The caller owns every
 *     buffer, including workspace and checkpoints, sized by the query functions.
 *     The library allocates, frees and copies nothing, keeps no global state
 *     (re-entrant), never synchronises, and orders all work on `stream`.
 *   - Layouts (Bt = batch, L = seqlen, D = d_inner, N = d_state):
 *       x, z, dt, y, dy, dx, dz, ddt : [Bt, L, D]    io dtype
 *       B, C, dB, dC                 : [Bt, L, N]    io dtype
 *       A_log, dA_log                : [D, N]        f32
 *       D, dt_bias, dD, ddt_bias     : [D]           f32
 *       h0, h_last, dh0, step state  : [Bt, D, N]    f32
 *   - io dtype SSM_BF16: activations and activation gradients are bf16
 *     (round-to-nearest-even on store); parameters, their gradients and states
 *     are f32; all arithmetic is f32.
 *   - Nullable inputs: z (no gate: y = C.h + D*x), D (treated as 0),
 *     dt_bias (0), h0 (zero initial state).
 *   - Errors: arguments are validated on the host before anything is launched;
 *     a non-OK status means nothing was enqueued, except SSM_E_LAUNCH, which
 *     reports a failed launch (earlier launches of the same call may have been
 *     enqueued).  Faults inside kernels surface at the caller's next
 *     synchronisation.  The entry points never abort.  Pending HIP errors of
 *     the calling thread are cleared on entry.
 *   - NaN inputs propagate to the outputs; nothing is masked.
 *   - d_state must be 16 (others: SSM_E_UNSUPPORTED); batch <= 65535.
 *   - seqlen may be 0: the forward writes h_last = h0 (or 0) and the backward
 *     writes zero parameter gradients and dh0 = 0; activation pointers may
 *     then be NULL.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSM_OK = 0,
    SSM_E_NULLPTR = 1,     /* a required pointer is NULL */
    SSM_E_SHAPE = 2,       /* a dimension is out of range */
    SSM_E_DTYPE = 3,       /* unknown io dtype */
    SSM_E_ALIGN = 4,       /* a pointer is not 16-byte aligned */
    SSM_E_WORKSPACE = 5,   /* workspace smaller than the query function returns */
    SSM_E_LAUNCH = 6,      /* a kernel launch failed (hipGetLastError) */
    SSM_E_UNSUPPORTED = 7  /* valid but outside the limits a header states (d_state != 16, ...) */
} ssm_status;

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

typedef struct {
    int64_t batch;
    int64_t seqlen;
    int64_t d_inner;
    int64_t d_state;
    int32_t io_dtype; /* ssm_dtype */
} ssm_dims;

#define SSM_TIMING_MAX 64

/* Optional launch log.  When a non-NULL ssm_timing* is passed, the library
 * records events[2*i] before and events[2*i+1] after its i-th kernel launch
 * (ssm_block.h: also each hipBLASLt GEMM) on `stream` (for i < capacity <=
 * SSM_TIMING_MAX) and writes the kernel's id into kernel_id[i]; `count` is
 * incremented per recorded launch (the caller zeroes it); launches past the
 * capacity are not recorded.  The caller creates the events (hipEventCreate)
 * and reads them after synchronising.  Used for per-kernel timing; NULL costs
 * nothing. */
typedef struct {
    hipEvent_t *events;
    int32_t capacity;
    int32_t count;
    int32_t kernel_id[SSM_TIMING_MAX];
} ssm_timing;

/* Kernel ids reported in ssm_timing.kernel_id. */
enum {
    SSM_K_FWD_CHUNK = 1,     /* per-chunk zero-start end state and delta sum */
    SSM_K_FWD_CARRY = 2,     /* sequential combine of chunk states -> chunk start states */
    SSM_K_FWD_MAIN = 3,      /* recurrence from chunk start, writes y, checkpoints, h_last */
    SSM_K_BWD_CHUNK = 4,     /* per-chunk zero-end adjoint and delta sum */
    SSM_K_BWD_CARRY = 5,     /* reverse combine -> adjoint entering each chunk */
    SSM_K_BWD_MAIN = 6,      /* recompute + reverse adjoint sweep, per-element grads, partials */
    SSM_K_BWD_REDUCE_BC = 7, /* fixed-order sum of dB/dC partials over channel blocks */
    SSM_K_BWD_REDUCE_P = 8,  /* fixed-order sum of dA_log/dD/ddt_bias partials */
    SSM_K_STEP = 9,          /* single-token state update */
    SSM_K_FILL = 10,         /* small fills for seqlen == 0 */
    SSM_K_CONV_FWD = 11,     /* causal depthwise conv1d + SiLU (ssm_conv1d.h) */
    SSM_K_CONV_BWD = 12,     /* its adjoint: dx, ring gradient, dw/dbias partials */
    SSM_K_CONV_BWD_REDUCE = 13, /* fixed-order sum of dw/dbias partials */
    SSM_K_CONV_STEP = 14,    /* one token through the conv ring */
    SSM_K_CONV_RING = 15,    /* ring copies/fills when seqlen == 0 */
    SSM_K_BLOCK_BC = 16,     /* x_proj's B/C columns split / joined (ssm_block.h) */
    SSM_K_GDN2_FWD = 17,     /* Gated DeltaNet-2 forward recurrence (ssm_gdn2.h) */
    SSM_K_GDN2_WY = 18,      /* GDN2 chunked form: key side per chunk (decays, A, P, M^-1) */
    SSM_K_GDN2_STATE = 19,   /* GDN2 chunked form: state pass over the chunks (MFMA) */
    SSM_K_BLOCK_GEMM = 20,   /* one projection GEMM of the block (hipBLASLt; ssm_block.h) */
    SSM_K_BLOCK_SUM = 21,    /* fixed-order sum of a split weight gradient's partials */
    SSM_K_FWD_STATE = 22     /* forward in one pass, one lane per (channel, state): y, checkpoints, h_last */
};

/* Name of a kernel id (for matching profiler output); "?" if unknown. */
const char *ssm_kernel_name(int32_t kernel_id);

/* Human-readable text of a status code (an ssm_status value, taken as a plain
 * 32-bit integer so that any code, known or not, is a valid argument); "unknown
 * status" for codes outside the enum.  Never NULL. */
const char *ssm_status_str(int32_t status);

/* Bytes of the checkpoint buffer a training forward writes and the backward
 * reads (f32 states at a fixed token stride; the layout is private to the
 * library).  0 for invalid dims. */
size_t ssm_scan_ckpt_bytes(const ssm_dims *dims);

/* Workspace bytes ssm_scan_fwd / ssm_scan_bwd need for these dims (may be 0).
 * 0 for invalid dims. */
size_t ssm_scan_fwd_workspace_bytes(const ssm_dims *dims);
size_t ssm_scan_bwd_workspace_bytes(const ssm_dims *dims);

/* Forward selective scan (commit replacing the MambaBlock stub: the S6
 * recurrence and gated readout above).
 *   x, dt, B, C, z : inputs in io dtype (z nullable)
 *   A_log, D, dt_bias : f32 parameters (D, dt_bias nullable)
 *   h0     : [Bt, D, N] f32 initial state or NULL (zero)
 *   y      : [Bt, L, D] output, io dtype (required when seqlen > 0)
 *   h_last : [Bt, D, N] f32 final state, or NULL
 *   ckpt   : ssm_scan_ckpt_bytes() bytes for a later ssm_scan_bwd, or NULL
 *            (inference)
 *   ws     : ssm_scan_fwd_workspace_bytes() bytes (may be NULL when that is 0)
 *   timing : optional launch log, or NULL */
ssm_status ssm_scan_fwd(const ssm_dims *dims, const void *x, const void *dt, const void *B,
                        const void *C, const void *z, const float *A_log, const float *D,
                        const float *dt_bias, const float *h0, void *y, float *h_last,
                        float *ckpt, void *ws, size_t ws_bytes, hipStream_t stream,
                        ssm_timing *timing);

/* Backward: the reverse-time adjoint of ssm_scan_fwd for L = sum(dy * y)
 * (commit adding the hand-written VJP).  Needs the ckpt written by
 * ssm_scan_fwd with the same dims and inputs.
 *   h0                      : NOT READ.  The initial state reaches the backward
 *                             through ckpt, whose first entry ssm_scan_fwd wrote
 *                             from the h0 it was given; the argument exists so
 *                             that both calls take the same list, and may be
 *                             NULL.  A different h0 here changes nothing: to
 *                             differentiate at another initial state, rerun
 *                             ssm_scan_fwd with it.
 *   dy                      : [Bt, L, D] upstream gradient, io dtype
 *   dx, ddt, dz             : [Bt, L, D] io dtype; ddt is w.r.t. the raw dt input
 *                             (d delta * sigmoid(dt + dt_bias)); dz required iff z
 *   dB, dC                  : [Bt, L, N] io dtype, summed over channels
 *   dA_log, dD, ddt_bias    : f32, summed over batch and time, OVERWRITTEN
 *                             (dA_log = dA * A)
 *   dh0                     : [Bt, D, N] f32 gradient of h0, or NULL
 *   ws                      : ssm_scan_bwd_workspace_bytes() bytes */
ssm_status ssm_scan_bwd(const ssm_dims *dims, const void *x, const void *dt, const void *B,
                        const void *C, const void *z, const float *A_log, const float *D,
                        const float *dt_bias, const float *h0, const float *ckpt,
                        const void *dy, void *dx, void *ddt, void *dB, void *dC, void *dz,
                        float *dA_log, float *dD, float *ddt_bias, float *dh0, void *ws,
                        size_t ws_bytes, hipStream_t stream, ssm_timing *timing);

/* Single-token step (commit introducing MambaRecurrence::step): the forward's
 * per-token body applied to a caller-held state, updated in place.  Stepping
 * token by token from a zero state equals ssm_scan_fwd bit for bit (states and
 * y) whenever the forward runs its sequence as one chunk with one lane per
 * channel: when batch*d_inner >= 262144, or seqlen < 128 and d_inner is not a
 * multiple of 16.  Where the forward runs one lane per state instead
 * (batch*d_inner < 262144, d_inner a multiple of 16, and batch*d_inner >= 8192
 * or seqlen <= 512) the states still agree bit for bit and y to rounding: its
 * readout sums the 16 states in another order.
 *   h          : [batch, d_inner, N] f32, read and overwritten
 *   x, dt, z   : [batch, d_inner] io dtype (z nullable)
 *   B, C       : [batch, N] io dtype
 *   y          : [batch, d_inner] io dtype */
ssm_status ssm_scan_step(int64_t batch, int64_t d_inner, int64_t d_state, int32_t io_dtype,
                         float *h, const void *x, const void *dt, const void *B, const void *C,
                         const void *z, const float *A_log, const float *D,
                         const float *dt_bias, void *y, hipStream_t stream, ssm_timing *timing);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
