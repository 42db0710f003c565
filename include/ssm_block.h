/*
 * ssm_block.h -- C ABI of libssmblock.so: one Mamba block around the selective
 * scan on one MI355X (gfx950), forward and backward.
 *
 * Source of the operation: the rustytorch commit log, page
 * "crates/training/rtx-transformers/tests":
 *   - the commit replacing the MambaBlock stub defines the block; written as
 *     equations over tokens (rows) of X [T, d_model]:
 *         [u | z]        = X W_in^T                  (two d_inner halves)
 *         v              = silu(conv1d_causal(u; conv_w) + conv_b)
 *         [r | B | C]    = v W_x^T                   (dt_rank, d_state, d_state)
 *         delta          = softplus(r W_dt^T + dt_bias)
 *         y              = scan(v, delta, B, C; A_log, D) * silu(z)
 *         Y              = y W_out^T                 (residual added by the caller);
 *   - the hand-written VJP commit returns gradients for in_proj, conv1d_weight,
 *     conv1d_bias, A_log, x_proj, dt_proj, dt_bias, D and out_proj, summed over
 *     the batch;
 *   - the CUDA backward commit sends the four projections (forward and their
 *     gradient GEMMs) to a vendor BLAS and leaves the rest on the host; here the
 *     projections run on hipBLASLt and the conv and the scan on this project's
 *     kernels (ssm_conv1d.h, ssm_scan.h), all on the caller's stream.
 * Readings: projections are bias-free, y = x W^T with [out, in] weights; in_proj's
 * first d_inner outputs feed the conv, the next d_inner are the gate z; x_proj's
 * outputs are (dt_low [dt_rank], B [d_state], C [d_state]); dt_proj's bias is
 * dt_bias inside the softplus.
 *
 * Conventions (as in ssm_scan.h): DEVICE pointers, dense row-major, 16-byte
 * aligned, caller-owned; arguments are checked on the host before any launch;
 * work is ordered on `stream`.  Exceptions to "allocates nothing": the context
 * owns a hipBLASLt handle (created by ssm_block_create), and hipBLASLt manages
 * that handle's own device memory; the context also keeps, per GEMM shape seen,
 * the descriptors and the algorithm the library's heuristic chose (host memory).
 * A context may be used by one thread at a time.
 *   - Layouts (T = batch*seqlen tokens, dm = d_model, di = d_inner, N = d_state,
 *     R = dt_rank, K = d_conv, P = R + 2N):
 *       X, Y, dX, dY        : [batch, seqlen, dm]   io dtype
 *       W_in                : [2 di, dm]            io dtype
 *       W_x                 : [P, di]               io dtype
 *       W_dt                : [di, R]               io dtype
 *       W_out               : [dm, di]              io dtype
 *       conv_w / conv_b     : [di, K] / [di]        f32
 *       dt_bias, D / A_log  : [di] / [di, N]        f32
 *       every gradient of a weight or parameter: the same shape, f32,
 *       OVERWRITTEN with the sum over batch and time.
 *   - io dtype SSM_BF16: activations, their gradients and the four projection
 *     weights are bf16; GEMMs accumulate in f32; everything else as in the scan.
 *   - Limits: d_state 16, 1 <= d_conv <= 4, dt_rank >= 1, d_model and d_inner
 *     multiples of 8, T < 2^31, batch <= 65535.
 */
#ifndef SSM_BLOCK_H
#define SSM_BLOCK_H

#include "ssm_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ssm_block_ctx ssm_block_ctx;

typedef struct {
    int64_t batch;
    int64_t seqlen;
    int64_t d_model;
    int64_t d_inner;
    int64_t d_state;
    int64_t dt_rank;
    int64_t d_conv;
    int32_t io_dtype; /* ssm_dtype */
} ssm_block_dims;

typedef struct {
    const void *W_in;      /* [2 d_inner, d_model] io dtype */
    const float *conv_w;   /* [d_inner, d_conv] */
    const float *conv_b;   /* [d_inner] or NULL */
    const void *W_x;       /* [dt_rank + 2 d_state, d_inner] io dtype */
    const void *W_dt;      /* [d_inner, dt_rank] io dtype */
    const float *dt_bias;  /* [d_inner] */
    const float *A_log;    /* [d_inner, d_state] */
    const float *D;        /* [d_inner] */
    const void *W_out;     /* [d_model, d_inner] io dtype */
} ssm_block_params;

typedef struct { /* all f32, overwritten */
    float *dW_in, *dconv_w, *dconv_b, *dW_x, *dW_dt, *ddt_bias, *dA_log, *dD, *dW_out;
} ssm_block_grads;

/* Creates a context on the current HIP device (one hipBLASLt handle).  Returns
 * SSM_E_LAUNCH if the handle cannot be created. */
ssm_status ssm_block_create(ssm_block_ctx **ctx);
void ssm_block_destroy(ssm_block_ctx *ctx);

/* Bytes of the activations a training forward keeps for the backward, and of
 * the per-call workspaces; 0 for invalid dims.  Every workspace starts with
 * 64 MiB for the projections' GEMMs.  ssm_block_fwd_workspace_bytes is what an
 * inference call (saved == NULL) needs; a training call uses only the leading
 * ssm_block_fwd_training_workspace_bytes of it (the GEMMs' part and the scan's
 * workspace) and accepts a buffer of that size. */
size_t ssm_block_saved_bytes(const ssm_block_dims *dims);
size_t ssm_block_fwd_workspace_bytes(const ssm_block_dims *dims);
size_t ssm_block_fwd_training_workspace_bytes(const ssm_block_dims *dims);
size_t ssm_block_bwd_workspace_bytes(const ssm_block_dims *dims);

/* Forward: Y = block(X).  `saved` (ssm_block_saved_bytes, nullable for
 * inference) receives the activations ssm_block_bwd needs. */
ssm_status ssm_block_fwd(ssm_block_ctx *ctx, const ssm_block_dims *dims, const void *X,
                         const ssm_block_params *p, void *Y, void *saved, void *ws, size_t ws_bytes,
                         hipStream_t stream, ssm_timing *timing);

/* Backward of ssm_block_fwd for the loss sum(dY * Y), from the forward's
 * `saved` buffer: writes dX and every gradient in `g`. */
ssm_status ssm_block_bwd(ssm_block_ctx *ctx, const ssm_block_dims *dims, const void *X,
                         const ssm_block_params *p, const void *saved, const void *dY, void *dX,
                         const ssm_block_grads *g, void *ws, size_t ws_bytes, hipStream_t stream,
                         ssm_timing *timing);

#ifdef __cplusplus
}
#endif

#endif /* SSM_BLOCK_H */
