/*
 * ssm_gdn2.h -- C ABI (in libssmscan.so) of the Gated DeltaNet-2 forward on one
 * MI355X (gfx950): a gated delta rule with a decay per key dimension and
 * separate erase and write gates.
 *
 * Source of the operation: burn-gdn2 0.1.4, page "src/forward.rs": the chunked
 * WY forward and its check against a sequential reference.  The page prints the
 * chunk form only; the per-token recurrence that this form regroups exactly
 * (with the decays kept per key dimension) is, for a [K, V] state S,
 *     S'   = diag(exp(g_t)) S_{t-1}
 *     vn_t = w_t * v_t - S'^T (b_t * k_t)
 *     S_t  = S' + k_t vn_t^T
 *     o_t  = scale * S_t^T q_t
 * and that recurrence is what this call computes (the page's average of the
 * decays over the key dimension, an approximation, is not reproduced).
 *
 * Conventions (as in ssm_scan.h): DEVICE pointers, dense row-major, 16-byte
 * aligned, caller-owned; arguments are checked on the host before any launch;
 * work is ordered on `stream`; nothing is allocated.
 *   - q, k, g, b : [batch, heads, seqlen, k_dim] io dtype (g: log-decays, normally <= 0)
 *   - v, w, o    : [batch, heads, seqlen, v_dim] io dtype
 *   - io dtype SSM_F32, or SSM_BF16 (values read as bf16, arithmetic and state in
 *     f32, o rounded to nearest even)
 *   - S0, S_last : [batch, heads, k_dim, v_dim] f32; S0 NULL = zero state;
 *                  S_last NULL = not written; S_last may not alias S0.
 *   - Limits: k_dim in {16, 32, 64, 128}; batch, heads <= 65535.  seqlen 0 writes
 *     S_last = S0 (zeros when S0 is NULL).
 */
#ifndef SSM_GDN2_H
#define SSM_GDN2_H

#include "ssm_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int64_t batch;
    int64_t heads;
    int64_t seqlen;
    int64_t k_dim;
    int64_t v_dim;
    int32_t io_dtype; /* ssm_dtype */
} ssm_gdn2_dims;

/* Forward over the whole sequence from S0: writes o and, if non-NULL, S_last.
 * Chaining calls through S_last -> S0 reproduces one call over the joined
 * sequence bit for bit. */
ssm_status ssm_gdn2_fwd(const ssm_gdn2_dims *dims, const void *q, const void *k, const void *v,
                        const void *g, const void *b, const void *w, const float *S0, float scale,
                        void *o, float *S_last, hipStream_t stream, ssm_timing *timing);

/* The same forward in chunks of 64 tokens: the WY form of the page's chunked
 * forward with the decays kept per key dimension, its products on MFMA
 * (v_mfma_f32_16x16x4f32, f32).  Per chunk, with G the inclusive cumulative sum
 * of g inside the chunk:
 *     A[i][j] = sum_k b_i k_i k_j exp(G_i - G_j)  (j < i),  M = I + A
 *     P[i][j] = sum_k q_i k_j exp(G_i - G_j)      (j <= i)
 *     vn = M^{-1} (w*v - (b*k*exp(G)) S),  o = scale (P vn + (q*exp(G)) S)
 *     S  = diag(exp(G_last)) S + (k*exp(G_last - G))^T vn
 * Every exp(G_i - G_j) has i >= j (<= 1 for g <= 0) and is formed either per
 * element (inside a 16-token block) or as exp(G_i - E) * exp(E - G_j) with E
 * the G at the end of j's block (both factors <= 1), so strongly gated heads
 * cannot overflow it.  Equal to ssm_gdn2_fwd up to f32
 * rounding (not bit for bit).  Chaining calls through S_last -> S0 reproduces
 * one call over the joined sequence bit for bit when every call but the last
 * has a multiple of 64 tokens (the chunk grouping is then the same).
 *   - Same arguments and layouts as ssm_gdn2_fwd, plus a caller-owned
 *     workspace of ssm_gdn2_chunked_workspace_bytes(dims) bytes (per pair and
 *     chunk: 192 k_dim + 8192 + k_dim floats, rounded up to 64), overwritten.
 *   - Limits: k_dim in {16, 32, 64, 128}, v_dim a multiple of 16
 *     (SSM_E_UNSUPPORTED otherwise; ssm_gdn2_fwd takes any v_dim);
 *     batch*heads and the chunk count at most 65535.
 *   - seqlen 0 writes S_last = S0 (zeros when S0 is NULL); ws may be NULL. */
size_t ssm_gdn2_chunked_workspace_bytes(const ssm_gdn2_dims *dims);
ssm_status ssm_gdn2_fwd_chunked(const ssm_gdn2_dims *dims, const void *q, const void *k,
                                const void *v, const void *g, const void *b, const void *w,
                                const float *S0, float scale, void *o, float *S_last, void *ws,
                                size_t ws_bytes, hipStream_t stream, ssm_timing *timing);

#ifdef __cplusplus
}
#endif

#endif /* SSM_GDN2_H */
