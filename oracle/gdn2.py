"""f64 CPU oracle of the Gated DeltaNet-2 forward (a gated delta rule with
per-key-dimension decay and separate erase and write gates).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it; it shares no code with the HIP
library.

Source: burn-gdn2 0.1.4, page "src/forward.rs", its chunked WY forward (per
chunk: inclusive cumulative sum of the log-decays g, a strictly lower
triangular key-key matrix weighted by b * k and the decays, a forward
substitution giving the WY factors of b * k * exp(G) and w * v, the corrected
values u - W S, the output as an intra-chunk term plus a gated read of the
state, and the state update) and its check against a sequential reference that
the page calls but does not print.

Reading (the page leaves the recurrence implicit; this is the one its chunk
algebra reproduces exactly when the decays are kept per key dimension): with
S the [K, V] state, per token t
    S'   = diag(exp(g_t)) S_{t-1}
    u_t  = S'^T (b_t * k_t)
    vn_t = w_t * v_t - u_t
    S_t  = S' + k_t vn_t^T
    o_t  = scale * S_t^T q_t
The page's chunk form averages exp(G_i - G_j) over the key dimension before
using it; that is an approximation of this recurrence and is not reproduced.

``recurrent`` is the definition above, token by token.  ``chunked`` is the same
operation regrouped into chunks of C tokens (the exact WY form, decays kept per
key dimension), written from the algebra: it must equal ``recurrent`` up to
rounding for every C, and pins the grouping a chunked kernel uses.
"""
import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def recurrent(q, k, v, g, b, w, S0=None, scale=1.0):
    """q, k, g, b [B, H, T, K]; v, w [B, H, T, V]; S0 [B, H, K, V] or None (zero).
    Returns (o [B, H, T, V], S_T [B, H, K, V]), float64."""
    q, k, v, g, b, w = map(_f64, (q, k, v, g, b, w))
    Bt, H, T, K = q.shape
    V = v.shape[-1]
    S = np.zeros((Bt, H, K, V)) if S0 is None else _f64(S0).copy()
    o = np.empty((Bt, H, T, V))
    for t in range(T):
        S = np.exp(g[:, :, t, :])[..., None] * S
        u = np.einsum("bhk,bhkv->bhv", b[:, :, t] * k[:, :, t], S)
        vn = w[:, :, t] * v[:, :, t] - u
        S = S + k[:, :, t][..., None] * vn[:, :, None, :]
        o[:, :, t] = scale * np.einsum("bhk,bhkv->bhv", q[:, :, t], S)
    return o, S


def chunked(q, k, v, g, b, w, S0=None, scale=1.0, chunk=64):
    """The same operation in chunks of `chunk` tokens (exact WY form)."""
    q, k, v, g, b, w = map(_f64, (q, k, v, g, b, w))
    Bt, H, T, K = q.shape
    V = v.shape[-1]
    S = np.zeros((Bt, H, K, V)) if S0 is None else _f64(S0).copy()
    o = np.empty((Bt, H, T, V))
    for s in range(0, T, chunk):
        e = min(s + chunk, T)
        c = e - s
        qc, kc, vc, bc, wc = q[:, :, s:e], k[:, :, s:e], v[:, :, s:e], b[:, :, s:e], w[:, :, s:e]
        G = np.cumsum(g[:, :, s:e], axis=2)                      # [B, H, c, K], inclusive
        dec = np.exp(G[:, :, :, None, :] - G[:, :, None, :, :])  # [B, H, i, j, K]: exp(G_i - G_j)
        lower = np.tril(np.ones((c, c)), -1)                     # j < i
        causal = np.tril(np.ones((c, c)))                        # j <= i
        A = np.einsum("bhik,bhjk,bhijk->bhij", bc * kc, kc, dec) * lower
        P = np.einsum("bhik,bhjk,bhijk->bhij", qc, kc, dec) * causal
        M = np.eye(c) + A                                        # unit lower triangular
        Wf = np.linalg.solve(M, bc * kc * np.exp(G))             # [B, H, c, K]
        U = np.linalg.solve(M, wc * vc)                          # [B, H, c, V]
        vn = U - Wf @ S                                          # corrected values
        o[:, :, s:e] = scale * (P @ vn + (qc * np.exp(G)) @ S)
        Gl = G[:, :, -1:, :]                                     # [B, H, 1, K]
        S = np.exp(Gl[:, :, 0, :])[..., None] * S + np.swapaxes(kc * np.exp(Gl - G), 2, 3) @ vn
    return o, S
