"""f64 CPU oracle of one Mamba block around the selective scan, and its exact
adjoint.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it; it shares no code with the HIP
library.

Definition (rustytorch commit log, page "crates/training/rtx-transformers/
tests": the commit replacing the MambaBlock stub defines the block, here as
equations over token rows of X: [u | z] = X W_in^T; v = silu(causal depthwise
conv of u + conv_b); [r | B | C] = v W_x^T; delta = softplus(r W_dt^T + dt_bias);
y = scan(v, delta, B, C) * silu(z); Y = y W_out^T, the residual being the
caller's.  The hand-written VJP commit gives the parameter list whose gradients
are returned, each summed over the batch).

Readings where the pages are silent: the projections are bias-free linear maps
y = x W^T with PyTorch's [out, in] weight layout; in_proj's first d_inner
outputs feed the conv and the next d_inner are the gate z; x_proj's outputs are
(dt_low [dt_rank], B [d_state], C [d_state]) in that order; dt_proj is the
low-rank map dt = dt_low W_dt^T whose bias is dt_bias inside the softplus.

Each step is a library matmul (numpy) or the f64 conv / scan oracles of this
package, composed in the order above; the backward is the chain rule through
the same steps in reverse.
"""
import numpy as np

from . import bwd as scan_bwd
from . import conv_bwd, conv_fwd
from . import fwd as scan_fwd

PARAMS = ("W_in", "conv_w", "conv_b", "W_x", "W_dt", "dt_bias", "A_log", "D", "W_out")


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _split(p):
    d_inner = p["W_in"].shape[0] // 2
    rank = p["W_dt"].shape[1]
    n = p["A_log"].shape[1]
    return d_inner, rank, n


def block_fwd(X, p):
    """X [batch, L, d_model]; p: dict of PARAMS (W_in [2 d_inner, d_model], conv_w
    [d_inner, K], conv_b [d_inner], W_x [dt_rank + 2 N, d_inner], W_dt [d_inner,
    dt_rank], dt_bias [d_inner], A_log [d_inner, N], D [d_inner], W_out [d_model,
    d_inner]).  Returns the output Y and every intermediate, all f64."""
    X = _f64(X)
    p = {k: _f64(v) for k, v in p.items()}
    di, r, n = _split(p)
    xi = X @ p["W_in"][:di].T
    z = X @ p["W_in"][di:].T
    xc = conv_fwd(xi, p["conv_w"], p["conv_b"])["y"]
    proj = xc @ p["W_x"].T
    dt_low, Bm, Cm = proj[..., :r], proj[..., r:r + n], proj[..., r + n:]
    dt = dt_low @ p["W_dt"].T
    y_s = scan_fwd(xc, dt, Bm, Cm, z, p["A_log"], p["D"], p["dt_bias"])["y"]
    Y = y_s @ p["W_out"].T
    return {"Y": Y, "xi": xi, "z": z, "xc": xc, "proj": proj, "dt": dt, "y_s": y_s}


def _wgrad(dout, inp):
    """sum over (batch, time) of dout^T inp: [out, in]."""
    return np.tensordot(dout, inp, axes=([0, 1], [0, 1]))


def block_bwd(X, p, dY):
    """Gradients of sum(dY * Y): dict with dX and d<name> for every PARAMS entry."""
    X = _f64(X)
    dY = _f64(dY)
    p = {k: _f64(v) for k, v in p.items()}
    di, r, n = _split(p)
    f = block_fwd(X, p)
    g = {"dW_out": _wgrad(dY, f["y_s"])}
    dy_s = dY @ p["W_out"]
    proj = f["proj"]
    s = scan_bwd(f["xc"], f["dt"], proj[..., r:r + n], proj[..., r + n:], f["z"], p["A_log"], p["D"],
                 p["dt_bias"], dy_s)
    g.update(dA_log=s["dA_log"], dD=s["dD"], ddt_bias=s["ddt_bias"])
    dt_low = proj[..., :r]
    g["dW_dt"] = _wgrad(s["ddt"], dt_low)
    dproj = np.concatenate([s["ddt"] @ p["W_dt"], s["dB"], s["dC"]], axis=-1)
    g["dW_x"] = _wgrad(dproj, f["xc"])
    dxc = s["dx"] + dproj @ p["W_x"]
    c = conv_bwd(f["xi"], p["conv_w"], p["conv_b"], dxc)
    g.update(dconv_w=c["dw"], dconv_b=c["dbias"])
    dxi, dz = c["dx"], s["dz"]
    g["dW_in"] = np.concatenate([_wgrad(dxi, X), _wgrad(dz, X)], axis=0)
    g["dX"] = dxi @ p["W_in"][:di] + dz @ p["W_in"][di:]
    return g
