"""f64 CPU oracle of the Mamba S6 selective scan (forward, reverse-time adjoint, step).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and the HIP library never calls it.

The arithmetic lives in ``ssm_oracle.c`` (the scan) and ``conv_oracle.c`` (the
causal depthwise conv1d + SiLU in front of it): plain f64 loops, OpenMP over
channels.  This module only marshals numpy arrays: every input is promoted to
f64 exactly (f32 and bf16 values are representable in f64) and every output is
returned as f64.

Definition followed (rustytorch commit log, page "crates/training/rtx-transformers/
tests": the commit replacing the MambaBlock stub with a real S6 forward, the
commit adding the hand-written VJP, and the one adding MambaRecurrence::step):
    delta = softplus(dt + dt_bias), A = -exp(A_log)
    h_t   = exp(delta*A)*h_{t-1} + delta*B_t*x_t
    y_t   = (sum_n C_t*h_t + D*x_t) * silu(z_t)
and its exact adjoint; parameter gradients are summed over batch and time,
dB/dC over channels, and dA_log = dA * A.
"""
import ctypes
import os

import numpy as np

from ._build import LIB_PATH, build_oracle

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build_oracle()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int64
    lib.oracle_fwd.argtypes = [I, I, I, I] + [P] * 12
    lib.oracle_fwd.restype = ctypes.c_int
    lib.oracle_bwd.argtypes = [I, I, I, I] + [P] * 20
    lib.oracle_bwd.restype = ctypes.c_int
    lib.oracle_step.argtypes = [I, I, I] + [P] * 10
    lib.oracle_step.restype = ctypes.c_int
    lib.oracle_conv_fwd.argtypes = [I, I, I, I] + [P] * 7
    lib.oracle_conv_fwd.restype = ctypes.c_int
    lib.oracle_conv_bwd.argtypes = [I, I, I, I] + [P] * 9
    lib.oracle_conv_bwd.restype = ctypes.c_int
    lib.oracle_conv_step.argtypes = [I, I, I] + [P] * 5
    lib.oracle_conv_step.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads():
    """OpenMP threads the oracle runs with."""
    return int(_load().oracle_num_threads())


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dims(x, B):
    x = np.asarray(x)
    Bsz = np.asarray(B)
    if x.ndim != 3 or Bsz.ndim != 3:
        raise ValueError("x must be [batch, seqlen, d_inner] and B [batch, seqlen, d_state]")
    return x.shape[0], x.shape[1], x.shape[2], Bsz.shape[2]


def fwd(x, dt, B, C, z, A_log, D, dt_bias, h0=None):
    """Forward scan.  Returns dict(y, h_last, delta), all f64."""
    bt, L, d, n = _dims(x, B)
    args = [_f64(a) for a in (x, dt, B, C, z, A_log, D, dt_bias, h0)]
    y = np.empty((bt, L, d))
    h_last = np.empty((bt, d, n))
    delta = np.empty((bt, L, d))
    rc = _load().oracle_fwd(bt, L, d, n, *[_ptr(a) for a in args], _ptr(y), _ptr(h_last), _ptr(delta))
    if rc != 0:
        raise RuntimeError(f"oracle_fwd failed: {rc}")
    return {"y": y, "h_last": h_last, "delta": delta}


def bwd(x, dt, B, C, z, A_log, D, dt_bias, dy, h0=None):
    """Reverse-time adjoint.  Returns dict of f64 gradients:
    dx, ddt, dz (None without a gate), dB, dC, dA_log, dD, ddt_bias, dh0, ddelta
    (ddelta is the gradient w.r.t. the post-softplus delta; ddt = ddelta*sigmoid(u))."""
    bt, L, d, n = _dims(x, B)
    args = [_f64(a) for a in (x, dt, B, C, z, A_log, D, dt_bias, h0, dy)]
    out = {
        "dx": np.empty((bt, L, d)), "ddt": np.empty((bt, L, d)),
        "dB": np.empty((bt, L, n)), "dC": np.empty((bt, L, n)),
        "dz": np.empty((bt, L, d)) if z is not None else None,
        "dA_log": np.empty((d, n)), "dD": np.empty(d), "ddt_bias": np.empty(d),
        "dh0": np.empty((bt, d, n)), "ddelta": np.empty((bt, L, d)),
    }
    order = ["dx", "ddt", "dB", "dC", "dz", "dA_log", "dD", "ddt_bias", "dh0", "ddelta"]
    rc = _load().oracle_bwd(bt, L, d, n, *[_ptr(a) for a in args], *[_ptr(out[k]) for k in order])
    if rc != 0:
        raise RuntimeError(f"oracle_bwd failed: {rc}")
    return out


def step(h, x, dt, B, C, z, A_log, D, dt_bias):
    """Single-token update.  h: f64 array [batch, d_inner, d_state], updated in place.
    x, dt, z: [batch, d_inner]; B, C: [batch, d_state].  Returns y [batch, d_inner]."""
    if not (isinstance(h, np.ndarray) and h.dtype == np.float64 and h.flags.c_contiguous):
        raise ValueError("h must be a C-contiguous float64 array (updated in place)")
    bt, d, n = h.shape
    args = [_f64(a) for a in (x, dt, B, C, z, A_log, D, dt_bias)]
    y = np.empty((bt, d))
    rc = _load().oracle_step(bt, d, n, _ptr(h), *[_ptr(a) for a in args], _ptr(y))
    if rc != 0:
        raise RuntimeError(f"oracle_step failed: {rc}")
    return y


def _conv_dims(x, w):
    x = np.asarray(x)
    w = np.asarray(w)
    if x.ndim != 3 or w.ndim != 2 or w.shape[0] != x.shape[2]:
        raise ValueError("x must be [batch, seqlen, d_inner] and w [d_inner, d_conv]")
    return x.shape[0], x.shape[1], x.shape[2], w.shape[1]


def conv_fwd(x, w, bias, s0=None):
    """Causal depthwise conv1d + SiLU.  Returns dict(y, pre, s_last), all f64:
    y = silu(pre) [batch, L, d_inner]; s_last [batch, d_inner, d_conv-1] the last
    d_conv-1 inputs, oldest first (from s0 when L < d_conv-1)."""
    bt, L, d, k = _conv_dims(x, w)
    args = [_f64(a) for a in (x, w, bias, s0)]
    y = np.empty((bt, L, d))
    pre = np.empty((bt, L, d))
    s_last = np.empty((bt, d, k - 1))
    rc = _load().oracle_conv_fwd(bt, L, d, k, *[_ptr(a) for a in args], _ptr(y), _ptr(s_last), _ptr(pre))
    if rc != 0:
        raise RuntimeError(f"oracle_conv_fwd failed: {rc}")
    return {"y": y, "pre": pre, "s_last": s_last}


def conv_bwd(x, w, bias, dy, s0=None):
    """Adjoint of conv_fwd.  Returns dict(dx, dw, dbias, ds0), all f64; dw and dbias
    are summed over batch and time; ds0 is the gradient of the initial ring."""
    bt, L, d, k = _conv_dims(x, w)
    args = [_f64(a) for a in (x, w, bias, s0, dy)]
    out = {"dx": np.empty((bt, L, d)), "dw": np.empty((d, k)), "dbias": np.empty(d),
           "ds0": np.empty((bt, d, k - 1))}
    rc = _load().oracle_conv_bwd(bt, L, d, k, *[_ptr(a) for a in args],
                                 *[_ptr(out[n]) for n in ("dx", "dw", "dbias", "ds0")])
    if rc != 0:
        raise RuntimeError(f"oracle_conv_bwd failed: {rc}")
    return out


def conv_step(ring, x, w, bias):
    """One token of conv_fwd.  ring: f64 [batch, d_inner, d_conv-1], updated in
    place (drops the oldest input, appends x); x: [batch, d_inner].  Returns y."""
    if not (isinstance(ring, np.ndarray) and ring.dtype == np.float64 and ring.flags.c_contiguous):
        raise ValueError("ring must be a C-contiguous float64 array (updated in place)")
    w = _f64(w)
    bt, d = np.asarray(x).shape
    k = w.shape[1]
    y = np.empty((bt, d))
    rc = _load().oracle_conv_step(bt, d, k, _ptr(ring), _ptr(_f64(x)), _ptr(w), _ptr(_f64(bias)), _ptr(y))
    if rc != 0:
        raise RuntimeError(f"oracle_conv_step failed: {rc}")
    return y
