"""Pins of the f64 oracle against things other than itself.

Each test fixes the oracle to an independent formula, a closed form, a library
routine, finite differences or an invariant of the method, chosen so that a
dropped term, a wrong sign, a wrong index or a transposed operand in the
oracle fails at least one of them:

* dual form: y_t = sum_{s<=t} sum_n C_t exp(A (cum_t - cum_s)) delta_s B_s x_s
  + D x_t (the unrolled recurrence, O(L^2), no recursion), random A_log;
* geometric series for constant inputs; the delta -> 0 limit; N = 1 as a
  first-order IIR filter (scipy.signal.lfilter);
* every gradient against f64 central differences, and against torch-f64
  autograd of a separate vectorised implementation written here;
* the adjoint dot-product identity at a larger size;
* step == forward exactly, causality, split invariance, finite delta at
  dt = +100, and the constants the pages fix (tests/golden/page_constants.txt).
"""
import os

import numpy as np
import pytest
from scipy.signal import lfilter
from scipy.special import expit

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.txt")


def _small(batch=2, L=7, D=3, N=4, seed=3, dt_bias=0.2, with_z=True, h0=True):
    rng = np.random.default_rng(seed)
    inp = {
        "x": rng.standard_normal((batch, L, D)),
        "dt": 0.5 * rng.standard_normal((batch, L, D)),
        "B": rng.standard_normal((batch, L, N)),
        "C": rng.standard_normal((batch, L, N)),
        "z": rng.standard_normal((batch, L, D)) if with_z else None,
        "A_log": np.log(np.arange(1, N + 1))[None, :] + 0.3 * rng.standard_normal((D, N)),
        "D": rng.standard_normal(D),
        "dt_bias": dt_bias + 0.1 * rng.standard_normal(D),
        "h0": rng.standard_normal((batch, D, N)) if h0 else None,
    }
    dy = rng.standard_normal((batch, L, D))
    return inp, dy


def _softplus(u):
    return np.logaddexp(0.0, u)


def _silu(z):
    return z * expit(z)


def _dual_form(inp):
    """Unrolled solution of the recurrence, written from its closed form."""
    x, dt, B, C = inp["x"], inp["dt"], inp["B"], inp["C"]
    A = -np.exp(inp["A_log"])                      # [D, N]
    delta = _softplus(dt + inp["dt_bias"])        # [b, L, D]
    cum = np.cumsum(delta, axis=1)                 # inclusive prefix sum over time
    bsz, L, D = x.shape
    y = np.zeros_like(x)
    for b in range(bsz):
        for t in range(L):
            for d in range(D):
                s = np.arange(t + 1)
                decay = np.exp(A[d][None, :] * (cum[b, t, d] - cum[b, s, d])[:, None])  # [s, N]
                h = (decay * (delta[b, s, d] * x[b, s, d])[:, None] * B[b, s, :]).sum(0)
                if inp.get("h0") is not None:
                    h = h + np.exp(A[d] * cum[b, t, d]) * inp["h0"][b, d]
                ypre = (C[b, t] * h).sum() + inp["D"][d] * x[b, t, d]
                y[b, t, d] = ypre * (_silu(inp["z"][b, t, d]) if inp["z"] is not None else 1.0)
    return y


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def _fwd(inp):
    return oracle.fwd(inp["x"], inp["dt"], inp["B"], inp["C"], inp["z"], inp["A_log"], inp["D"],
                      inp["dt_bias"], inp.get("h0"))


def _bwd(inp, dy):
    return oracle.bwd(inp["x"], inp["dt"], inp["B"], inp["C"], inp["z"], inp["A_log"], inp["D"],
                      inp["dt_bias"], dy, inp.get("h0"))


@pytest.mark.parametrize("with_z,h0", [(True, True), (False, False), (True, False)])
def test_forward_matches_dual_form(with_z, h0):
    inp, _ = _small(batch=2, L=23, D=5, N=16, seed=11, with_z=with_z, h0=h0)
    y = _fwd(inp)["y"]
    assert _rel(y, _dual_form(inp)) < 1e-12


def test_forward_dual_form_active_regime_config_shape():
    # tiny config shape (1 x 64 x 32 x 16) with the pages' init and delta ~ 0.69
    inp = W.make_config("c1_tiny")
    inp = {k: (None if v is None else v.astype(np.float64)) for k, v in inp.items()}
    inp["h0"] = None
    y = _fwd(inp)["y"]
    assert _rel(y, _dual_form(inp)) < 1e-12


def test_geometric_series_constant_inputs():
    # constant x, dt, B, C, z over time: h_t = delta*b*x*expm1((t+1)*delta*A)/expm1(delta*A)
    bsz, L, D, N = 1, 300, 4, 16
    rng = np.random.default_rng(5)
    xv, dtv, zv = rng.standard_normal(D), 0.3 * rng.standard_normal(D), rng.standard_normal(D)
    bv, cv = rng.standard_normal(N), rng.standard_normal(N)
    A_log = W.a_log_canonical(D, N).astype(np.float64) - 2.0
    dt_bias = np.full(D, -1.0)
    inp = {
        "x": np.broadcast_to(xv, (bsz, L, D)).copy(), "dt": np.broadcast_to(dtv, (bsz, L, D)).copy(),
        "z": np.broadcast_to(zv, (bsz, L, D)).copy(), "B": np.broadcast_to(bv, (bsz, L, N)).copy(),
        "C": np.broadcast_to(cv, (bsz, L, N)).copy(), "A_log": A_log, "D": np.full(D, 0.7),
        "dt_bias": dt_bias, "h0": None,
    }
    out = _fwd(inp)
    delta = _softplus(dtv + dt_bias)
    A = -np.exp(A_log)
    t = np.arange(L)
    for d in range(D):
        dA = delta[d] * A[d]                                   # [N]
        h = (delta[d] * bv * xv[d])[None, :] * np.expm1((t[:, None] + 1) * dA[None, :]) / np.expm1(dA)[None, :]
        y = (h @ cv + 0.7 * xv[d]) * (zv[d] / (1 + np.exp(-zv[d])))
        assert _rel(out["y"][0, :, d], y) < 1e-13
    assert np.allclose(out["delta"][0, 0], delta, rtol=1e-15, atol=0)


def test_delta_to_zero_limit():
    inp, dy = _small(batch=2, L=40, D=6, N=16, seed=7, dt_bias=-40.0, h0=False)
    out = _fwd(inp)
    assert np.max(out["delta"]) < 1e-16
    expect = inp["D"][None, None, :] * inp["x"] * _silu(inp["z"])
    assert np.max(np.abs(out["y"] - expect)) <= 1e-14 * np.max(np.abs(expect))
    g = _bwd(inp, dy)
    gate = dy * _silu(inp["z"])
    assert np.max(np.abs(g["dC"])) < 1e-14
    assert np.max(np.abs(g["dx"] - gate * inp["D"][None, None, :])) < 1e-14
    assert _rel(g["dD"], (gate * inp["x"]).sum((0, 1))) < 1e-13


def test_single_state_is_first_order_iir_filter():
    # N = 1 with constant delta: h is y = lfilter([1], [1, -a], delta*B*x)
    L, D = 500, 3
    rng = np.random.default_rng(9)
    inp = {
        "x": rng.standard_normal((1, L, D)), "dt": np.zeros((1, L, D)),
        "B": rng.standard_normal((1, L, 1)), "C": rng.standard_normal((1, L, 1)), "z": None,
        "A_log": np.array([[0.1], [-0.5], [1.2]]), "D": np.array([0.3, -0.2, 0.0]),
        "dt_bias": np.array([0.4, -1.0, 2.0]), "h0": None,
    }
    out = _fwd(inp)
    for d in range(D):
        delta = _softplus(inp["dt_bias"][d])
        a = np.exp(-np.exp(inp["A_log"][d, 0]) * delta)
        u = delta * inp["B"][0, :, 0] * inp["x"][0, :, d]
        h = lfilter([1.0], [1.0, -a], u)
        y = inp["C"][0, :, 0] * h + inp["D"][d] * inp["x"][0, :, d]
        assert _rel(out["y"][0, :, d], y) < 1e-12


def test_step_equals_forward_exactly():
    inp, _ = _small(batch=3, L=50, D=8, N=16, seed=2, h0=False)
    y_full = _fwd(inp)["y"]
    h = np.zeros((3, 8, 16))
    ys = []
    for t in range(50):
        ys.append(oracle.step(h, inp["x"][:, t], inp["dt"][:, t], inp["B"][:, t], inp["C"][:, t],
                              inp["z"][:, t], inp["A_log"], inp["D"], inp["dt_bias"]))
    assert np.max(np.abs(np.stack(ys, 1) - y_full)) == 0.0
    assert np.max(np.abs(h - _fwd(inp)["h_last"])) == 0.0


def test_causality_exact():
    inp, _ = _small(batch=1, L=60, D=4, N=16, seed=4)
    y0 = _fwd(inp)["y"]
    inp2 = dict(inp)
    inp2["x"] = inp["x"].copy()
    inp2["x"][:, 37] += 1.0
    y1 = _fwd(inp2)["y"]
    assert np.max(np.abs(y1[:, :37] - y0[:, :37])) == 0.0
    assert np.max(np.abs(y1[:, 37:] - y0[:, 37:])) > 0.0


def test_split_invariance_exact():
    inp, _ = _small(batch=2, L=64, D=5, N=16, seed=6, h0=True)
    full = _fwd(inp)
    L1 = 29
    a = {k: (v[:, :L1] if k in ("x", "dt", "B", "C", "z") else v) for k, v in inp.items()}
    first = _fwd(a)
    b = {k: (v[:, L1:] if k in ("x", "dt", "B", "C", "z") else v) for k, v in inp.items()}
    b["h0"] = first["h_last"]
    second = _fwd(b)
    assert np.max(np.abs(np.concatenate([first["y"], second["y"]], 1) - full["y"])) == 0.0
    assert np.max(np.abs(second["h_last"] - full["h_last"])) == 0.0


def test_finite_delta_at_large_dt():
    inp, dy = _small(batch=1, L=16, D=3, N=16, seed=8)
    inp["dt"] = np.full_like(inp["dt"], 100.0)
    inp["dt_bias"] = np.zeros(3)
    out = _fwd(inp)
    assert np.all(out["delta"] == 100.0)
    assert np.all(np.isfinite(out["y"]))
    g = _bwd(inp, dy)
    for k, v in g.items():
        if v is not None:
            assert np.all(np.isfinite(v)), k


def test_page_constants():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            vals[parts[0]] = parts[1]
    # delta at dt = 0, dt_bias = 0 is the active regime value; dt_bias_slow gives 0.01
    inp, _ = _small(batch=1, L=2, D=2, N=16, seed=1)
    inp["dt"] = np.zeros_like(inp["dt"])
    inp["dt_bias"] = np.array([0.0, W.DT_BIAS_SLOW])
    out = _fwd(inp)
    assert abs(out["delta"][0, 0, 0] - float(vals["softplus_active"])) < 1e-15
    assert abs(out["delta"][0, 0, 1] - float(vals["softplus_slow"])) < 1e-8
    # A = -(1..N) from A_log = ln(1..N): with delta = ln 2 the decay of state n is 2^-(n+1).
    N = 16
    inp = {"x": np.ones((1, 1, 1)), "dt": np.zeros((1, 1, 1)), "B": np.zeros((1, 1, N)),
           "C": np.eye(N)[None, :1, :], "z": None, "A_log": np.log(np.arange(1.0, N + 1))[None, :],
           "D": np.zeros(1), "dt_bias": np.zeros(1), "h0": np.ones((1, 1, N))}
    h = _fwd(inp)["h_last"][0, 0]
    assert np.allclose(h, 2.0 ** -np.arange(1, N + 1), rtol=1e-13, atol=0)
    assert float(vals["step_vs_forward_diff"]) == 0.0


# ---------------------------------------------------------------- gradients

def _loss(inp, dy):
    return float((_fwd(inp)["y"] * dy).sum())


@pytest.mark.parametrize("with_z,h0", [(True, True), (False, False)])
def test_gradients_match_central_differences(with_z, h0):
    inp, dy = _small(batch=2, L=7, D=3, N=4, seed=13, with_z=with_z, h0=h0)
    g = _bwd(inp, dy)
    names = {"x": "dx", "dt": "ddt", "B": "dB", "C": "dC", "A_log": "dA_log", "D": "dD",
             "dt_bias": "ddt_bias"}
    if with_z:
        names["z"] = "dz"
    if h0:
        names["h0"] = "dh0"
    eps = 1e-6
    for inname, gname in names.items():
        base = inp[inname]
        fd = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            p = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
            m = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
            p[inname][idx] += eps
            m[inname][idx] -= eps
            fd[idx] = (_loss(p, dy) - _loss(m, dy)) / (2 * eps)
        err = np.max(np.abs(fd - g[gname])) / max(np.max(np.abs(fd)), 1e-12)
        assert err < 1e-7, (inname, err)


def _torch_reference(inp, dy):
    """Separate vectorised f64 implementation, differentiated by torch autograd."""
    import torch
    import torch.nn.functional as F
    t = {k: (None if v is None else torch.tensor(v, dtype=torch.float64, requires_grad=True))
         for k, v in inp.items()}
    A = -torch.exp(t["A_log"])
    delta = torch.logaddexp(torch.zeros((), dtype=torch.float64), t["dt"] + t["dt_bias"])
    bsz, L, D = t["x"].shape
    h = t["h0"] if t["h0"] is not None else torch.zeros(bsz, D, A.shape[1], dtype=torch.float64)
    ys = []
    for s in range(L):
        dA = torch.exp(delta[:, s, :, None] * A[None])
        h = dA * h + (delta[:, s, :, None] * t["x"][:, s, :, None]) * t["B"][:, s, None, :]
        ypre = (h * t["C"][:, s, None, :]).sum(-1) + t["D"] * t["x"][:, s]
        ys.append(ypre * F.silu(t["z"][:, s]) if t["z"] is not None else ypre)
    y = torch.stack(ys, 1)
    (y * torch.tensor(dy)).sum().backward()
    grads = {k: (None if v is None else v.grad.numpy()) for k, v in t.items()}
    return y.detach().numpy(), grads


def test_gradients_match_torch_autograd():
    inp, dy = _small(batch=2, L=33, D=6, N=16, seed=21, h0=True)
    y_ref, gr = _torch_reference(inp, dy)
    assert _rel(_fwd(inp)["y"], y_ref) < 1e-13
    g = _bwd(inp, dy)
    pairs = {"x": "dx", "dt": "ddt", "B": "dB", "C": "dC", "z": "dz", "A_log": "dA_log",
             "D": "dD", "dt_bias": "ddt_bias", "h0": "dh0"}
    for k, gk in pairs.items():
        assert _rel(g[gk], gr[k]) < 1e-12, k


def test_adjoint_dot_product_and_internal_sums():
    # <dy, J v> (J v by central differences along a random direction) == sum(grad * v)
    inp, dy = _small(batch=2, L=256, D=24, N=16, seed=31, h0=True)
    g = _bwd(inp, dy)
    rng = np.random.default_rng(99)
    dirs = {k: rng.standard_normal(np.shape(v)) for k, v in inp.items() if v is not None}
    eps = 1e-6
    p = {k: (v + eps * dirs[k] if v is not None else None) for k, v in inp.items()}
    m = {k: (v - eps * dirs[k] if v is not None else None) for k, v in inp.items()}
    jv = (_loss(p, dy) - _loss(m, dy)) / (2 * eps)
    names = {"x": "dx", "dt": "ddt", "B": "dB", "C": "dC", "z": "dz", "A_log": "dA_log",
             "D": "dD", "dt_bias": "ddt_bias", "h0": "dh0"}
    vjp = sum(float((g[gn] * dirs[k]).sum()) for k, gn in names.items())
    assert abs(jv - vjp) <= 1e-6 * abs(vjp)
    # ddt_bias is the time/batch sum of ddt; dD is the sum of (dy*silu(z))*x;
    # ddt = ddelta * sigmoid(dt + dt_bias)
    assert _rel(g["ddt_bias"], g["ddt"].sum((0, 1))) < 1e-13
    assert _rel(g["dD"], (dy * _silu(inp["z"]) * inp["x"]).sum((0, 1))) < 1e-13
    assert _rel(g["ddt"], g["ddelta"] * expit(inp["dt"] + inp["dt_bias"])) < 1e-14


def test_results_do_not_depend_on_thread_count():
    # dB/dC are block sums in fixed order; a single-thread run must agree bit for bit
    import subprocess
    import sys
    code = ("import numpy as np, oracle, json, sys;"
            "from tests.test_oracle_pins import _small, _bwd;"
            "inp, dy = _small(batch=2, L=40, D=40, N=16, seed=17);"
            "g = _bwd(inp, dy); np.save(sys.argv[1], np.concatenate([g['dB'].ravel(), g['dC'].ravel(), g['dA_log'].ravel()]))")
    outs = []
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for nt in ("1", "3"):
        fn = os.path.join("/tmp", f"oracle_threads_{nt}_{os.getpid()}.npy")
        env = dict(os.environ, OMP_NUM_THREADS=nt, PYTHONPATH=root)
        subprocess.run([sys.executable, "-c", code, fn], check=True, env=env, cwd=root)
        outs.append(np.load(fn))
        os.remove(fn)
    assert np.array_equal(outs[0], outs[1])
