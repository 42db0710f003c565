"""Pins of the f64 Mamba-block oracle (oracle/block.py): its output and every
gradient against f64 central differences and against torch autograd of an
independent formulation (torch linear / conv1d layers and a step loop for the
scan), so that a mis-wired composition (a transposed projection, a swapped
in_proj half, a dropped gradient path) fails.

Definition: rustytorch commit log, page "crates/training/rtx-transformers/tests"
(commit replacing the MambaBlock stub; hand-written VJP commit).
"""
import numpy as np
import pytest

import workloads as W
from oracle.block import PARAMS, block_bwd, block_fwd

torch = pytest.importorskip("torch")


def _small(seed=0, bt=2, L=7, dm=5, di=6, r=2, k=3, bias=True):
    X, p, dY = W.make_block_inputs(bt, L, dm, di, 16, r, k, seed=seed)
    X, dY = X.astype(np.float64), dY.astype(np.float64)
    p = {kk: v.astype(np.float64) for kk, v in p.items()}
    rng = np.random.default_rng(seed + 100)
    if bias:
        p["conv_b"] = 0.3 * rng.standard_normal(di)
    p["dt_bias"] = p["dt_bias"] + 0.5 * rng.standard_normal(di)  # spread the decays
    p["D"] = 1.0 + 0.5 * rng.standard_normal(di)
    return X, p, dY


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(float(np.max(np.abs(b))), 1e-300))


def test_gradients_match_finite_differences():
    X, p, dY = _small()
    g = block_bwd(X, p, dY)
    eps = 1e-6
    targets = [("X", X, "dX")] + [(k, p[k], "d" + k) for k in PARAMS]
    for name, arr, gname in targets:
        fd = np.empty_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            save = arr[i]
            arr[i] = save + eps
            lp = float(np.sum(dY * block_fwd(X, p)["Y"]))
            arr[i] = save - eps
            lm = float(np.sum(dY * block_fwd(X, p)["Y"]))
            arr[i] = save
            fd[i] = (lp - lm) / (2 * eps)
        assert _rel(g[gname], fd) < 1e-6, name


def _torch_block(X, p, dY):
    import torch.nn.functional as F
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p.items()}
    Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    di = t["W_in"].shape[0] // 2
    r = t["W_dt"].shape[1]
    n = t["A_log"].shape[1]
    K = t["conv_w"].shape[1]
    L = X.shape[1]
    u = F.linear(Xt, t["W_in"])                       # [b, L, 2 di]
    xi, z = u[..., :di], u[..., di:]
    pre = F.conv1d(xi.transpose(1, 2), t["conv_w"][:, None, :], t["conv_b"], padding=K - 1, groups=di)[..., :L]
    xc = F.silu(pre).transpose(1, 2)
    proj = F.linear(xc, t["W_x"])
    dt = F.linear(proj[..., :r], t["W_dt"])
    Bm, Cm = proj[..., r:r + n], proj[..., r + n:]
    delta = F.softplus(dt + t["dt_bias"])
    A = -torch.exp(t["A_log"])
    h = torch.zeros(X.shape[0], di, n, dtype=torch.float64)
    ys = []
    for s in range(L):
        h = torch.exp(delta[:, s, :, None] * A) * h + (delta[:, s] * xc[:, s])[..., None] * Bm[:, s, None, :]
        ys.append(((h * Cm[:, s, None, :]).sum(-1) + t["D"] * xc[:, s]) * F.silu(z[:, s]))
    Y = F.linear(torch.stack(ys, 1), t["W_out"])
    (Y * torch.tensor(dY)).sum().backward()
    grads = {"d" + k: v.grad.numpy() for k, v in t.items()}
    grads["dX"] = Xt.grad.numpy()
    return Y.detach().numpy(), grads


@pytest.mark.parametrize("k", [1, 4])
def test_matches_torch_autograd(k):
    X, p, dY = _small(seed=3, bt=2, L=19, dm=8, di=12, r=3, k=k)
    Y_ref, gr = _torch_block(X, p, dY)
    assert _rel(block_fwd(X, p)["Y"], Y_ref) < 1e-12
    g = block_bwd(X, p, dY)
    for name in ["dX"] + ["d" + k for k in PARAMS]:
        assert _rel(g[name], gr[name]) < 1e-11, name


def test_intermediates_are_consistent():
    """x_proj's outputs are (dt_low, B, C) in that order and the gate uses in_proj's
    second half: swapping either changes Y."""
    X, p, dY = _small(seed=5)
    f = block_fwd(X, p)
    q = dict(p)
    q["W_in"] = np.concatenate([p["W_in"][6:], p["W_in"][:6]], axis=0)
    assert _rel(block_fwd(X, q)["Y"], f["Y"]) > 1e-3
    assert f["proj"].shape[-1] == 2 + 32 and f["dt"].shape == f["xc"].shape
