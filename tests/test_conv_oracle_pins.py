"""Pins of the f64 conv1d + SiLU oracle (oracle/conv_oracle.c) against things
other than itself: library convolutions (numpy, torch), finite differences,
torch autograd of an independent formulation, and exact invariants of a causal
filter (step chain == forward, split invariance).

Definition (rustytorch commit log, page "crates/training/rtx-transformers/tests":
the real-S6-forward commit applies a causal depthwise conv1d then SiLU before
x_proj; the VJP commit returns conv1d_weight and conv1d_bias gradients;
MambaRecurrence::step carries the conv ring).  Reading: PyTorch's
Conv1d(groups=d_inner, padding=K-1) truncated to the first L outputs.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def _inputs(bt=2, L=37, d=5, k=4, seed=0, ring=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((bt, L, d))
    w = rng.standard_normal((d, k)) * 0.5
    b = rng.standard_normal(d) * 0.3
    s0 = rng.standard_normal((bt, d, k - 1)) if ring else None
    dy = rng.standard_normal((bt, L, d))
    return x, w, b, s0, dy


def _silu(p):
    return p / (1.0 + np.exp(-p))


def _left_context(x, s0, k):
    """[bt, K-1+L, d]: the ring (or zeros) followed by the sequence."""
    bt, L, d = x.shape
    ctx = np.zeros((bt, k - 1, d)) if s0 is None else np.transpose(s0, (0, 2, 1))
    return np.concatenate([ctx, x], axis=1)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("ring", [False, True])
def test_matches_numpy_convolve(k, ring):
    x, w, b, s0, _ = _inputs(k=k, ring=ring and k > 1)
    v = _left_context(x, s0, k)
    ref = np.empty_like(x)
    for bi in range(x.shape[0]):
        for d in range(x.shape[2]):
            # np.convolve flips its kernel: flipping w back gives the causal
            # cross-correlation with tap k on input t-(K-1)+k
            ref[bi, :, d] = np.convolve(v[bi, :, d], w[d, ::-1], mode="valid") + b[d]
    got = oracle.conv_fwd(x, w, b, s0)
    np.testing.assert_allclose(got["pre"], ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(got["y"], _silu(ref), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("k", [1, 3, 4])
def test_matches_torch_conv1d(k):
    x, w, b, _, _ = _inputs(bt=3, L=50, d=7, k=k, ring=False)
    xt = torch.from_numpy(x).permute(0, 2, 1)  # [bt, d, L]
    pre = torch.nn.functional.conv1d(xt, torch.from_numpy(w)[:, None, :], torch.from_numpy(b),
                                     padding=k - 1, groups=x.shape[2])[..., :x.shape[1]]
    ref = torch.nn.functional.silu(pre).permute(0, 2, 1).numpy()
    np.testing.assert_allclose(oracle.conv_fwd(x, w, b)["y"], ref, rtol=1e-13, atol=1e-13)


def test_kernel_width_one_is_pointwise():
    x, w, b, _, _ = _inputs(k=1, ring=False)
    np.testing.assert_allclose(oracle.conv_fwd(x, w, b)["y"], _silu(x * w[:, 0] + b), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("L", [0, 1, 2, 3, 10])
def test_final_ring_holds_last_inputs(L):
    x, w, b, s0, _ = _inputs(L=L, k=4)
    v = _left_context(x, s0, 4)          # [bt, 3+L, d]
    want = np.transpose(v[:, -3:, :], (0, 2, 1))
    np.testing.assert_array_equal(oracle.conv_fwd(x, w, b, s0)["s_last"], want)


@pytest.mark.parametrize("ring", [False, True])
def test_step_chain_equals_forward_exactly(ring):
    x, w, b, s0, _ = _inputs(L=29, k=4, ring=ring)
    full = oracle.conv_fwd(x, w, b, s0)
    r = np.zeros((x.shape[0], x.shape[2], 3)) if s0 is None else s0.copy()
    ys = np.stack([oracle.conv_step(r, x[:, t], w, b) for t in range(x.shape[1])], axis=1)
    np.testing.assert_array_equal(ys, full["y"])
    np.testing.assert_array_equal(r, full["s_last"])


@pytest.mark.parametrize("split", [1, 2, 3, 17])
def test_split_invariance_exact(split):
    x, w, b, s0, _ = _inputs(L=30, k=4)
    full = oracle.conv_fwd(x, w, b, s0)
    a = oracle.conv_fwd(x[:, :split], w, b, s0)
    c = oracle.conv_fwd(x[:, split:], w, b, a["s_last"])
    np.testing.assert_array_equal(np.concatenate([a["y"], c["y"]], axis=1), full["y"])
    np.testing.assert_array_equal(c["s_last"], full["s_last"])


def test_causality():
    x, w, b, s0, _ = _inputs(L=20, k=4)
    y0 = oracle.conv_fwd(x, w, b, s0)["y"]
    x2 = x.copy()
    x2[:, 12:] += 3.0
    y1 = oracle.conv_fwd(x2, w, b, s0)["y"]
    np.testing.assert_array_equal(y0[:, :12], y1[:, :12])
    assert np.all(np.abs(y0[:, 12:] - y1[:, 12:]).max(axis=(0, 2)) > 0)


def _loss(x, w, b, s0, dy):
    return float(np.sum(dy * oracle.conv_fwd(x, w, b, s0)["y"]))


@pytest.mark.parametrize("k", [1, 2, 4])
def test_gradients_match_finite_differences(k):
    x, w, b, s0, dy = _inputs(bt=2, L=9, d=3, k=k, ring=k > 1)
    g = oracle.conv_bwd(x, w, b, dy, s0)
    eps = 1e-6
    named = {"dx": x, "dw": w, "dbias": b}
    if k > 1:
        named["ds0"] = s0
    for name, arr in named.items():
        fd = np.empty_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            save = arr[i]
            arr[i] = save + eps
            lp = _loss(x, w, b, s0, dy)
            arr[i] = save - eps
            lm = _loss(x, w, b, s0, dy)
            arr[i] = save
            fd[i] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[name], fd, rtol=1e-7, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("k", [2, 4])
def test_gradients_match_torch_autograd(k):
    x, w, b, s0, dy = _inputs(bt=3, L=41, d=6, k=k)
    xt = torch.from_numpy(x).requires_grad_()
    wt = torch.from_numpy(w).requires_grad_()
    bt_ = torch.from_numpy(b).requires_grad_()
    st = torch.from_numpy(s0).requires_grad_()
    v = torch.cat([st, xt.permute(0, 2, 1)], dim=2)  # ring as left context, no padding
    pre = torch.nn.functional.conv1d(v, wt[:, None, :], bt_, groups=x.shape[2])
    y = torch.nn.functional.silu(pre).permute(0, 2, 1)
    (y * torch.from_numpy(dy)).sum().backward()
    g = oracle.conv_bwd(x, w, b, dy, s0)
    np.testing.assert_allclose(g["dx"], xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dw"], wt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dbias"], bt_.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["ds0"], st.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_no_ring_gradient_is_zero_context():
    """Without an initial ring the context is zero: the same as a zero ring."""
    x, w, b, _, dy = _inputs(k=4, ring=False)
    z = np.zeros((x.shape[0], x.shape[2], 3))
    a, c = oracle.conv_bwd(x, w, b, dy), oracle.conv_bwd(x, w, b, dy, z)
    for n in ("dx", "dw", "dbias"):
        np.testing.assert_array_equal(a[n], c[n])
