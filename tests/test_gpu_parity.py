"""GPU parity of the HIP selective scan against the f64 oracle.

Pass criterion per output tensor (max relative error):
    max_i |gpu_i - oracle_i| <= rtol * max_i |oracle_i|
with rtol = 1e-5 for the f32 forward, 1e-4 for f32 gradients and 2e-2 for
every output of the bf16-I/O workload (bf16 storage alone is 2^-9 relative).
These are the tolerances of the rustytorch commit log's CUDA-vs-CPU gradient
check (1e-4) and of the scan's stated f32/bf16 accuracy.

Covers the five workloads (tiny f32, Mamba-130M-shaped f32 fwd and fwd+bwd,
Mamba-2.8B-shaped bf16 fwd+bwd, 1024 decode steps) and guard shapes: long
memory (128 chunks), random A_log, ragged lengths/channels, split invariance,
determinism, delta -> 0, delta = 100, constant inputs, no gate / no D / no
bias / h0 / dh0, seqlen 0, and the one-lane-per-state forward used at widths
of 8192 to 262143 batch rows x channels.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

ssm = pytest.importorskip("selective_state_space_04_amd")

pytestmark = pytest.mark.gpu

F32_FWD = 1e-5
F32_GRAD = 1e-4
BF16_TOL = 2e-2
DEV = torch.device("cuda:0")
GRADS = ("dx", "ddt", "dz", "dB", "dC", "dA_log", "dD", "ddt_bias")


def _t(a, io=torch.float32):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(io)


def _np(t):
    return t.detach().to(torch.float64).cpu().numpy()


def _rel(g, o):
    g = _np(g) if isinstance(g, torch.Tensor) else g
    return float(np.max(np.abs(g - o)) / max(float(np.max(np.abs(o))), 1e-30))


def _gpu_fwd_bwd(inp, io=torch.float32, h0=None, want_dh0=False, bwd=True):
    t = {k: _t(inp[k], io if k in ("x", "z", "dt", "B", "C", "dy") else torch.float32)
         for k in ("x", "z", "dt", "B", "C", "dy", "A_log", "D", "dt_bias") if k in inp}
    h0t = _t(h0) if h0 is not None else None
    y, h_last, ckpt = ssm.ssm_scan_fwd(t["x"], t["dt"], t["B"], t["C"], t.get("z"), t["A_log"], t.get("D"),
                                       t.get("dt_bias"), h0t, training=bwd, return_last_state=True)
    g = None
    if bwd:
        g = ssm.ssm_scan_bwd(t["x"], t["dt"], t["B"], t["C"], t.get("z"), t["A_log"], t.get("D"),
                             t.get("dt_bias"), ckpt, t["dy"], h0t, want_dh0=want_dh0)
    torch.cuda.synchronize()
    return y, h_last, g


def _check_all(inp, io=torch.float32, h0=None, fwd_tol=F32_FWD, grad_tol=F32_GRAD, bwd=True,
               want_dh0=False):
    y, h_last, g = _gpu_fwd_bwd(inp, io, h0, want_dh0, bwd)
    ref = oracle.fwd(inp["x"], inp["dt"], inp["B"], inp["C"], inp.get("z"), inp["A_log"], inp.get("D"),
                     inp.get("dt_bias"), h0)
    errs = {"y": _rel(y, ref["y"]), "h_last": _rel(h_last, ref["h_last"])}
    assert errs["y"] <= fwd_tol, errs
    assert errs["h_last"] <= fwd_tol, errs
    if bwd:
        gr = oracle.bwd(inp["x"], inp["dt"], inp["B"], inp["C"], inp.get("z"), inp["A_log"], inp.get("D"),
                        inp.get("dt_bias"), inp["dy"], h0)
        for k in GRADS + (("dh0",) if want_dh0 else ()):
            if gr[k] is None or g[k] is None:
                continue
            errs[k] = _rel(g[k], gr[k])
        bad = {k: v for k, v in errs.items() if k not in ("y", "h_last") and v > grad_tol}
        assert not bad, errs
    return errs


# ------------------------------------------------------------------ workloads

def test_c1_tiny_fwd_bwd():
    inp = W.make_config("c1_tiny")
    _check_all(inp, want_dh0=True)


def test_c2_mamba130m_fwd_full():
    inp = W.make_config("c2_mamba130m_fwd")
    _check_all(inp, bwd=False)


@pytest.mark.timeout(300)
def test_c3_mamba130m_fwd_bwd_full():
    inp = W.make_config("c3_mamba130m_fwdbwd")
    _check_all(inp)


@pytest.mark.timeout(300)
def test_c3_full_length_fd_spot_check():
    """GPU gradients at sampled coordinates against f64 central differences of
    the oracle's loss sum(dy*y), evaluated on the channels each coordinate reaches."""
    inp = W.make_config("c3_mamba130m_fwdbwd")
    _, _, g = _gpu_fwd_bwd(inp)
    rng = np.random.default_rng(123)
    bsz, L, D = inp["x"].shape
    eps = 1e-6

    def loss(sl_b, sl_d, mod):
        sub = {k: inp[k][sl_b][:, :, sl_d] for k in ("x", "z", "dt", "dy")}
        sub.update({k: inp[k][sl_b] for k in ("B", "C")})
        sub.update({"A_log": inp["A_log"][sl_d], "D": inp["D"][sl_d], "dt_bias": inp["dt_bias"][sl_d]})
        sub = {k: v.astype(np.float64) for k, v in sub.items()}
        mod(sub)
        y = oracle.fwd(sub["x"], sub["dt"], sub["B"], sub["C"], sub["z"], sub["A_log"], sub["D"],
                       sub["dt_bias"])["y"]
        return float((y * sub["dy"]).sum())

    cases = []
    for name in ("x", "z", "dt"):
        for _ in range(8):
            b, t, d = rng.integers(bsz), rng.integers(L), rng.integers(D)
            cases.append((name, (b, t, d), slice(b, b + 1), slice(d, d + 1), (0, t, 0)))
    for name in ("B", "C"):
        for _ in range(8):
            b, t, n = rng.integers(bsz), rng.integers(L), rng.integers(16)
            cases.append((name, (b, t, n), slice(b, b + 1), slice(0, D), (0, t, n)))
    for name in ("A_log",):
        for _ in range(8):
            d, n = rng.integers(D), rng.integers(16)
            cases.append((name, (d, n), slice(0, bsz), slice(d, d + 1), (0, n)))
    for name in ("D", "dt_bias"):
        for _ in range(8):
            d = rng.integers(D)
            cases.append((name, (d,), slice(0, bsz), slice(d, d + 1), (0,)))
    gname = {"x": "dx", "z": "dz", "dt": "ddt", "B": "dB", "C": "dC", "A_log": "dA_log", "D": "dD",
             "dt_bias": "ddt_bias"}
    scale = {k: float(torch.max(torch.abs(g[v])).item()) for k, v in gname.items()}
    for name, full_idx, sb, sd, loc in cases:
        def plus(s, name=name, loc=loc):
            s[name][loc] += eps

        def minus(s, name=name, loc=loc):
            s[name][loc] -= eps
        fd = (loss(sb, sd, plus) - loss(sb, sd, minus)) / (2 * eps)
        got = float(g[gname[name]][full_idx].item())
        assert abs(got - fd) <= F32_GRAD * scale[name], (name, full_idx, got, fd)


def _rel_rows(g, o):
    """max|g - o| / max|o| over a [batch, ...] tensor, one batch row at a time
    (bounds host memory at the full-size workloads)."""
    num = den = 0.0
    for i in range(o.shape[0]):
        gi = _np(g[i]) if isinstance(g, torch.Tensor) else np.asarray(g[i], dtype=np.float64)
        num = max(num, float(np.max(np.abs(gi - o[i]))))
        den = max(den, float(np.max(np.abs(o[i]))))
    return num / max(den, 1e-30)


@pytest.mark.timeout(600)
def test_c4_mamba2p8b_bf16_full():
    """bf16 I/O at full size (batch 4 x 8192 x 5120): every element of every
    output and gradient against the f64 oracle run on the same bf16 values --
    y, h_last, dx, ddt, dz, dB, dC on all four batch rows and dA_log, dD,
    ddt_bias on all 5120 channels.  This covers the multi-block dB/dC partials
    of every batch row and the parameter partials of every (row, chunk)."""
    inp = W.make_config("c4_mamba2p8b_bf16")
    y, h_last, g = _gpu_fwd_bwd(inp, io=torch.bfloat16)
    args = [inp[k] for k in ("x", "dt", "B", "C", "z", "A_log", "D", "dt_bias")]
    ref = oracle.fwd(*args)
    errs = {"y": _rel_rows(y, ref["y"]), "h_last": _rel_rows(h_last, ref["h_last"])}
    del ref
    gr = oracle.bwd(*args, inp["dy"])
    for k in ("dx", "ddt", "dz", "dB", "dC"):
        errs[k] = _rel_rows(g[k], gr[k])
    for k in ("dA_log", "dD", "ddt_bias"):
        errs[k] = _rel(g[k], gr[k])
    print("c4 max rel errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    assert all(v <= BF16_TOL for v in errs.values()), errs


@pytest.mark.timeout(600)
def test_c5_decode_steps_equal_forward():
    """1024 single-token steps from a zero state at batch 256 x d_inner 5120:
    bit-identical to the full-sequence forward (which runs its sequence in one
    chunk at this width), and every y and final state of all 256 batch rows
    within 1e-5 of the oracle (run 32 rows at a time to bound host memory)."""
    c = W.CONFIGS["c5_decode_step"]
    inp = W.make_config("c5_decode_step", with_dy=False)
    bsz, L, D = inp["x"].shape
    assert ssm.fwd_workspace_bytes(bsz, L, D) == 0  # single chunk: sequential order
    x, z, dt = (_t(inp[k]) for k in ("x", "z", "dt"))
    Bm, Cm = _t(inp["B"]), _t(inp["C"])
    A_log, Dp, bias = _t(inp["A_log"]), _t(inp["D"]), _t(inp["dt_bias"])
    y_full, h_full, _ = ssm.ssm_scan_fwd(x, dt, Bm, Cm, z, A_log, Dp, bias, return_last_state=True)
    # time-major copies so each step reads dense [batch, d_inner] slices
    xt, zt, dtt = (v.transpose(0, 1).contiguous() for v in (x, z, dt))
    Bt_, Ct_ = Bm.transpose(0, 1).contiguous(), Cm.transpose(0, 1).contiguous()
    del x, z, dt
    h = torch.zeros(bsz, D, 16, dtype=torch.float32, device=DEV)
    ys = torch.empty(L, bsz, D, dtype=torch.float32, device=DEV)
    for t in range(L):
        ssm.ssm_scan_step(h, xt[t], dtt[t], Bt_[t], Ct_[t], zt[t], A_log, Dp, bias, y=ys[t])
    torch.cuda.synchronize()
    del xt, zt, dtt, Bt_, Ct_
    assert torch.equal(ys.transpose(0, 1), y_full)
    assert torch.equal(h, h_full)
    del ys
    num_y = den_y = num_h = den_h = 0.0
    for r0 in range(0, bsz, 32):
        rows = slice(r0, min(r0 + 32, bsz))
        ref = oracle.fwd(inp["x"][rows], inp["dt"][rows], inp["B"][rows], inp["C"][rows], inp["z"][rows],
                         inp["A_log"], inp["D"], inp["dt_bias"])
        for i in range(rows.stop - rows.start):
            gy = _np(y_full[r0 + i])
            num_y = max(num_y, float(np.max(np.abs(gy - ref["y"][i]))))
            den_y = max(den_y, float(np.max(np.abs(ref["y"][i]))))
        gh = _np(h[rows])
        num_h = max(num_h, float(np.max(np.abs(gh - ref["h_last"]))))
        den_h = max(den_h, float(np.max(np.abs(ref["h_last"]))))
        del ref
    errs = {"y": num_y / den_y, "h": num_h / den_h}
    print("c5 max rel errors (all 256 rows):", {k: f"{v:.2e}" for k, v in errs.items()})
    assert errs["y"] <= F32_FWD and errs["h"] <= F32_FWD, errs
    assert c["batch"] == bsz and c["seqlen"] == L


# --------------------------------------------------------------------- guards

@pytest.mark.timeout(300)
def test_g1_long_memory_many_chunks():
    # |A| <= 0.0146 and delta ~ 0.01: state memory spans the whole 8192 tokens,
    # so every chunk carry matters (128 chunks of 64 tokens here).
    inp = W.make_inputs(2, 8192, 64, dt_bias=W.DT_BIAS_SLOW, a_log=W.a_log_canonical(64, 16, shift=-7.0),
                        seed=11)
    assert ssm.fwd_workspace_bytes(2, 8192, 64) > 0
    _check_all(inp, want_dh0=True)


def test_g2_random_a_log():
    inp = W.make_inputs(2, 700, 96, a_log=W.random_a_log(96, seed=3), seed=12)
    _check_all(inp)


@pytest.mark.parametrize("L", [1, 2, 63, 258, 1000])
@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_g3_ragged(L, io):
    """Sequences whose last 8-token checkpoint block holds 1, 2, 7, 2 and 8 tokens
    (the backward fetches a block's rows clamped into the block, and dy, z two
    tokens ahead)."""
    bf = io == torch.bfloat16
    inp = W.make_inputs(3, L, 100, seed=13 + L, bf16=bf)
    tol = (BF16_TOL, BF16_TOL) if bf else (F32_FWD, F32_GRAD)
    _check_all(inp, io=io, fwd_tol=tol[0], grad_tol=tol[1], want_dh0=True)


def test_g4_split_invariance_prefill_then_continue():
    inp = W.make_inputs(2, 3000, 300, seed=14, dt_bias=W.DT_BIAS_SLOW, with_dy=False)
    t = {k: _t(v) for k, v in inp.items() if v is not None}
    y, h, _ = ssm.ssm_scan_fwd(t["x"], t["dt"], t["B"], t["C"], t["z"], t["A_log"], t["D"], t["dt_bias"],
                               return_last_state=True)
    L1 = 1234
    a = {k: (t[k][:, :L1].contiguous() if k in ("x", "dt", "B", "C", "z") else t[k]) for k in t}
    b = {k: (t[k][:, L1:].contiguous() if k in ("x", "dt", "B", "C", "z") else t[k]) for k in t}
    y1, h1, _ = ssm.ssm_scan_fwd(a["x"], a["dt"], a["B"], a["C"], a["z"], a["A_log"], a["D"], a["dt_bias"],
                                 return_last_state=True)
    y2, h2, _ = ssm.ssm_scan_fwd(b["x"], b["dt"], b["B"], b["C"], b["z"], b["A_log"], b["D"], b["dt_bias"],
                                 h1, return_last_state=True)
    torch.cuda.synchronize()
    yc = torch.cat([y1, y2], 1)
    assert (yc - y).abs().max().item() <= F32_FWD * y.abs().max().item()
    assert (h2 - h).abs().max().item() <= F32_FWD * h.abs().max().item()


def test_g6_bitwise_deterministic():
    inp = W.make_inputs(2, 1500, 700, seed=15)
    y1, h1, g1 = _gpu_fwd_bwd(inp, want_dh0=True)
    y2, h2, g2 = _gpu_fwd_bwd(inp, want_dh0=True)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    for k in GRADS + ("dh0",):
        assert torch.equal(g1[k], g2[k]), k


def test_g7_large_dt_finite():
    inp = W.make_inputs(2, 200, 80, seed=16)
    inp["dt"] = np.full_like(inp["dt"], 100.0)
    y, h, g = _gpu_fwd_bwd(inp)
    assert torch.isfinite(y).all() and torch.isfinite(h).all()
    for k in GRADS:
        assert torch.isfinite(g[k]).all(), k
    _check_all(inp)


def test_g8_delta_to_zero_limit():
    inp = W.make_inputs(2, 300, 64, seed=17, dt_bias=-40.0)
    y, h, g = _gpu_fwd_bwd(inp)
    gate = inp["z"] / (1.0 + np.exp(-inp["z"].astype(np.float64)))
    expect = inp["D"][None, None, :] * inp["x"] * gate
    assert _rel(y, expect) <= 1e-6
    assert float(torch.abs(g["dC"]).max()) <= 1e-6
    _check_all(inp)


def test_g9_constant_inputs():
    bsz, L, D = 1, 600, 40
    inp = W.make_inputs(bsz, 1, D, seed=18)
    for k in ("x", "z", "dt", "dy"):
        inp[k] = np.ascontiguousarray(np.broadcast_to(inp[k], (bsz, L, D)))
    for k in ("B", "C"):
        inp[k] = np.ascontiguousarray(np.broadcast_to(inp[k], (bsz, L, 16)))
    inp["A_log"] = W.a_log_canonical(D, 16, shift=-3.0)
    _check_all(inp)


def test_no_gate_no_skip_no_bias_with_h0():
    inp = W.make_inputs(2, 333, 70, seed=19)
    inp["z"] = None
    inp["D"] = None
    inp["dt_bias"] = None
    h0 = np.random.default_rng(5).standard_normal((2, 70, 16)).astype(np.float32)
    _check_all(inp, h0=h0, want_dh0=True)


def test_h0_with_chunked_sequence():
    inp = W.make_inputs(1, 4096, 64, seed=20, dt_bias=W.DT_BIAS_SLOW)
    h0 = np.random.default_rng(6).standard_normal((1, 64, 16)).astype(np.float32)
    assert ssm.fwd_workspace_bytes(1, 4096, 64) > 0
    _check_all(inp, h0=h0, want_dh0=True)


def test_seqlen_zero():
    x = torch.zeros(2, 0, 32, device=DEV)
    bc = torch.zeros(2, 0, 16, device=DEV)
    A_log = _t(W.a_log_canonical(32))
    h0 = torch.randn(2, 32, 16, device=DEV)
    y, h_last, ckpt = ssm.ssm_scan_fwd(x, x, bc, bc, None, A_log, None, None, h0, return_last_state=True,
                                       training=True)
    g = ssm.ssm_scan_bwd(x, x, bc, bc, None, A_log, None, None, ckpt, x, h0, want_dh0=True)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.equal(h_last, h0)
    assert float(g["dA_log"].abs().max()) == 0.0 and float(g["dh0"].abs().max()) == 0.0
    assert float(g["ddt_bias"].abs().max()) == 0.0


def test_step_bf16_matches_forward():
    inp = W.make_inputs(4, 40, 300, seed=21, bf16=True, with_dy=False)
    t = {k: (_t(v, torch.bfloat16) if k in ("x", "z", "dt", "B", "C") else _t(v)) for k, v in inp.items()
         if v is not None}
    y, h, _ = ssm.ssm_scan_fwd(t["x"], t["dt"], t["B"], t["C"], t["z"], t["A_log"], t["D"], t["dt_bias"],
                               return_last_state=True)
    hs = torch.zeros(4, 300, 16, device=DEV)
    ys = []
    for s in range(40):
        sl = {k: t[k][:, s].contiguous() for k in ("x", "z", "dt", "B", "C")}
        ys.append(ssm.ssm_scan_step(hs, sl["x"], sl["dt"], sl["B"], sl["C"], sl["z"], t["A_log"], t["D"],
                                    t["dt_bias"]))
    torch.cuda.synchronize()
    assert torch.equal(torch.stack(ys, 1), y)
    assert torch.equal(hs, h)


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("gate", [True, False])
def test_step_row_groups_match_forward(io, gate):
    """Steps at a width where a wave takes several batch rows in turn: batch 257
    leaves a last group of one row, and d_inner 5100 a partly filled last wave.
    Bit-identical to the forward, which runs this width as one sequential chunk."""
    bf = io == torch.bfloat16
    inp = W.make_inputs(257, 3, 5100, seed=23, bf16=bf, with_dy=False)
    if not gate:
        inp["z"] = None
    t = {k: (_t(v, io) if k in ("x", "z", "dt", "B", "C") else _t(v)) for k, v in inp.items()
         if v is not None}
    z = t.get("z")
    assert ssm.fwd_workspace_bytes(257, 3, 5100, io_dtype=io) == 0  # one sequential chunk
    y, h, _ = ssm.ssm_scan_fwd(t["x"], t["dt"], t["B"], t["C"], z, t["A_log"], t["D"], t["dt_bias"],
                               return_last_state=True)
    hs = torch.zeros(257, 5100, 16, device=DEV)
    ys = []
    for s_ in range(3):
        sl = {k: t[k][:, s_].contiguous() for k in ("x", "dt", "B", "C")}
        zs = z[:, s_].contiguous() if z is not None else None
        ys.append(ssm.ssm_scan_step(hs, sl["x"], sl["dt"], sl["B"], sl["C"], zs, t["A_log"], t["D"],
                                    t["dt_bias"]))
    torch.cuda.synchronize()
    assert torch.equal(torch.stack(ys, 1), y)
    assert torch.equal(hs, h)


# Widths from 8192 up to 262143 batch rows x channels (d_inner a multiple of 16)
# run the forward with one lane per (channel, state) over the whole sequence
# (k_fwd_state, no chunks, no forward workspace); 2 x 4096 below.
@pytest.mark.parametrize("L", [1, 16, 17, 32, 48, 1000])
@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("gate", [True, False])
def test_state_lane_forward(L, io, gate):
    """One-token, whole-tile and ragged sequences (16, 32, 48 = one, two, three
    16-token tiles and no partial one; 17 = one tile and one token; 1000 = 62
    tiles and 8 tokens), with h0; with the gate, D and dt_bias, or with none of
    them.  Whole tiles followed by whole tiles advance their row pointers by a
    tile; the last whole tile and a partial one clamp their rows.  The backward
    reads the checkpoints this forward writes."""
    assert ssm.fwd_workspace_bytes(2, L, 4096, io_dtype=io) == 0
    inp = W.make_inputs(2, L, 4096, seed=31 + L, bf16=io == torch.bfloat16)
    if not gate:
        inp["z"] = None
        inp["D"] = None
        inp["dt_bias"] = None
    h0 = (0.5 * np.random.default_rng(7).standard_normal((2, 4096, 16))).astype(np.float32)
    tol = (F32_FWD, F32_GRAD) if io == torch.float32 else (BF16_TOL, BF16_TOL)
    _check_all(inp, io=io, h0=h0, fwd_tol=tol[0], grad_tol=tol[1], want_dh0=True)


def test_state_lane_inference_equals_training_forward():
    """Without checkpoints (inference) the same kernel computes the same bits."""
    inp = W.make_inputs(2, 300, 4096, seed=41, with_dy=False)
    t = {k: _t(v) for k, v in inp.items()}
    args = (t["x"], t["dt"], t["B"], t["C"], t["z"], t["A_log"], t["D"], t["dt_bias"])
    y1, h1, ck = ssm.ssm_scan_fwd(*args, training=True, return_last_state=True)
    y2, h2, _ = ssm.ssm_scan_fwd(*args, training=False, return_last_state=True)
    torch.cuda.synchronize()
    assert ck is not None
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_state_lane_states_match_step_chain():
    """Each state goes through the same operations as in the single-token step:
    after 40 tokens the states agree bit for bit.  The readout sums the 16
    states in butterfly order rather than state order, so y agrees to
    rounding."""
    inp = W.make_inputs(2, 40, 4096, seed=43, with_dy=False)
    t = {k: _t(v) for k, v in inp.items()}
    y, h, _ = ssm.ssm_scan_fwd(t["x"], t["dt"], t["B"], t["C"], t["z"], t["A_log"], t["D"], t["dt_bias"],
                               return_last_state=True)
    hs = torch.zeros(2, 4096, 16, device=DEV)
    ys = []
    for s_ in range(40):
        sl = {k: t[k][:, s_].contiguous() for k in ("x", "dt", "B", "C", "z")}
        ys.append(ssm.ssm_scan_step(hs, sl["x"], sl["dt"], sl["B"], sl["C"], sl["z"], t["A_log"], t["D"],
                                    t["dt_bias"]))
    torch.cuda.synchronize()
    assert torch.equal(hs, h)
    assert _rel(torch.stack(ys, 1), _np(y)) <= 1e-6


def test_state_lane_bf16_is_nearest_even_of_f32():
    """bf16 I/O on the lane-per-state forward: the stored y is the nearest-even
    rounding of the f32-I/O result, bit for bit."""
    inp = W.make_inputs(2, 100, 4096, seed=44, bf16=True, with_dy=False)
    y32, _, _ = _gpu_fwd_bwd(inp, io=torch.float32, bwd=False)
    y16, _, _ = _gpu_fwd_bwd(inp, io=torch.bfloat16, bwd=False)
    assert torch.equal(y16, y32.to(torch.bfloat16))


@pytest.mark.parametrize("L", [3, 17])
def test_state_lane_forward_many_batch_rows(L):
    """16383 batch rows x 16 channels (262128 lanes' worth, the widest the
    lane-per-state forward takes): a grid of 16383 rows of workgroups, one
    16-channel block each, with whole and partial tiles; the backward reads the
    checkpoints they write."""
    inp = W.make_inputs(16383, L, 16, seed=46 + L)
    assert ssm.fwd_workspace_bytes(16383, L, 16) == 0
    _check_all(inp, want_dh0=True)


def test_long_sequence_forwards_agree():
    """From 16384 tokens a forward that writes checkpoints takes the chunked form
    (the lane-per-state forward's checkpoint stores fall behind there), while
    inference keeps one lane per state: both must give the same y and h_last to
    rounding (they sum in different orders)."""
    assert ssm.fwd_workspace_bytes(1, 16400, 8192) > 0  # training: chunked
    inp = W.make_inputs(1, 16400, 8192, seed=45, with_dy=False, dt_bias=W.DT_BIAS_SLOW)
    t = {k: _t(v) for k, v in inp.items()}
    args = (t["x"], t["dt"], t["B"], t["C"], t["z"], t["A_log"], t["D"], t["dt_bias"])
    y_tr, h_tr, ck = ssm.ssm_scan_fwd(*args, training=True, return_last_state=True)
    y_in, h_in, _ = ssm.ssm_scan_fwd(*args, training=False, return_last_state=True)
    torch.cuda.synchronize()
    assert ck is not None
    assert _rel(y_in, _np(y_tr)) <= 1e-5
    assert _rel(h_in, _np(h_tr)) <= 1e-5


def test_bf16_outputs_are_nearest_even_roundings_of_the_f32_path():
    """With bf16-representable inputs the bf16-I/O kernels do the same f32
    arithmetic as the f32-I/O kernels; every stored bf16 output must be the
    round-to-nearest-even of the corresponding f32 result, bit for bit."""
    inp = W.make_inputs(2, 300, 200, seed=22, bf16=True)
    y32, _, g32 = _gpu_fwd_bwd(inp, io=torch.float32)
    y16, _, g16 = _gpu_fwd_bwd(inp, io=torch.bfloat16)
    assert torch.equal(y16, y32.to(torch.bfloat16))
    for k in ("dx", "ddt", "dz", "dB", "dC"):
        assert torch.equal(g16[k], g32[k].to(torch.bfloat16)), k
    for k in ("dA_log", "dD", "ddt_bias"):
        assert torch.equal(g16[k], g32[k]), k


def test_max_chunk_count_long_sequence():
    """2^18 tokens on 64 channels: the chunk planner reaches its largest chunk
    counts (thousands of chunks in both directions), with slow decay so that
    every carry is visible in the outputs."""
    inp = W.make_inputs(1, 1 << 18, 64, dt_bias=W.DT_BIAS_SLOW, a_log=W.a_log_canonical(64, 16, shift=-4.0),
                        seed=31)
    _check_all(inp, want_dh0=True)


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_max_batch(io):
    """batch 65535 (the largest grid dimension the launches use) on a short
    sequence and few channels."""
    bf = io == torch.bfloat16
    inp = W.make_inputs(65535, 3, 4, seed=32, bf16=bf)
    tol = (BF16_TOL, BF16_TOL) if bf else (F32_FWD, F32_GRAD)
    _check_all(inp, io=io, fwd_tol=tol[0], grad_tol=tol[1], want_dh0=True)
