"""The library orders all its work on the caller's stream and allocates nothing
inside a call, so its entry points run on any stream and can be captured into a
HIP graph.  Checked here: results on a side stream equal the default stream's,
and a captured forward + backward (scan and conv1d) replayed several times, with
eager work and synchronisation between the replays, reproduces the eager results
bit for bit on every replay.  (No kernel of the library records a memset.)
"""
import numpy as np
import pytest
import torch

import workloads as W

ssm = pytest.importorskip("selective_state_space_04_amd")

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


# (2, 1000, 384): the chunked forward; (2, 1000, 4096): one lane per state
SCAN_SHAPES = [(2, 1000, 384), (2, 1000, 4096)]


def _scan_inputs(io=torch.bfloat16, shape=SCAN_SHAPES[0]):
    inp = W.make_inputs(*shape, seed=61, bf16=io == torch.bfloat16)
    return {k: torch.from_numpy(v).to(DEV).to(io if k in ("x", "z", "dt", "B", "C", "dy") else torch.float32)
            for k, v in inp.items() if v is not None}


def _scan_step(t, y, g, stream=None):
    _, _, ck = ssm.ssm_scan_fwd(t["x"], t["dt"], t["B"], t["C"], t["z"], t["A_log"], t["D"], t["dt_bias"],
                                training=True, y=y, stream=stream)
    ssm.ssm_scan_bwd(t["x"], t["dt"], t["B"], t["C"], t["z"], t["A_log"], t["D"], t["dt_bias"], ck, t["dy"],
                     out=g, stream=stream)


def _fresh_grads(t):
    return {"dx": torch.empty_like(t["x"]), "ddt": torch.empty_like(t["x"]), "dz": torch.empty_like(t["x"]),
            "dB": torch.empty_like(t["B"]), "dC": torch.empty_like(t["C"]), "dA_log": torch.empty_like(t["A_log"]),
            "dD": torch.empty_like(t["D"]), "ddt_bias": torch.empty_like(t["dt_bias"]), "dh0": None}


def _same(a, b):
    return all(torch.equal(a[k], b[k]) for k in a if a[k] is not None)


@pytest.mark.parametrize("shape", SCAN_SHAPES)
def test_scan_on_a_side_stream_matches_default_stream(shape):
    t = _scan_inputs(shape=shape)
    y0, g0 = torch.empty_like(t["x"]), _fresh_grads(t)
    _scan_step(t, y0, g0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    y1, g1 = torch.empty_like(t["x"]), _fresh_grads(t)
    with torch.cuda.stream(s):
        _scan_step(t, y1, g1, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and _same(g0, g1)


@pytest.mark.parametrize("shape", SCAN_SHAPES)
def test_explicit_stream_without_entering_its_context(shape):
    """stream= passed while another stream is current: the workspace, checkpoints
    and outputs the binding allocates must belong to the launch stream, so that
    allocations made meanwhile on the current stream cannot reuse them while the
    kernels still run.  Busy work on the side stream keeps the kernels in flight
    while the current stream allocates and fills fresh memory."""
    t = _scan_inputs(shape=shape)
    y0, g0 = torch.empty_like(t["x"]), _fresh_grads(t)
    _scan_step(t, y0, g0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        spin = torch.ones(1 << 24, device=DEV)
        for _ in range(20):
            spin.mul_(1.0000001)           # keeps s busy before the scan's kernels
    y1, ck = ssm.ssm_scan_fwd(t["x"], t["dt"], t["B"], t["C"], t["z"], t["A_log"], t["D"], t["dt_bias"],
                              training=True, stream=s)[0::2]
    g1 = ssm.ssm_scan_bwd(t["x"], t["dt"], t["B"], t["C"], t["z"], t["A_log"], t["D"], t["dt_bias"], ck,
                          t["dy"], stream=s)
    for _ in range(8):                     # the current stream allocates and scribbles meanwhile
        junk = torch.empty(1 << 22, dtype=torch.uint8, device=DEV)
        junk.fill_(0xFF)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and _same(g0, g1)


@pytest.mark.parametrize("shape", SCAN_SHAPES)
def test_scan_fwd_bwd_graph_replays_equal_eager(shape):
    t = _scan_inputs(shape=shape)
    y_ref, g_ref = torch.empty_like(t["x"]), _fresh_grads(t)
    _scan_step(t, y_ref, g_ref)
    torch.cuda.synchronize()
    y, g = torch.empty_like(t["x"]), _fresh_grads(t)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _scan_step(t, y, g)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _scan_step(t, y, g)
    for _ in range(3):
        y.fill_(7.0)                                  # eager work between the replays
        for v in g.values():
            if v is not None:
                v.fill_(-3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and _same(g, g_ref)


def test_conv_fwd_bwd_graph_replays_equal_eager():
    ci = W.make_conv_inputs(2, 700, 256, 4, seed=62, bf16=True, with_ring=True)
    c = {k: torch.from_numpy(v).to(DEV).to(torch.bfloat16 if k in ("x", "dy") else torch.float32)
         for k, v in ci.items()}

    def run(y, ring, g):
        ssm.ssm_conv1d_fwd(c["x"], c["w"], c["bias"], c["ring0"], y=y)
        ssm.ssm_conv1d_bwd(c["x"], c["w"], c["bias"], c["dy"], c["ring0"], want_dring0=True, out=g)

    def fresh():
        return {"dx": torch.empty_like(c["x"]), "dw": torch.empty_like(c["w"]), "dbias": torch.empty_like(c["bias"]),
                "dring0": torch.empty_like(c["ring0"])}

    y_ref, g_ref = torch.empty_like(c["x"]), fresh()
    run(y_ref, None, g_ref)
    torch.cuda.synchronize()
    y, g = torch.empty_like(c["x"]), fresh()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(y, None, g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(y, None, g)
    for _ in range(3):
        y.zero_()
        for v in g.values():
            v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and _same(g, g_ref)
