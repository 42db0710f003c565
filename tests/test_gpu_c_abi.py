"""The selective scan through its C ABI from a host program with no Python or
PyTorch in it (tests/c_abi/scan_from_c.cpp, built by the package build): a
training forward and a backward on hipMalloc'd buffers and a stream of its own.
Every output it writes is compared with the f64 oracle on the inputs it
generated, at the f32 tolerances of tests/test_gpu_parity.py (1e-5 forward,
1e-4 gradients, relative to the largest oracle value)."""
import os
import subprocess

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "c_abi", "scan_from_c")


def _read(path):
    with open(path, "rb") as f:
        Bt, L, D, N = np.frombuffer(f.read(32), dtype=np.int64)
        act, bc, st = Bt * L * D, Bt * L * N, Bt * D * N

        def take(n, shape):
            return np.frombuffer(f.read(4 * n), dtype=np.float32).reshape(shape).astype(np.float64)

        a, b, s = (Bt, L, D), (Bt, L, N), (Bt, D, N)
        out = {}
        for name, n, shp in (("x", act, a), ("dt", act, a), ("B", bc, b), ("C", bc, b), ("z", act, a),
                             ("dy", act, a), ("A_log", D * N, (D, N)), ("D", D, (D,)), ("dt_bias", D, (D,)),
                             ("y", act, a), ("h_last", st, s), ("dx", act, a), ("ddt", act, a),
                             ("dz", act, a), ("dB", bc, b), ("dC", bc, b), ("dA_log", D * N, (D, N)),
                             ("dD", D, (D,)), ("ddt_bias", D, (D,))):
            out[name] = take(n, shp)
        assert not f.read(1), "trailing bytes"
    return out


def _rel(g, o):
    return float(np.max(np.abs(g - o)) / max(float(np.max(np.abs(o))), 1e-30))


@pytest.mark.parametrize("shape", [None, (1, 1000, 48), (3, 64, 256)])
def test_scan_from_a_c_program(tmp_path, shape):
    assert os.path.exists(DRIVER), "build the package first (it compiles tests/c_abi/scan_from_c)"
    out = str(tmp_path / "scan.bin")
    args = [DRIVER, out] + ([str(v) for v in shape] if shape else [])
    res = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    r = _read(out)
    names = ("x", "dt", "B", "C", "z", "A_log", "D", "dt_bias")
    ref = oracle.fwd(*[r[n] for n in names])
    gref = oracle.bwd(*[r[n] for n in names], r["dy"])
    assert _rel(r["y"], ref["y"]) <= 1e-5 and _rel(r["h_last"], ref["h_last"]) <= 1e-5
    for n in ("dx", "ddt", "dz", "dB", "dC", "dA_log", "dD", "ddt_bias"):
        assert _rel(r[n], gref[n]) <= 1e-4, (n, _rel(r[n], gref[n]))


BLOCK_DRIVER = os.path.join(ROOT, "tests", "c_abi", "block_from_c")


def test_block_from_a_c_program(tmp_path):
    """One f32 Mamba block (batch 2 x 100 tokens, d_model 64, d_inner 128) through
    libssmblock.so from a C++ program, so its GEMMs run on the system ROCm
    hipBLASLt; every output against the f64 block oracle at 1e-4."""
    from oracle.block import PARAMS, block_bwd, block_fwd

    assert os.path.exists(BLOCK_DRIVER), "build the package first (it compiles tests/c_abi/block_from_c)"
    out = str(tmp_path / "block.bin")
    res = subprocess.run([BLOCK_DRIVER, "check", out], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    with open(out, "rb") as f:
        Bt, L, dm, di, N, R, K = (int(v) for v in np.frombuffer(f.read(56), dtype=np.int64))
        P = R + 2 * N

        def take(*shape):
            n = int(np.prod(shape))
            return np.frombuffer(f.read(4 * n), dtype=np.float32).reshape(shape).astype(np.float64)

        X, dY = take(Bt, L, dm), take(Bt, L, dm)
        p = {"W_in": take(2 * di, dm), "conv_w": take(di, K), "conv_b": take(di), "W_x": take(P, di),
             "W_dt": take(di, R), "dt_bias": take(di), "A_log": take(di, N), "D": take(di), "W_out": take(dm, di)}
        got = {"Y": take(Bt, L, dm), "dX": take(Bt, L, dm)}
        for n in PARAMS:
            got["d" + n] = take(*p[n].shape)
        assert not f.read(1), "trailing bytes"
    ref, gr = block_fwd(X, p), block_bwd(X, p, dY)
    errs = {"Y": _rel(got["Y"], ref["Y"]), "dX": _rel(got["dX"], gr["dX"])}
    errs.update({"d" + n: _rel(got["d" + n], gr["d" + n]) for n in PARAMS})
    assert all(v <= 1e-4 for v in errs.values()), errs
