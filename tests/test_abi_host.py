"""Host-side checks of the C ABI (no GPU needed, nothing is launched):
the library loads, exports every function include/ssm_scan.h,
include/ssm_conv1d.h and include/ssm_gdn2.h declare, and rejects bad arguments
with the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("ssm_scan.h", "ssm_conv1d.h", "ssm_gdn2.h")]
BLOCK_HEADER = os.path.join(ROOT, "include", "ssm_block.h")

ssm = pytest.importorskip("selective_state_space_04_amd")
lib = ssm.library()

OK, NULLPTR, SHAPE, DTYPE, ALIGN, WORKSPACE, LAUNCH, UNSUPPORTED = range(8)


def _declared_functions(headers=HEADERS):
    names = set()
    for h in headers:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(ssm_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_header_exports_present():
    names = _declared_functions()
    assert {"ssm_scan_fwd", "ssm_scan_bwd", "ssm_scan_step", "ssm_scan_ckpt_bytes",
            "ssm_scan_fwd_workspace_bytes", "ssm_scan_bwd_workspace_bytes", "ssm_status_str",
            "ssm_kernel_name", "ssm_conv1d_fwd", "ssm_conv1d_bwd", "ssm_conv1d_step",
            "ssm_conv1d_bwd_workspace_bytes", "ssm_gdn2_fwd"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in a header but not exported"


def test_block_header_exports_present():
    blib = ssm.block_library()
    names = _declared_functions([BLOCK_HEADER])
    assert {"ssm_block_create", "ssm_block_destroy", "ssm_block_fwd", "ssm_block_bwd", "ssm_block_saved_bytes",
            "ssm_block_fwd_workspace_bytes", "ssm_block_fwd_training_workspace_bytes",
            "ssm_block_bwd_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(blib, n), f"{n} declared in ssm_block.h but not exported by libssmblock.so"


def test_kernel_names():
    names = [ssm.kernel_name(i) for i in range(1, 23)]
    assert "?" not in names and len(set(names)) == 22
    assert ssm.kernel_name(99) == "?"


def test_status_strings():
    for code in range(8):
        assert ssm.status_str(code)
    assert ssm.status_str(99) == "unknown status"


def _dims(b=2, L=64, d=32, n=16, io=0):
    return ssm.SsmDims(b, L, d, n, io)


def test_query_sizes():
    d = _dims(2, 64, 32)
    assert lib.ssm_scan_ckpt_bytes(ctypes.byref(d)) == 4 * 2 * 8 * 32 * 16  # state every 8 tokens
    assert lib.ssm_scan_fwd_workspace_bytes(ctypes.byref(d)) == 0          # one chunk: no carries
    assert lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(d)) > 0
    for bad in (_dims(0), _dims(L=-1), _dims(d=0), _dims(n=8), _dims(io=5)):
        assert lib.ssm_scan_ckpt_bytes(ctypes.byref(bad)) == 0
        assert lib.ssm_scan_fwd_workspace_bytes(ctypes.byref(bad)) == 0
    big = _dims(2, 4096, 1536)
    assert lib.ssm_scan_fwd_workspace_bytes(ctypes.byref(big)) > 0       # chunked sequence
    lanes = _dims(8, 2048, 1536)
    assert lib.ssm_scan_fwd_workspace_bytes(ctypes.byref(lanes)) == 0     # one lane per state, no chunks


def test_size_queries_on_valid_dims_of_every_planner_regime():
    """The chunk planner runs on every valid shape: empty, one-token and short
    sequences, widths below and above each regime's bounds.  A planner bug such
    as a zero chunk length for an empty sequence would end the process here."""
    for b in (1, 2, 3, 64, 300):
        for L in (0, 1, 2, 7, 8, 9, 15, 16, 17, 63, 64, 65, 127, 128, 129, 511, 512, 513, 4096, 16384):
            for d in (1, 16, 33, 256, 1536, 5120):
                dm = _dims(b, L, d)
                lib.ssm_scan_fwd_workspace_bytes(ctypes.byref(dm))
                lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(dm))
                assert lib.ssm_scan_ckpt_bytes(ctypes.byref(dm)) == 4 * b * ((L + 7) // 8) * d * 16


FAKE = 1 << 20  # 16-byte aligned non-null fake device address: never dereferenced


def _fwd(dims, **over):
    a = dict(x=FAKE, dt=FAKE, B=FAKE, C=FAKE, z=None, A_log=FAKE, D=None, dt_bias=None, h0=None,
             y=FAKE, h_last=None, ckpt=None, ws=None, ws_bytes=0)
    a.update(over)
    P = ctypes.c_void_p
    return lib.ssm_scan_fwd(ctypes.byref(dims) if dims is not None else None,
                            *[P(a[k]) if a[k] else None for k in
                              ("x", "dt", "B", "C", "z", "A_log", "D", "dt_bias", "h0", "y", "h_last", "ckpt", "ws")],
                            a["ws_bytes"], None, None)


def test_fwd_rejects_bad_arguments():
    assert _fwd(None) == NULLPTR
    assert _fwd(_dims(0)) == SHAPE
    assert _fwd(_dims(d=0)) == SHAPE
    assert _fwd(_dims(n=8)) == UNSUPPORTED
    assert _fwd(_dims(b=70000)) == UNSUPPORTED
    assert _fwd(_dims(io=2)) == DTYPE
    assert _fwd(_dims(), x=None) == NULLPTR
    assert _fwd(_dims(), A_log=None) == NULLPTR
    assert _fwd(_dims(), y=None) == NULLPTR
    assert _fwd(_dims(), dt=FAKE + 4) == ALIGN
    assert _fwd(_dims(), z=FAKE + 2) == ALIGN
    big = _dims(2, 4096, 1536)  # chunked: needs a workspace
    need = lib.ssm_scan_fwd_workspace_bytes(ctypes.byref(big))
    assert _fwd(big) == WORKSPACE
    assert _fwd(big, ws=FAKE, ws_bytes=need - 1) == WORKSPACE


def _bwd(dims, **over):
    a = dict(x=FAKE, dt=FAKE, B=FAKE, C=FAKE, z=None, A_log=FAKE, D=None, dt_bias=None, h0=None,
             ckpt=FAKE, dy=FAKE, dx=FAKE, ddt=FAKE, dB=FAKE, dC=FAKE, dz=None, dA_log=FAKE, dD=None,
             ddt_bias=FAKE, dh0=None, ws=None, ws_bytes=0)
    a.update(over)
    P = ctypes.c_void_p
    keys = ("x", "dt", "B", "C", "z", "A_log", "D", "dt_bias", "h0", "ckpt", "dy", "dx", "ddt", "dB",
            "dC", "dz", "dA_log", "dD", "ddt_bias", "dh0", "ws")
    return lib.ssm_scan_bwd(ctypes.byref(dims), *[P(a[k]) if a[k] else None for k in keys],
                            a["ws_bytes"], None, None)


def test_bwd_rejects_bad_arguments():
    d = _dims()
    assert _bwd(_dims(n=32)) == UNSUPPORTED
    assert _bwd(d, ckpt=None) == NULLPTR
    assert _bwd(d, dy=None) == NULLPTR
    assert _bwd(d, z=FAKE) == NULLPTR            # gate given but no dz output
    assert _bwd(d, D=FAKE) == NULLPTR            # D given but no dD output
    assert _bwd(d, dA_log=None) == NULLPTR
    assert _bwd(d, dB=FAKE + 8) == ALIGN
    need = lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert _bwd(d) == WORKSPACE
    assert _bwd(d, ws=FAKE, ws_bytes=need - 256) == WORKSPACE


def test_step_rejects_bad_arguments():
    P = ctypes.c_void_p

    def step(b=4, d=32, n=16, io=0, **over):
        a = dict(h=FAKE, x=FAKE, dt=FAKE, B=FAKE, C=FAKE, z=None, A_log=FAKE, D=None, dt_bias=None, y=FAKE)
        a.update(over)
        keys = ("h", "x", "dt", "B", "C", "z", "A_log", "D", "dt_bias", "y")
        return lib.ssm_scan_step(b, d, n, io, *[P(a[k]) if a[k] else None for k in keys], None, None)

    assert step(b=0) == SHAPE
    assert step(n=4) == UNSUPPORTED
    assert step(io=7) == DTYPE
    assert step(h=None) == NULLPTR
    assert step(y=None) == NULLPTR
    assert step(x=FAKE + 1) == ALIGN


def test_binding_rejects_strided_and_mistyped_tensors():
    import torch
    x = torch.zeros(2, 8, 4).transpose(0, 1)
    with pytest.raises((ValueError, TypeError)):
        ssm.ssm_scan_fwd(x, x, torch.zeros(8, 2, 16), torch.zeros(8, 2, 16), None,
                         torch.zeros(4, 16), None, None)
    x = torch.zeros(2, 8, 4, dtype=torch.float64)
    b = torch.zeros(2, 8, 16, dtype=torch.float64)
    with pytest.raises(TypeError):
        ssm.ssm_scan_fwd(x, x, b, b, None, torch.zeros(4, 16), None, None)


def _cdims(b=2, L=64, d=32, k=4, io=0):
    return ssm.ConvDims(b, L, d, k, io)


def test_conv_workspace_size():
    # partials: one row of (d_conv + 1) sums per channel per (batch, 256-token block)
    assert lib.ssm_conv1d_bwd_workspace_bytes(ctypes.byref(_cdims(2, 300, 32, 4))) == 4 * 2 * 2 * 32 * 5
    assert lib.ssm_conv1d_bwd_workspace_bytes(ctypes.byref(_cdims(L=0))) == 0
    for bad in (_cdims(b=0), _cdims(d=0), _cdims(k=0), _cdims(k=5), _cdims(io=3), _cdims(L=-1)):
        assert lib.ssm_conv1d_bwd_workspace_bytes(ctypes.byref(bad)) == 0


def test_conv_rejects_bad_arguments():
    P = ctypes.c_void_p

    def fwd(dims, **over):
        a = dict(x=FAKE, w=FAKE, bias=None, ring0=None, y=FAKE, ring_last=None)
        a.update(over)
        keys = ("x", "w", "bias", "ring0", "y", "ring_last")
        return lib.ssm_conv1d_fwd(ctypes.byref(dims) if dims is not None else None,
                                  *[P(a[k]) if a[k] else None for k in keys], None, None)

    def bwd(dims, **over):
        a = dict(x=FAKE, w=FAKE, bias=None, ring0=None, dy=FAKE, dx=FAKE, dw=FAKE, dbias=FAKE,
                 dring0=None, ws=None, ws_bytes=0)
        a.update(over)
        keys = ("x", "w", "bias", "ring0", "dy", "dx", "dw", "dbias", "dring0", "ws")
        return lib.ssm_conv1d_bwd(ctypes.byref(dims), *[P(a[k]) if a[k] else None for k in keys],
                                  a["ws_bytes"], None, None)

    def step(b=4, d=32, k=4, io=0, **over):
        a = dict(ring=FAKE, x=FAKE, w=FAKE, bias=None, y=FAKE)
        a.update(over)
        keys = ("ring", "x", "w", "bias", "y")
        return lib.ssm_conv1d_step(b, d, k, io, *[P(a[k]) if a[k] else None for k in keys], None, None)

    assert fwd(None) == NULLPTR
    assert fwd(_cdims(b=0)) == SHAPE
    assert fwd(_cdims(k=0)) == SHAPE
    assert fwd(_cdims(k=5)) == UNSUPPORTED
    assert fwd(_cdims(b=70000)) == UNSUPPORTED
    assert fwd(_cdims(io=2)) == DTYPE
    assert fwd(_cdims(), x=None) == NULLPTR
    assert fwd(_cdims(), w=None) == NULLPTR
    assert fwd(_cdims(), y=FAKE + 2) == ALIGN
    assert fwd(_cdims(), ring0=FAKE + 4) == ALIGN
    assert fwd(_cdims(), ring0=FAKE, ring_last=FAKE) == UNSUPPORTED  # in-place ring update
    d = _cdims()
    need = lib.ssm_conv1d_bwd_workspace_bytes(ctypes.byref(d))
    assert bwd(d) == WORKSPACE
    assert bwd(d, ws=FAKE, ws_bytes=need - 4) == WORKSPACE
    assert bwd(d, dw=None, ws=FAKE, ws_bytes=need) == NULLPTR
    assert bwd(d, dbias=None, ws=FAKE, ws_bytes=need) == NULLPTR
    assert bwd(d, dy=None, ws=FAKE, ws_bytes=need) == NULLPTR
    assert bwd(d, dx=FAKE + 8, ws=FAKE, ws_bytes=need) == ALIGN
    assert bwd(_cdims(k=9)) == UNSUPPORTED
    assert step(b=0) == SHAPE
    assert step(k=6) == UNSUPPORTED
    assert step(io=4) == DTYPE
    assert step(ring=None) == NULLPTR
    assert step(x=None) == NULLPTR
    assert step(y=FAKE + 2) == ALIGN


def test_conv_binding_rejects_bad_tensors():
    import torch
    x = torch.zeros(2, 8, 4).transpose(0, 1)
    with pytest.raises((ValueError, TypeError)):
        ssm.ssm_conv1d_fwd(x, torch.zeros(2, 4))
    x = torch.zeros(2, 8, 4)
    with pytest.raises(ValueError):
        ssm.ssm_conv1d_fwd(x, torch.zeros(5, 4))             # w rows != d_inner
    with pytest.raises(TypeError):
        ssm.ssm_conv1d_fwd(x, torch.zeros(4, 4, dtype=torch.float64))


def _bdims(b=2, L=64, dm=32, di=64, n=16, r=4, k=4, io=0):
    return ssm.BlockDims(b, L, dm, di, n, r, k, io)


def test_block_sizes():
    blib = ssm.block_library()
    d = _bdims()
    T, di, P = 2 * 64, 64, 4 + 32
    act = T * di * 4
    # xi, z, xc, dt, y_s [T, d_inner], proj [T, dt_rank + 32], dt_low [T, dt_rank], B and
    # C [T, 16], then the scan checkpoints (every piece a multiple of 256 bytes here)
    assert blib.ssm_block_saved_bytes(ctypes.byref(d)) == 5 * act + T * P * 4 + T * 4 * 4 + 2 * T * 16 * 4 + \
        lib.ssm_scan_ckpt_bytes(ctypes.byref(_dims(2, 64, 64)))
    for bad in (_bdims(b=0), _bdims(L=0), _bdims(dm=12), _bdims(di=60), _bdims(n=8), _bdims(k=5),
                _bdims(r=0), _bdims(io=4)):
        assert blib.ssm_block_saved_bytes(ctypes.byref(bad)) == 0
        assert blib.ssm_block_fwd_workspace_bytes(ctypes.byref(bad)) == 0
        assert blib.ssm_block_fwd_training_workspace_bytes(ctypes.byref(bad)) == 0
        assert blib.ssm_block_bwd_workspace_bytes(ctypes.byref(bad)) == 0
    # every workspace leads with 64 MiB for the GEMMs; a training forward needs that
    # and the scan's workspace, an inference forward also room for the intermediates
    gemm = 64 << 20
    scan = lib.ssm_scan_fwd_workspace_bytes(ctypes.byref(_dims(2, 64, 64)))
    assert blib.ssm_block_fwd_training_workspace_bytes(ctypes.byref(d)) == gemm + scan
    assert blib.ssm_block_fwd_workspace_bytes(ctypes.byref(d)) > gemm + scan
    assert blib.ssm_block_bwd_workspace_bytes(ctypes.byref(d)) > gemm


def test_block_rejects_bad_arguments():
    # every call below fails a host-side check before the context is touched,
    # so a fake (never dereferenced) context pointer is enough
    blib = ssm.block_library()
    P = ctypes.c_void_p
    names = ssm.BLOCK_PARAMS

    def params(**over):
        v = {n: FAKE for n in names}
        v["conv_b"] = None
        v.update(over)
        return ssm.BlockParams(*[v[n] for n in names])

    def fwd(dims, ctx=FAKE, X=FAKE, Y=FAKE, ws=None, ws_bytes=0, **over):
        pp = params(**over)
        return blib.ssm_block_fwd(P(ctx) if ctx else None, ctypes.byref(dims) if dims is not None else None,
                                  P(X) if X else None, ctypes.byref(pp), P(Y) if Y else None, None,
                                  P(ws) if ws else None, ws_bytes, None, None)

    def bwd(dims, saved=FAKE, ws=None, ws_bytes=0, **over):
        pp = params()
        gg = ssm.BlockGrads(*[FAKE] * len(names))
        for k, v in over.items():
            setattr(gg, k, v)
        return blib.ssm_block_bwd(P(FAKE), ctypes.byref(dims), P(FAKE), ctypes.byref(pp),
                                  P(saved) if saved else None, P(FAKE), P(FAKE), ctypes.byref(gg),
                                  P(ws) if ws else None, ws_bytes, None, None)

    d = _bdims()
    assert fwd(d, ctx=None) == NULLPTR
    assert fwd(None) == NULLPTR
    assert fwd(_bdims(L=0)) == SHAPE
    assert fwd(_bdims(dm=20)) == SHAPE            # rows must stay 16-byte aligned
    assert fwd(_bdims(io=3)) == DTYPE
    assert fwd(_bdims(n=32)) == UNSUPPORTED
    assert fwd(_bdims(k=6)) == UNSUPPORTED
    assert fwd(d, X=None) == NULLPTR
    assert fwd(d, W_x=None) == NULLPTR
    assert fwd(d, W_in=FAKE + 4) == ALIGN
    assert fwd(d) == WORKSPACE
    need = blib.ssm_block_fwd_workspace_bytes(ctypes.byref(d))
    assert fwd(d, ws=FAKE, ws_bytes=need - 1) == WORKSPACE
    assert bwd(d, saved=None) == NULLPTR
    assert bwd(d, dW_x=None) == NULLPTR
    assert bwd(d, dA_log=FAKE + 8) == ALIGN
    assert bwd(d) == WORKSPACE


def test_gdn2_rejects_bad_arguments():
    P = ctypes.c_void_p

    def call(dims, S0=None, S_last=None, **over):
        v = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, w=FAKE, o=FAKE)
        v.update(over)
        return lib.ssm_gdn2_fwd(ctypes.byref(dims) if dims is not None else None,
                                *[P(v[n]) if v[n] else None for n in ("q", "k", "v", "g", "b", "w")],
                                P(S0) if S0 else None, 1.0, P(v["o"]) if v["o"] else None,
                                P(S_last) if S_last else None, None, None)

    def dims(b=2, h=3, L=8, kd=64, vd=32, io=0):
        return ssm.Gdn2Dims(b, h, L, kd, vd, io)

    assert call(None) == NULLPTR
    assert call(dims(b=0)) == SHAPE
    assert call(dims(L=-1)) == SHAPE
    assert call(dims(vd=0)) == SHAPE
    assert call(dims(io=7)) == DTYPE
    assert call(dims(io=1), q=FAKE + 2) == ALIGN     # bf16 activations, misaligned
    assert call(dims(kd=48)) == UNSUPPORTED         # k_dim in {16, 32, 64, 128}
    assert call(dims(kd=256)) == UNSUPPORTED
    assert call(dims(h=70000)) == UNSUPPORTED
    assert call(dims(), q=None) == NULLPTR
    assert call(dims(), o=None) == NULLPTR
    assert call(dims(), S0=FAKE, S_last=FAKE) == UNSUPPORTED   # in-place state update
    assert call(dims(), w=FAKE + 4) == ALIGN
    assert call(dims(), S_last=FAKE + 8) == ALIGN
    assert call(dims(L=0), q=None, k=None, v=None, g=None, b=None, w=None, o=None) == OK  # nothing to do
