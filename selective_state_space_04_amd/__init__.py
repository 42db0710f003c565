"""MI355X-native Mamba S6 selective scan.

Thin Python binding of ``libssmscan.so`` (built from ``csrc/ssm_scan.hip`` and
``csrc/ssm_conv1d.hip``): it checks tensors, allocates outputs/workspace through
torch's caching allocator and passes raw device pointers and the current HIP
stream to the C ABI declared in ``include/ssm_scan.h`` and ``include/ssm_conv1d.h``.  Every step of the scan runs in the library's HIP
kernels; there is no other code path.  Importing fails loudly when the library
has not been built (``__graft_entry__.build()``).

Operation (rustytorch commit log, page "crates/training/rtx-transformers/tests",
commits introducing the real S6 forward, its hand-written VJP and
MambaRecurrence::step):
    delta = softplus(dt + dt_bias), A = -exp(A_log)
    h_t   = exp(delta*A) h_{t-1} + delta B_t x_t,   y_t = (C_t.h_t + D x_t) silu(z_t)
and, in front of it, the causal depthwise conv1d + SiLU with its conv ring
(same page: the real-S6-forward commit's in_proj -> conv1d -> SiLU -> x_proj).
"""
import ctypes
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SSM_SCAN_LIB may point at another build of the same library (A/B timing).
LIB_PATH = os.environ.get("SSM_SCAN_LIB") or os.path.join(_HERE, "libssmscan.so")

SSM_F32, SSM_BF16 = 0, 1
D_STATE = 16
TIMING_MAX = 64


class SsmDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("d_inner", ctypes.c_int64), ("d_state", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32)]


class ConvDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("d_inner", ctypes.c_int64), ("d_conv", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32)]


class Gdn2Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("k_dim", ctypes.c_int64), ("v_dim", ctypes.c_int64), ("io_dtype", ctypes.c_int32)]


class SsmTiming(ctypes.Structure):
    _fields_ = [("events", ctypes.c_void_p), ("capacity", ctypes.c_int32),
                ("count", ctypes.c_int32), ("kernel_id", ctypes.c_int32 * TIMING_MAX)]


class SsmError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


def _load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first (python -c "
            f"'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    DP = ctypes.POINTER(SsmDims)
    TP = ctypes.POINTER(SsmTiming)
    lib.ssm_status_str.argtypes = [ctypes.c_int32]
    lib.ssm_status_str.restype = ctypes.c_char_p
    lib.ssm_kernel_name.argtypes = [I32]
    lib.ssm_kernel_name.restype = ctypes.c_char_p
    for fn in ("ssm_scan_ckpt_bytes", "ssm_scan_fwd_workspace_bytes", "ssm_scan_bwd_workspace_bytes"):
        getattr(lib, fn).argtypes = [DP]
        getattr(lib, fn).restype = SZ
    lib.ssm_scan_fwd.argtypes = [DP] + [P] * 12 + [P, SZ, P, TP]
    lib.ssm_scan_fwd.restype = ctypes.c_int
    lib.ssm_scan_bwd.argtypes = [DP] + [P] * 20 + [P, SZ, P, TP]
    lib.ssm_scan_bwd.restype = ctypes.c_int
    lib.ssm_scan_step.argtypes = [I64, I64, I64, I32] + [P] * 10 + [P, TP]
    lib.ssm_scan_step.restype = ctypes.c_int
    CP = ctypes.POINTER(ConvDims)
    lib.ssm_conv1d_bwd_workspace_bytes.argtypes = [CP]
    lib.ssm_conv1d_bwd_workspace_bytes.restype = SZ
    lib.ssm_conv1d_fwd.argtypes = [CP] + [P] * 6 + [P, TP]
    lib.ssm_conv1d_fwd.restype = ctypes.c_int
    lib.ssm_conv1d_bwd.argtypes = [CP] + [P] * 9 + [P, SZ, P, TP]
    lib.ssm_conv1d_bwd.restype = ctypes.c_int
    lib.ssm_conv1d_bwd_noalloc.argtypes = [CP] + [P] * 9 + [P, TP]
    lib.ssm_conv1d_bwd_noalloc.restype = ctypes.c_int
    lib.ssm_conv1d_step.argtypes = [I64, I64, I64, I32] + [P] * 5 + [P, TP]
    lib.ssm_conv1d_step.restype = ctypes.c_int
    lib.ssm_gdn2_fwd.argtypes = [ctypes.POINTER(Gdn2Dims)] + [P] * 7 + [ctypes.c_float, P, P, P, TP]
    lib.ssm_gdn2_fwd.restype = ctypes.c_int
    lib.ssm_gdn2_chunked_workspace_bytes.argtypes = [ctypes.POINTER(Gdn2Dims)]
    lib.ssm_gdn2_chunked_workspace_bytes.restype = SZ
    lib.ssm_gdn2_fwd_chunked.argtypes = [ctypes.POINTER(Gdn2Dims)] + [P] * 7 + [ctypes.c_float, P, P, P, SZ, P, TP]
    lib.ssm_gdn2_fwd_chunked.restype = ctypes.c_int
    return lib


_lib = _load_library()


def library():
    """The loaded ctypes library (for tests that call the C ABI directly)."""
    return _lib


def status_str(code):
    return _lib.ssm_status_str(int(code)).decode()


def kernel_name(kid):
    return _lib.ssm_kernel_name(int(kid)).decode()


def _raise(fn, code):
    if code != 0:
        raise SsmError(fn, code, status_str(code))


def _io_code(dtype):
    if dtype == torch.float32:
        return SSM_F32
    if dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"unsupported io dtype {dtype}: use float32 or bfloat16")


def dims(batch, seqlen, d_inner, d_state=D_STATE, io_dtype=torch.float32):
    return SsmDims(int(batch), int(seqlen), int(d_inner), int(d_state), _io_code(io_dtype))


def ckpt_bytes(batch, seqlen, d_inner, d_state=D_STATE, io_dtype=torch.float32):
    return int(_lib.ssm_scan_ckpt_bytes(ctypes.byref(dims(batch, seqlen, d_inner, d_state, io_dtype))))


def fwd_workspace_bytes(batch, seqlen, d_inner, d_state=D_STATE, io_dtype=torch.float32):
    return int(_lib.ssm_scan_fwd_workspace_bytes(ctypes.byref(dims(batch, seqlen, d_inner, d_state, io_dtype))))


def bwd_workspace_bytes(batch, seqlen, d_inner, d_state=D_STATE, io_dtype=torch.float32):
    return int(_lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(dims(batch, seqlen, d_inner, d_state, io_dtype))))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype, device, required=True):
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    # dense row-major only: strides are never interpreted
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (dense row-major)")


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _timing_ptr(timing):
    return None if timing is None else ctypes.byref(timing.struct)


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _on_stream(fn):
    """Runs an entry point with its `stream` made current while it allocates.

    Workspaces, checkpoints and fresh outputs come from torch's caching
    allocator, which ties each block to the stream current at allocation.  A
    workspace freed when the call returns goes back to that stream's pool, so it
    must be allocated on the stream the kernels run on; otherwise the next
    allocation on the current stream could reuse it while the launched kernels
    still read it.  Outputs returned from a call with an explicit stream belong
    to that stream (use Tensor.record_stream before reading them elsewhere)."""
    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        s = kwargs.get("stream")
        if s is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(s):
            return fn(*args, **kwargs)
    return wrapper


@_on_stream
def ssm_scan_fwd(x, dt, B, C, z, A_log, D, dt_bias, h0=None, *, training=False,
                 return_last_state=False, y=None, stream=None, timing=None):
    """Forward scan.  x, dt, z: [batch, L, d_inner]; B, C: [batch, L, 16] (float32 or
    bfloat16, all the same); A_log [d_inner, 16], D, dt_bias [d_inner] float32; h0
    [batch, d_inner, 16] float32 or None.  Returns (y, h_last or None, ckpt or None);
    ckpt (training=True) is what ssm_scan_bwd needs."""
    dev = x.device
    bsz, L, din = x.shape
    io = x.dtype
    _check(x, "x", (bsz, L, din), io, dev)
    _check(dt, "dt", (bsz, L, din), io, dev)
    _check(B, "B", (bsz, L, D_STATE), io, dev)
    _check(C, "C", (bsz, L, D_STATE), io, dev)
    _check(z, "z", (bsz, L, din), io, dev, required=False)
    _check(A_log, "A_log", (din, D_STATE), torch.float32, dev)
    _check(D, "D", (din,), torch.float32, dev, required=False)
    _check(dt_bias, "dt_bias", (din,), torch.float32, dev, required=False)
    _check(h0, "h0", (bsz, din, D_STATE), torch.float32, dev, required=False)
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", (bsz, L, din), io, dev)
    dm = dims(bsz, L, din, D_STATE, io)
    h_last = torch.empty(bsz, din, D_STATE, dtype=torch.float32, device=dev) if return_last_state else None
    ckpt = None
    if training:
        ckpt = torch.empty(_lib.ssm_scan_ckpt_bytes(ctypes.byref(dm)) // 4, dtype=torch.float32, device=dev)
    nws = _lib.ssm_scan_fwd_workspace_bytes(ctypes.byref(dm))
    ws = _workspace(nws, dev)
    rc = _lib.ssm_scan_fwd(ctypes.byref(dm), _ptr(x), _ptr(dt), _ptr(B), _ptr(C), _ptr(z), _ptr(A_log),
                           _ptr(D), _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_last), _ptr(ckpt),
                           _ptr(ws), nws, _stream(dev, stream), _timing_ptr(timing))
    _raise("ssm_scan_fwd", rc)
    return y, h_last, ckpt


@_on_stream
def ssm_scan_bwd(x, dt, B, C, z, A_log, D, dt_bias, ckpt, dy, h0=None, *, want_dh0=False,
                 stream=None, timing=None, out=None):
    """Backward of ssm_scan_fwd for the loss sum(dy * y).  Returns a dict with dx, ddt,
    dz (None without z), dB, dC (io dtype) and dA_log, dD, ddt_bias, dh0 (float32).
    h0 is shape-checked but not read: the initial state comes from ckpt, which the
    forward wrote from its own h0."""
    dev = x.device
    bsz, L, din = x.shape
    io = x.dtype
    for t, n, shp in ((x, "x", (bsz, L, din)), (dt, "dt", (bsz, L, din)), (B, "B", (bsz, L, D_STATE)),
                      (C, "C", (bsz, L, D_STATE)), (dy, "dy", (bsz, L, din))):
        _check(t, n, shp, io, dev)
    _check(z, "z", (bsz, L, din), io, dev, required=False)
    _check(A_log, "A_log", (din, D_STATE), torch.float32, dev)
    _check(D, "D", (din,), torch.float32, dev, required=False)
    _check(dt_bias, "dt_bias", (din,), torch.float32, dev, required=False)
    _check(h0, "h0", (bsz, din, D_STATE), torch.float32, dev, required=False)
    dm = dims(bsz, L, din, D_STATE, io)
    nck = _lib.ssm_scan_ckpt_bytes(ctypes.byref(dm)) // 4
    _check(ckpt, "ckpt", (nck,), torch.float32, dev)
    g = out if out is not None else {}
    g.setdefault("dx", torch.empty_like(x))
    g.setdefault("ddt", torch.empty_like(x))
    g.setdefault("dz", torch.empty_like(x) if z is not None else None)
    g.setdefault("dB", torch.empty_like(B))
    g.setdefault("dC", torch.empty_like(C))
    g.setdefault("dA_log", torch.empty_like(A_log))
    g.setdefault("dD", torch.empty(din, dtype=torch.float32, device=dev))
    g.setdefault("ddt_bias", torch.empty(din, dtype=torch.float32, device=dev))
    g.setdefault("dh0", torch.empty(bsz, din, D_STATE, dtype=torch.float32, device=dev) if want_dh0 else None)
    nws = _lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(dm))
    ws = _workspace(nws, dev)
    rc = _lib.ssm_scan_bwd(ctypes.byref(dm), _ptr(x), _ptr(dt), _ptr(B), _ptr(C), _ptr(z), _ptr(A_log),
                           _ptr(D), _ptr(dt_bias), _ptr(h0), _ptr(ckpt), _ptr(dy), _ptr(g["dx"]),
                           _ptr(g["ddt"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dz"]), _ptr(g["dA_log"]),
                           _ptr(g["dD"]), _ptr(g["ddt_bias"]), _ptr(g["dh0"]), _ptr(ws), nws,
                           _stream(dev, stream), _timing_ptr(timing))
    _raise("ssm_scan_bwd", rc)
    return g


@_on_stream
def ssm_scan_step(h, x, dt, B, C, z, A_log, D, dt_bias, *, y=None, stream=None, timing=None):
    """One token: h [batch, d_inner, 16] float32 is updated in place; x, dt, z
    [batch, d_inner] and B, C [batch, 16] in the io dtype.  Returns y [batch, d_inner]."""
    dev = x.device
    bsz, din = x.shape
    io = x.dtype
    _check(h, "h", (bsz, din, D_STATE), torch.float32, dev)
    _check(x, "x", (bsz, din), io, dev)
    _check(dt, "dt", (bsz, din), io, dev)
    _check(B, "B", (bsz, D_STATE), io, dev)
    _check(C, "C", (bsz, D_STATE), io, dev)
    _check(z, "z", (bsz, din), io, dev, required=False)
    _check(A_log, "A_log", (din, D_STATE), torch.float32, dev)
    _check(D, "D", (din,), torch.float32, dev, required=False)
    _check(dt_bias, "dt_bias", (din,), torch.float32, dev, required=False)
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", (bsz, din), io, dev)
    rc = _lib.ssm_scan_step(bsz, din, D_STATE, _io_code(io), _ptr(h), _ptr(x), _ptr(dt), _ptr(B), _ptr(C),
                            _ptr(z), _ptr(A_log), _ptr(D), _ptr(dt_bias), _ptr(y), _stream(dev, stream),
                            _timing_ptr(timing))
    _raise("ssm_scan_step", rc)
    return y


def conv_dims(batch, seqlen, d_inner, d_conv, io_dtype=torch.float32):
    return ConvDims(int(batch), int(seqlen), int(d_inner), int(d_conv), _io_code(io_dtype))


def conv1d_bwd_workspace_bytes(batch, seqlen, d_inner, d_conv, io_dtype=torch.float32):
    return int(_lib.ssm_conv1d_bwd_workspace_bytes(ctypes.byref(conv_dims(batch, seqlen, d_inner, d_conv,
                                                                          io_dtype))))


def _ring(t, name, bsz, din, k, dev, required=False):
    if k == 1:
        return None  # width 1: the ring is empty and ignored
    _check(t, name, (bsz, din, k - 1), torch.float32, dev, required=required)
    return t


@_on_stream
def ssm_conv1d_fwd(x, w, bias=None, ring0=None, *, return_ring=False, y=None, stream=None, timing=None):
    """Causal depthwise conv1d + SiLU.  x [batch, L, d_inner] (float32 or bfloat16);
    w [d_inner, d_conv] float32 (PyTorch's [d_inner, 1, d_conv] squeezed); bias
    [d_inner] float32 or None; ring0 [batch, d_inner, d_conv-1] float32: the inputs
    before the sequence (None = zeros).  Returns (y, ring_last or None)."""
    dev = x.device
    bsz, L, din = x.shape
    io = x.dtype
    k = w.shape[1] if w.dim() == 2 else -1
    _check(x, "x", (bsz, L, din), io, dev)
    _check(w, "w", (din, k), torch.float32, dev)
    _check(bias, "bias", (din,), torch.float32, dev, required=False)
    ring0 = _ring(ring0, "ring0", bsz, din, k, dev)
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", (bsz, L, din), io, dev)
    ring_last = torch.empty(bsz, din, k - 1, dtype=torch.float32, device=dev) if return_ring and k > 1 else None
    dm = conv_dims(bsz, L, din, k, io)
    rc = _lib.ssm_conv1d_fwd(ctypes.byref(dm), _ptr(x), _ptr(w), _ptr(bias), _ptr(ring0), _ptr(y),
                             _ptr(ring_last), _stream(dev, stream), _timing_ptr(timing))
    _raise("ssm_conv1d_fwd", rc)
    return y, ring_last


@_on_stream
def ssm_gdn2_fwd(q, k, v, g, b, w, S0=None, *, scale=1.0, return_state=True, o=None, stream=None,
                 timing=None):
    """Gated DeltaNet-2 forward (the gated delta rule with per-key-dimension decay,
    token by token).  q, k, g, b [batch, heads, L, k_dim] and v, w [batch, heads, L,
    v_dim], all float32 or all bfloat16 (state and arithmetic f32 either way);
    S0 [batch, heads, k_dim, v_dim] float32 or None (zeros).  Returns
    (o [batch, heads, L, v_dim] in the activations' dtype, S_last float32 or None)."""
    dev = q.device
    io = q.dtype
    bsz, nh, L, kd = q.shape
    vd = v.shape[-1] if v.dim() == 4 else -1
    for t, n in ((q, "q"), (k, "k"), (g, "g"), (b, "b")):
        _check(t, n, (bsz, nh, L, kd), io, dev)
    for t, n in ((v, "v"), (w, "w")):
        _check(t, n, (bsz, nh, L, vd), io, dev)
    _check(S0, "S0", (bsz, nh, kd, vd), torch.float32, dev, required=False)
    if o is None:
        o = torch.empty(bsz, nh, L, vd, dtype=io, device=dev)
    _check(o, "o", (bsz, nh, L, vd), io, dev)
    S_last = torch.empty(bsz, nh, kd, vd, dtype=torch.float32, device=dev) if return_state else None
    dm = Gdn2Dims(bsz, nh, L, kd, vd, _io_code(io))
    rc = _lib.ssm_gdn2_fwd(ctypes.byref(dm), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), _ptr(S0),
                           float(scale), _ptr(o), _ptr(S_last), _stream(dev, stream), _timing_ptr(timing))
    _raise("ssm_gdn2_fwd", rc)
    return o, S_last


def gdn2_chunked_workspace_bytes(batch, heads, seqlen, k_dim, v_dim, io_dtype=torch.float32):
    dm = Gdn2Dims(int(batch), int(heads), int(seqlen), int(k_dim), int(v_dim), _io_code(io_dtype))
    return int(_lib.ssm_gdn2_chunked_workspace_bytes(ctypes.byref(dm)))


@_on_stream
def ssm_gdn2_fwd_chunked(q, k, v, g, b, w, S0=None, *, scale=1.0, return_state=True, o=None, stream=None,
                         timing=None):
    """The Gated DeltaNet-2 forward in chunks of 64 tokens (WY form, decays per key
    dimension, products on MFMA); same arguments and results as ssm_gdn2_fwd up to
    f32 rounding.  v_dim must be a multiple of 16."""
    dev = q.device
    io = q.dtype
    bsz, nh, L, kd = q.shape
    vd = v.shape[-1] if v.dim() == 4 else -1
    for t, n in ((q, "q"), (k, "k"), (g, "g"), (b, "b")):
        _check(t, n, (bsz, nh, L, kd), io, dev)
    for t, n in ((v, "v"), (w, "w")):
        _check(t, n, (bsz, nh, L, vd), io, dev)
    _check(S0, "S0", (bsz, nh, kd, vd), torch.float32, dev, required=False)
    if o is None:
        o = torch.empty(bsz, nh, L, vd, dtype=io, device=dev)
    _check(o, "o", (bsz, nh, L, vd), io, dev)
    S_last = torch.empty(bsz, nh, kd, vd, dtype=torch.float32, device=dev) if return_state else None
    dm = Gdn2Dims(bsz, nh, L, kd, vd, _io_code(io))
    nws = _lib.ssm_gdn2_chunked_workspace_bytes(ctypes.byref(dm))
    ws = _workspace(nws, dev)
    rc = _lib.ssm_gdn2_fwd_chunked(ctypes.byref(dm), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w),
                                   _ptr(S0), float(scale), _ptr(o), _ptr(S_last), _ptr(ws), nws,
                                   _stream(dev, stream), _timing_ptr(timing))
    _raise("ssm_gdn2_fwd_chunked", rc)
    return o, S_last


@_on_stream
def ssm_conv1d_bwd(x, w, bias, dy, ring0=None, *, want_dring0=False, stream=None, timing=None, out=None):
    """Backward of ssm_conv1d_fwd for the loss sum(dy * y).  Returns a dict with dx
    (io dtype), dw [d_inner, d_conv], dbias [d_inner] and dring0 (float32; None
    unless want_dring0)."""
    dev = x.device
    bsz, L, din = x.shape
    io = x.dtype
    k = w.shape[1] if w.dim() == 2 else -1
    _check(x, "x", (bsz, L, din), io, dev)
    _check(dy, "dy", (bsz, L, din), io, dev)
    _check(w, "w", (din, k), torch.float32, dev)
    _check(bias, "bias", (din,), torch.float32, dev, required=False)
    ring0 = _ring(ring0, "ring0", bsz, din, k, dev)
    g = out if out is not None else {}
    g.setdefault("dx", torch.empty_like(x))
    g.setdefault("dw", torch.empty_like(w))
    g.setdefault("dbias", torch.empty(din, dtype=torch.float32, device=dev))
    g.setdefault("dring0", torch.empty(bsz, din, k - 1, dtype=torch.float32, device=dev)
                 if want_dring0 and k > 1 else None)
    dm = conv_dims(bsz, L, din, k, io)
    nws = _lib.ssm_conv1d_bwd_workspace_bytes(ctypes.byref(dm))
    ws = _workspace(nws, dev)
    rc = _lib.ssm_conv1d_bwd(ctypes.byref(dm), _ptr(x), _ptr(w), _ptr(bias), _ptr(ring0), _ptr(dy),
                             _ptr(g["dx"]), _ptr(g["dw"]), _ptr(g["dbias"]), _ptr(g["dring0"]), _ptr(ws), nws,
                             _stream(dev, stream), _timing_ptr(timing))
    _raise("ssm_conv1d_bwd", rc)
    return g


CONV1D_SCRATCH_BYTES = 16 << 20


def ssm_conv1d_bwd_noalloc(x, w, bias, dy, ring0=None, *, dx, dw, dbias, dring0=None, stream=None,
                           timing=None):
    """ssm_conv1d_bwd without a workspace: its partials go to the library's static
    16 MiB device scratch, so the call allocates nothing (every output is the
    caller's).  Calls that overlap on one GPU share that scratch and race."""
    dev = x.device
    bsz, L, din = x.shape
    io = x.dtype
    k = w.shape[1] if w.dim() == 2 else -1
    _check(x, "x", (bsz, L, din), io, dev)
    _check(dy, "dy", (bsz, L, din), io, dev)
    _check(w, "w", (din, k), torch.float32, dev)
    _check(bias, "bias", (din,), torch.float32, dev, required=False)
    ring0 = _ring(ring0, "ring0", bsz, din, k, dev)
    _check(dx, "dx", (bsz, L, din), io, dev)
    _check(dw, "dw", (din, k), torch.float32, dev)
    _check(dbias, "dbias", (din,), torch.float32, dev)
    dring0 = _ring(dring0, "dring0", bsz, din, k, dev)
    dm = conv_dims(bsz, L, din, k, io)
    rc = _lib.ssm_conv1d_bwd_noalloc(ctypes.byref(dm), _ptr(x), _ptr(w), _ptr(bias), _ptr(ring0), _ptr(dy),
                                     _ptr(dx), _ptr(dw), _ptr(dbias), _ptr(dring0), _stream(dev, stream),
                                     _timing_ptr(timing))
    _raise("ssm_conv1d_bwd_noalloc", rc)


@_on_stream
def ssm_conv1d_step(ring, x, w, bias=None, *, y=None, stream=None, timing=None):
    """One token through the conv ring: ring [batch, d_inner, d_conv-1] float32 is
    updated in place (ignored for d_conv 1); x [batch, d_inner] io dtype.
    Returns y [batch, d_inner]."""
    dev = x.device
    bsz, din = x.shape
    io = x.dtype
    k = w.shape[1] if w.dim() == 2 else -1
    _check(x, "x", (bsz, din), io, dev)
    _check(w, "w", (din, k), torch.float32, dev)
    _check(bias, "bias", (din,), torch.float32, dev, required=False)
    ring = _ring(ring, "ring", bsz, din, k, dev, required=True)
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", (bsz, din), io, dev)
    rc = _lib.ssm_conv1d_step(bsz, din, k, _io_code(io), _ptr(ring), _ptr(x), _ptr(w), _ptr(bias), _ptr(y),
                              _stream(dev, stream), _timing_ptr(timing))
    _raise("ssm_conv1d_step", rc)
    return y


# ---------------------------------------------------------------- Mamba block
# SSM_BLOCK_LIB may point at another build of the block library (A/B timing).
BLOCK_LIB_PATH = os.environ.get("SSM_BLOCK_LIB") or os.path.join(_HERE, "libssmblock.so")
_block_lib = None
BLOCK_PARAMS = ("W_in", "conv_w", "conv_b", "W_x", "W_dt", "dt_bias", "A_log", "D", "W_out")


class BlockDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("d_model", ctypes.c_int64),
                ("d_inner", ctypes.c_int64), ("d_state", ctypes.c_int64), ("dt_rank", ctypes.c_int64),
                ("d_conv", ctypes.c_int64), ("io_dtype", ctypes.c_int32)]


class BlockParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BLOCK_PARAMS]


class BlockGrads(ctypes.Structure):
    _fields_ = [("d" + n, ctypes.c_void_p) for n in BLOCK_PARAMS]


def block_library():
    """libssmblock.so (the Mamba block: projections on hipBLASLt around this
    library's conv and scan kernels), loaded on first use."""
    global _block_lib
    if _block_lib is not None:
        return _block_lib
    if not os.path.exists(BLOCK_LIB_PATH):
        raise ImportError(f"{BLOCK_LIB_PATH} is missing: build the HIP libraries first")
    lib = ctypes.CDLL(BLOCK_LIB_PATH)
    P, SZ = ctypes.c_void_p, ctypes.c_size_t
    DP = ctypes.POINTER(BlockDims)
    lib.ssm_block_create.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.ssm_block_create.restype = ctypes.c_int
    lib.ssm_block_destroy.argtypes = [P]
    lib.ssm_block_destroy.restype = None
    for fn in ("ssm_block_saved_bytes", "ssm_block_fwd_workspace_bytes", "ssm_block_fwd_training_workspace_bytes",
               "ssm_block_bwd_workspace_bytes"):
        getattr(lib, fn).argtypes = [DP]
        getattr(lib, fn).restype = SZ
    lib.ssm_block_fwd.argtypes = [P, DP, P, ctypes.POINTER(BlockParams), P, P, P, SZ, P,
                                  ctypes.POINTER(SsmTiming)]
    lib.ssm_block_fwd.restype = ctypes.c_int
    lib.ssm_block_bwd.argtypes = [P, DP, P, ctypes.POINTER(BlockParams), P, P, P, ctypes.POINTER(BlockGrads),
                                  P, SZ, P, ctypes.POINTER(SsmTiming)]
    lib.ssm_block_bwd.restype = ctypes.c_int
    _block_lib = lib
    return lib


class BlockContext:
    """A hipBLASLt handle on the current device for ssm_block_fwd / ssm_block_bwd."""

    def __init__(self):
        self._lib = block_library()
        self.ptr = ctypes.c_void_p()
        _raise("ssm_block_create", self._lib.ssm_block_create(ctypes.byref(self.ptr)))

    def close(self):
        if self.ptr:
            self._lib.ssm_block_destroy(self.ptr)
            self.ptr = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _block_check(X, prm):
    dev = X.device
    bsz, L, dm = X.shape
    io = X.dtype
    di = prm["W_in"].shape[0] // 2
    R = prm["W_dt"].shape[1]
    N = prm["A_log"].shape[1]
    K = prm["conv_w"].shape[1]
    _check(X, "X", (bsz, L, dm), io, dev)
    shapes = {"W_in": ((2 * di, dm), io), "conv_w": ((di, K), torch.float32), "W_x": ((R + 2 * N, di), io),
              "W_dt": ((di, R), io), "dt_bias": ((di,), torch.float32), "A_log": ((di, N), torch.float32),
              "D": ((di,), torch.float32), "W_out": ((dm, di), io)}
    for n, (shp, dt) in shapes.items():
        _check(prm.get(n), n, shp, dt, dev)
    _check(prm.get("conv_b"), "conv_b", (di,), torch.float32, dev, required=False)
    dm_ = BlockDims(bsz, L, dm, di, N, R, K, _io_code(io))
    pp = BlockParams(*[None if prm.get(n) is None else prm[n].data_ptr() for n in BLOCK_PARAMS])
    return dm_, pp, dev


@_on_stream
def ssm_block_fwd(ctx, X, params, *, training=True, Y=None, stream=None, timing=None):
    """One Mamba block.  X [batch, L, d_model] (float32 or bfloat16); params: dict
    with W_in [2 d_inner, d_model], W_x [dt_rank + 32, d_inner], W_dt [d_inner,
    dt_rank], W_out [d_model, d_inner] (X's dtype) and conv_w [d_inner, d_conv],
    conv_b [d_inner] (optional), dt_bias [d_inner], A_log [d_inner, 16], D [d_inner]
    (float32).  Returns (Y, saved or None); ssm_block_bwd needs `saved`."""
    lib = block_library()
    dm, pp, dev = _block_check(X, params)
    if Y is None:
        Y = torch.empty_like(X)
    _check(Y, "Y", tuple(X.shape), X.dtype, dev)
    saved = None
    if training:
        saved = torch.empty(lib.ssm_block_saved_bytes(ctypes.byref(dm)), dtype=torch.uint8, device=dev)
        nws = lib.ssm_block_fwd_training_workspace_bytes(ctypes.byref(dm))
    else:
        nws = lib.ssm_block_fwd_workspace_bytes(ctypes.byref(dm))
    ws = _workspace(nws, dev)
    rc = lib.ssm_block_fwd(ctx.ptr, ctypes.byref(dm), _ptr(X), ctypes.byref(pp), _ptr(Y), _ptr(saved), _ptr(ws),
                           nws, _stream(dev, stream), _timing_ptr(timing))
    _raise("ssm_block_fwd", rc)
    return Y, saved


@_on_stream
def ssm_block_bwd(ctx, X, params, saved, dY, *, out=None, stream=None, timing=None):
    """Backward of ssm_block_fwd for the loss sum(dY * Y).  Returns a dict with dX
    (X's dtype) and d<name> (float32, summed over batch and time) for every
    parameter."""
    lib = block_library()
    dm, pp, dev = _block_check(X, params)
    _check(dY, "dY", tuple(X.shape), X.dtype, dev)
    _check(saved, "saved", (lib.ssm_block_saved_bytes(ctypes.byref(dm)),), torch.uint8, dev)
    g = out if out is not None else {}
    g.setdefault("dX", torch.empty_like(X))
    for n in BLOCK_PARAMS:
        ref = params[n] if params.get(n) is not None else params["D"]
        g.setdefault("d" + n, torch.empty(ref.shape, dtype=torch.float32, device=dev))
    gg = BlockGrads(*[g["d" + n].data_ptr() for n in BLOCK_PARAMS])
    nws = lib.ssm_block_bwd_workspace_bytes(ctypes.byref(dm))
    ws = _workspace(nws, dev)
    rc = lib.ssm_block_bwd(ctx.ptr, ctypes.byref(dm), _ptr(X), ctypes.byref(pp), _ptr(saved), _ptr(dY),
                           _ptr(g["dX"]), ctypes.byref(gg), _ptr(ws), nws, _stream(dev, stream),
                           _timing_ptr(timing))
    _raise("ssm_block_bwd", rc)
    return g


class LaunchTimer:
    """Per-kernel timing through the ABI's optional launch log: HIP events recorded
    by the library around each of its launches, on the launch stream."""

    def __init__(self, capacity=TIMING_MAX):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.capacity = min(capacity, TIMING_MAX)
        self._events = (ctypes.c_void_p * (2 * self.capacity))()
        for i in range(2 * self.capacity):
            ev = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self._events[i] = ev
        self.struct = SsmTiming()
        self.struct.events = ctypes.cast(self._events, ctypes.c_void_p)
        self.struct.capacity = self.capacity
        self.reset()

    def reset(self):
        self.struct.count = 0

    def results(self):
        """[(kernel name, milliseconds)] for the recorded launches (call after a sync)."""
        out = []
        for i in range(self.struct.count):
            ms = ctypes.c_float()
            rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), self._events[2 * i], self._events[2 * i + 1])
            if rc != 0:
                raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
            out.append((kernel_name(self.struct.kernel_id[i]), ms.value))
        return out

    def close(self):
        for i in range(2 * self.capacity):
            if self._events[i]:
                self._hip.hipEventDestroy(self._events[i])
                self._events[i] = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


__all__ = ["ssm_scan_fwd", "ssm_scan_bwd", "ssm_scan_step", "ckpt_bytes", "fwd_workspace_bytes",
           "bwd_workspace_bytes", "LaunchTimer", "SsmError", "library", "status_str", "kernel_name",
           "SsmDims", "SsmTiming", "ssm_conv1d_fwd", "ssm_conv1d_bwd", "ssm_conv1d_step",
           "conv1d_bwd_workspace_bytes", "ConvDims", "ssm_conv1d_bwd_noalloc", "CONV1D_SCRATCH_BYTES", "BlockContext", "ssm_block_fwd", "ssm_block_bwd",
           "block_library", "BlockDims", "ssm_gdn2_fwd", "Gdn2Dims", "ssm_gdn2_fwd_chunked",
           "gdn2_chunked_workspace_bytes"]
