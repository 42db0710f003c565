"""Seeded synthetic inputs for the S6 selective-scan workloads.

Shared by the oracle-side tests and the HIP-side tests/bench: it draws random
numbers and shapes them, and holds none of the scan's arithmetic.

Recipe (one numpy PCG64 stream per call, ``default_rng(seed)``):
  draw order x, z, dt_raw, B, C, then dy when a backward is needed, each with
  ``standard_normal(dtype=float32)``; dt = 0.1 * dt_raw; A_log[d, n] = ln(n + 1);
  D = 1; dt_bias = 0 for the "active" regime (softplus(0) = ln 2 ~ 0.69) and
  ln(expm1(0.01)) for the "slow" regime (softplus = 0.01).  These constants are
  the canonical S6 initialisation and the active_block override described in the
  rustytorch commit log (commit fixing the NaN from randn init).  For bf16 I/O the
  f32 draws are rounded to nearest-even bf16 and both sides consume the rounded
  values.
"""
import math

import numpy as np

D_STATE = 16

# dt_bias giving softplus(dt_bias) = 0.01 (inverse of softplus at 0.01).
DT_BIAS_SLOW = float(np.float32(math.log(math.expm1(0.01))))
DT_BIAS_ACTIVE = 0.0

CONFIGS = {
    # name: batch, seqlen, d_inner, d_state, io dtype, dt_bias regime, passes
    "c1_tiny": dict(batch=1, seqlen=64, d_inner=32, d_state=16, io="f32",
                    dt_bias=DT_BIAS_ACTIVE, passes="fwd+bwd"),
    "c2_mamba130m_fwd": dict(batch=8, seqlen=2048, d_inner=1536, d_state=16, io="f32",
                             dt_bias=DT_BIAS_SLOW, passes="fwd"),
    "c3_mamba130m_fwdbwd": dict(batch=8, seqlen=2048, d_inner=1536, d_state=16, io="f32",
                                dt_bias=DT_BIAS_SLOW, passes="fwd+bwd"),
    "c4_mamba2p8b_bf16": dict(batch=4, seqlen=8192, d_inner=5120, d_state=16, io="bf16",
                              dt_bias=DT_BIAS_ACTIVE, passes="fwd+bwd"),
    # decode: 1024 single-token steps; inputs drawn as [batch, ntok, d_inner] like c4,
    # rounded to bf16 and promoted back to f32.
    "c5_decode_step": dict(batch=256, seqlen=1024, d_inner=5120, d_state=16, io="f32",
                           dt_bias=DT_BIAS_ACTIVE, passes="step", bf16_values=True),
}


def round_bf16(a):
    """Round an f32 array to the nearest-even bf16 value, returned as f32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    nan = np.isnan(a)
    u = a.view(np.uint32).copy()
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)           # no overflow for finite values
    u += lsb
    u &= np.uint32(0xFFFF0000)
    out = u.view(np.float32)
    if nan.any():
        out[nan] = np.nan
    return out


def a_log_canonical(d_inner, d_state=D_STATE, shift=0.0):
    """A_log[d, n] = ln(n + 1) + shift, so A = -(n + 1) * exp(shift)."""
    row = np.log(np.arange(1, d_state + 1, dtype=np.float64)) + shift
    return np.ascontiguousarray(np.broadcast_to(row.astype(np.float32), (d_inner, d_state)))


def make_inputs(batch, seqlen, d_inner, d_state=D_STATE, *, seed=0, dt_bias=DT_BIAS_ACTIVE,
                dt_scale=0.1, bf16=False, with_dy=True, a_log=None, with_z=True, d_skip=1.0):
    """Draws one workload.  Returns a dict of C-contiguous f32 numpy arrays:
    x, z, dt, B, C, (dy), A_log, D, dt_bias.  With ``bf16`` the activations are
    rounded to bf16 values (still stored as f32)."""
    rng = np.random.default_rng(seed)
    shp = (batch, seqlen, d_inner)
    x = rng.standard_normal(shp, dtype=np.float32)
    z = rng.standard_normal(shp, dtype=np.float32)
    dt = rng.standard_normal(shp, dtype=np.float32)
    dt *= np.float32(dt_scale)
    Bm = rng.standard_normal((batch, seqlen, d_state), dtype=np.float32)
    Cm = rng.standard_normal((batch, seqlen, d_state), dtype=np.float32)
    dy = rng.standard_normal(shp, dtype=np.float32) if with_dy else None
    if bf16:
        x, z, dt, Bm, Cm = (round_bf16(v) for v in (x, z, dt, Bm, Cm))
        if dy is not None:
            dy = round_bf16(dy)
    out = {
        "x": x, "z": z if with_z else None, "dt": dt, "B": Bm, "C": Cm, "dy": dy,
        "A_log": a_log if a_log is not None else a_log_canonical(d_inner, d_state),
        "D": np.full(d_inner, d_skip, dtype=np.float32),
        "dt_bias": np.full(d_inner, dt_bias, dtype=np.float32),
    }
    return out


def make_config(name, *, seed=0, with_dy=None):
    """Inputs for a named workload of CONFIGS."""
    c = CONFIGS[name]
    if with_dy is None:
        with_dy = "bwd" in c["passes"]
    bf16 = c["io"] == "bf16" or c.get("bf16_values", False)
    return make_inputs(c["batch"], c["seqlen"], c["d_inner"], c["d_state"], seed=seed,
                       dt_bias=c["dt_bias"], bf16=bf16, with_dy=with_dy)


def random_a_log(d_inner, d_state=D_STATE, *, seed=1, spread=0.5):
    """A_log = ln(n+1) + spread*N(0,1) per (d, n) (guards against shortcuts that
    assume integer A)."""
    rng = np.random.default_rng(seed)
    base = np.log(np.arange(1, d_state + 1, dtype=np.float64))[None, :]
    return (base + spread * rng.standard_normal((d_inner, d_state))).astype(np.float32)


# Causal depthwise conv1d + SiLU in front of the scan: same batch/seqlen/d_inner
# as the bench workload, kernel width 4.
CONV_CONFIGS = {
    "conv_mamba2p8b_bf16": dict(batch=4, seqlen=8192, d_inner=5120, d_conv=4, io="bf16"),
}


def make_conv_inputs(batch, seqlen, d_inner, d_conv=4, *, seed=0, bf16=False, with_ring=False,
                     with_bias=True):
    """Inputs of the conv1d + SiLU.  Draw order from default_rng(seed), each
    standard_normal(float32): x [batch, seqlen, d_inner], w [d_inner, d_conv]
    (scaled by 1/sqrt(d_conv), the fan-in of a depthwise tap row), bias [d_inner]
    (scaled by 0.5; zero when with_bias is False, the canonical zero conv bias),
    ring0 [batch, d_inner, d_conv-1], dy [batch, seqlen, d_inner].  Every tensor is
    drawn whatever the flags, so the flags do not shift the stream.  With bf16 the
    activations (x, ring0, dy) are rounded to nearest-even bf16."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, seqlen, d_inner), dtype=np.float32)
    w = rng.standard_normal((d_inner, d_conv), dtype=np.float32) * np.float32(1.0 / math.sqrt(d_conv))
    bias = rng.standard_normal(d_inner, dtype=np.float32) * np.float32(0.5)
    ring0 = rng.standard_normal((batch, d_inner, max(d_conv - 1, 0)), dtype=np.float32)
    dy = rng.standard_normal((batch, seqlen, d_inner), dtype=np.float32)
    if bf16:
        x, ring0, dy = round_bf16(x), round_bf16(ring0), round_bf16(dy)
    return {"x": x, "w": w, "bias": bias if with_bias else np.zeros(d_inner, np.float32),
            "ring0": ring0 if with_ring and d_conv > 1 else None, "dy": dy}


def make_conv_config(name, *, seed=0):
    c = CONV_CONFIGS[name]
    return make_conv_inputs(c["batch"], c["seqlen"], c["d_inner"], c["d_conv"], seed=seed,
                            bf16=c["io"] == "bf16", with_bias=False)


# One Mamba block around the scan (Mamba-2.8B layer shapes): d_model 2560,
# d_inner 5120, d_state 16, dt_rank ceil(d_model / 16) = 160, d_conv 4.
BLOCK_CONFIGS = {
    "block_mamba2p8b_bf16": dict(batch=4, seqlen=8192, d_model=2560, d_inner=5120, d_state=16, dt_rank=160,
                                 d_conv=4, io="bf16"),
}


def make_block_inputs(batch, seqlen, d_model, d_inner, d_state=D_STATE, dt_rank=None, d_conv=4, *, seed=0,
                      bf16=False):
    """Inputs of one Mamba block.  Draw order from default_rng(seed), each
    standard_normal(float32): X [batch, seqlen, d_model], W_in [2 d_inner, d_model],
    conv_w [d_inner, d_conv], conv_b [d_inner], W_x [dt_rank + 2 d_state, d_inner],
    W_dt [d_inner, dt_rank], W_out [d_model, d_inner], dY [batch, seqlen, d_model].
    Weights are scaled by min(1/sqrt(fan_in), 0.5) (the canonical init's projection
    scale; the conv's fan-in is d_conv), the conv bias is zero, A_log = ln(1..N),
    D = 1 and dt_bias gives softplus = 0.01 (the canonical S6 init).  With bf16
    the activations X, dY and the projection weights are rounded to bf16."""
    if dt_rank is None:
        dt_rank = -(-d_model // 16)
    rng = np.random.default_rng(seed)

    def w(shape, fan_in):
        return rng.standard_normal(shape, dtype=np.float32) * np.float32(min(1.0 / math.sqrt(fan_in), 0.5))

    X = rng.standard_normal((batch, seqlen, d_model), dtype=np.float32)
    p = {"W_in": w((2 * d_inner, d_model), d_model), "conv_w": w((d_inner, d_conv), d_conv)}
    p["conv_b"] = np.zeros(d_inner, np.float32)
    p["W_x"] = w((dt_rank + 2 * d_state, d_inner), d_inner)
    p["W_dt"] = w((d_inner, dt_rank), dt_rank)
    p["W_out"] = w((d_model, d_inner), d_inner)
    dY = rng.standard_normal((batch, seqlen, d_model), dtype=np.float32)
    p["A_log"] = a_log_canonical(d_inner, d_state)
    p["D"] = np.ones(d_inner, np.float32)
    p["dt_bias"] = np.full(d_inner, DT_BIAS_SLOW, np.float32)
    if bf16:
        X, dY = round_bf16(X), round_bf16(dY)
        for k in ("W_in", "W_x", "W_dt", "W_out"):
            p[k] = round_bf16(p[k])
    return X, p, dY


def make_block_config(name, *, seed=0):
    c = BLOCK_CONFIGS[name]
    return make_block_inputs(c["batch"], c["seqlen"], c["d_model"], c["d_inner"], c["d_state"], c["dt_rank"],
                             c["d_conv"], seed=seed, bf16=c["io"] == "bf16")


def make_regime_corpus(n_seq, seqlen, d_model, *, seed=0):
    """Synthetic stand-in for a four-regime sequence corpus (the pages train on
    one but do not publish it).  Sequence i follows regime i mod 4 with parameters
    drawn from default_rng(seed): 0 a sinusoid, 1 an AR(1) process, 2 a square
    wave, 3 a damped oscillation restarted every period.  The scalar series s
    (length seqlen + 1, unit-scale) is embedded along one fixed random unit vector
    u: X[i, t] = s_t u and the next-step target Y[i, t] = s_{t+1} u.  Returns
    (X, Y), both float32 [n_seq, seqlen, d_model]."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(d_model).astype(np.float64)
    u /= np.linalg.norm(u)
    t = np.arange(seqlen + 1, dtype=np.float64)
    S = np.empty((n_seq, seqlen + 1))
    for i in range(n_seq):
        r = i % 4
        w = rng.uniform(0.05, 0.3)
        ph = rng.uniform(0.0, 2.0 * math.pi)
        if r == 0:
            S[i] = np.sin(w * t + ph)
        elif r == 1:
            e = rng.standard_normal(seqlen + 1)
            s = np.empty(seqlen + 1)
            s[0] = e[0]
            for k in range(1, seqlen + 1):
                s[k] = 0.95 * s[k - 1] + 0.3 * e[k]
            S[i] = s / max(np.max(np.abs(s)), 1e-9)
        elif r == 2:
            S[i] = 0.8 * np.sign(np.sin(w * t + ph))
        else:
            period = int(rng.integers(16, 48))
            S[i] = np.exp(-0.05 * (t % period)) * np.cos(w * t + ph)
    X = (S[:, :-1, None] * u).astype(np.float32)
    Y = (S[:, 1:, None] * u).astype(np.float32)
    return X, Y


GDN2_CONFIGS = {
    # name: batch, heads, seqlen, k_dim, v_dim (f32)
    "gdn2_b4h16t4096": dict(batch=4, heads=16, seqlen=4096, k_dim=128, v_dim=128),
}


def make_gdn2_inputs(batch, heads, seqlen, k_dim, v_dim, *, seed=0, with_state=False):
    """Gated DeltaNet-2 forward inputs.  Draw order from default_rng(seed), each
    standard_normal(float32) of its shape: q, k [B, H, L, K], v [B, H, L, V], then
    g_raw, b_raw [B, H, L, K], w_raw [B, H, L, V], then S0 [B, H, K, V] if asked.
    Shaping: k is scaled to unit L2 norm per token (the usual key normalisation of
    delta rules); g = -exp(0.5 g_raw - 3) (log-decays, decay factors exp(g) mostly
    0.9 .. 1); b = sigmoid(b_raw) and w = sigmoid(w_raw) (gates in (0, 1)); S0 is
    scaled by 0.1.  The scale 1/sqrt(K) is the caller's."""
    rng = np.random.default_rng(seed)
    shk, shv = (batch, heads, seqlen, k_dim), (batch, heads, seqlen, v_dim)
    q = rng.standard_normal(shk, dtype=np.float32)
    k = rng.standard_normal(shk, dtype=np.float32)
    v = rng.standard_normal(shv, dtype=np.float32)
    g_raw = rng.standard_normal(shk, dtype=np.float32)
    b_raw = rng.standard_normal(shk, dtype=np.float32)
    w_raw = rng.standard_normal(shv, dtype=np.float32)
    k = (k / np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), 1e-6)).astype(np.float32)
    g = (-np.exp(0.5 * g_raw - 3.0)).astype(np.float32)
    b = (1.0 / (1.0 + np.exp(-b_raw))).astype(np.float32)
    w = (1.0 / (1.0 + np.exp(-w_raw))).astype(np.float32)
    out = {"q": q, "k": k, "v": v, "g": g, "b": b, "w": w, "S0": None}
    if with_state:
        out["S0"] = (0.1 * rng.standard_normal((batch, heads, k_dim, v_dim), dtype=np.float32)).astype(np.float32)
    return out


def make_gdn2_config(name, *, seed=0):
    c = GDN2_CONFIGS[name]
    return make_gdn2_inputs(c["batch"], c["heads"], c["seqlen"], c["k_dim"], c["v_dim"], seed=seed)
