"""Throughput of the S6 selective scan on one MI355X.

One step of the default workload = ssm_scan_fwd (training, writes checkpoints)
+ ssm_scan_bwd over one batch of the Mamba-2.8B-shaped workload: batch 4,
seqlen 8192, d_inner 5120, d_state 16, bf16 activations, f32 state and
arithmetic.  --config picks another of the five scan workloads (the tiny f32
case, the Mamba-130M-shaped forward and forward+backward, the decode chain).
Inputs are seeded synthetic tensors already resident in HBM.  The metric is
elements (batch*seqlen*d_inner*d_state) per second; each timed step starts
after a read of 512 MiB of unrelated data, which leaves the caches cold and
clean (the flushed time is `value`, the back-to-back time is reported beside
it).

Prints ONE JSON line.  Besides the contract fields it carries
  roofline      : the dominant kernel against HBM bandwidth: its algorithmic
                  bytes per launch (inputs read once, outputs written once) /
                  its average launch time (HIP events the library records
                  around each launch on the launch stream), against 8 TB/s,
                  and against a plain device copy measured in the same run;
                  `traffic` is its profiler-counted bytes when they were taken
                  on the current kernel source, else null;
  valu          : the same kernel's counted VALU lane instructions per second
                  against the non-packed issue peak (when counted on this source);
  step_hbm      : the whole step's algorithmic bytes / step time;
  cpu_baseline  : the f64 oracle timed on a bounded sample on the host cores.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
CSRC = os.path.join(ROOT, "selective_state_space_04_amd", "csrc")
# (kernel source, committed counter summary) per workload
TRAFFIC = {"scan": (os.path.join(CSRC, "ssm_scan.hip"),
                    os.path.join(ROOT, "profiles", "c4_mamba2p8b_bf16_traffic.txt")),
           "conv1d": (os.path.join(CSRC, "ssm_conv1d.hip"),
                      os.path.join(ROOT, "profiles", "conv_mamba2p8b_bf16_traffic.txt")),
           "decode": (os.path.join(CSRC, "ssm_scan.hip"),
                      os.path.join(ROOT, "profiles", "c5_decode_step_traffic.txt")),
           "gdn2": (os.path.join(CSRC, "ssm_gdn2.hip"),
                    os.path.join(ROOT, "profiles", "gdn2_b4h16t4096_traffic.txt")),
           "gdn2_chunked": (os.path.join(CSRC, "ssm_gdn2_chunk.hip"),
                            os.path.join(ROOT, "profiles", "gdn2_chunked_b4h16t4096_traffic.txt"))}

def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c4_mamba2p8b_bf16",
                    choices=("c1_tiny", "c2_mamba130m_fwd", "c3_mamba130m_fwdbwd", "c4_mamba2p8b_bf16",
                             "c5_decode_step"),
                    help="scan workload (c5_decode_step runs the decode bench)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--out", default=None, help="also write the JSON line to this file")
    ap.add_argument("--op", choices=("scan", "conv1d", "decode", "block", "block-c", "train", "gdn2"),
                    default="scan",
                    help="scan: the selective scan fwd+bwd (default); conv1d: the causal depthwise "
                         "conv1d + SiLU fwd+bwd in front of it, on the same batch/seqlen/d_inner; "
                         "decode: 1024 single-token steps at batch 256 x d_inner 5120, eager and "
                         "replayed from a captured HIP graph; block: one Mamba block (projections on "
                         "hipBLASLt around the conv and the scan) fwd+bwd at the 2.8B layer shape")
    ap.add_argument("--gdn2-form", choices=("chunked", "recurrent"), default="chunked",
                    help="--op gdn2: the chunked WY form on MFMA or the token recurrence")
    ap.add_argument("--dim", type=int, default=16,
                    help="--op train: d_model of the one-block model (d_inner = 2 d_model)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (known bytes) to calibrate "
                         "profiler FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def algorithmic_bytes(cfg, esz):
    """Compulsory bytes: every input read once, every output written once."""
    b, L, d, n = cfg["batch"], cfg["seqlen"], cfg["d_inner"], cfg["d_state"]
    btd, btn = b * L * d, b * L * n
    params = 4 * (d * n + 2 * d)
    fwd = btd * esz * 4 + btn * esz * 2 + params          # x, dt, z in; y out; B, C in
    bwd_main = btd * esz * 7 + btn * esz * 2 + params     # x, dt, z, dy in; dx, ddt, dz out; B, C in
    bwd = bwd_main + btn * esz * 2 + params               # + dB, dC, param grads out
    return {"fwd": fwd, "bwd": bwd, "bwd_main": bwd_main, "fwd_main": fwd}


def measured_traffic(kernel, op="scan"):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None
    when the summary was taken on a different kernel source."""
    import hashlib
    src_path, traffic_path = TRAFFIC[op]
    try:
        lines = open(traffic_path).read().split("\n")
        src = hashlib.sha256(open(src_path, "rb").read()).hexdigest()
    except OSError:
        return None
    kv = {}
    for ln in lines:
        parts = ln.split()
        if len(parts) >= 2 and not ln.startswith("#"):
            kv[parts[0]] = parts[1:]
    if kv.get("source_sha256", [None])[0] != src or kernel not in kv:
        return None
    f = dict(p.split("=") for p in kv[kernel])
    return int(float(f["fetch_bytes"]) + float(f["write_bytes"]))


def copy_probe(dev):
    """A plain 1 GiB device-to-device copy: known bytes for calibrating the
    profiler's FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def conv_bench(args):
    """Causal depthwise conv1d + SiLU, forward + backward, on the conv workload."""
    import numpy as np
    import torch

    import selective_state_space_04_amd as ssm
    import workloads as W

    name = "conv_mamba2p8b_bf16"
    cfg = W.CONV_CONFIGS[name]
    dev = torch.device("cuda:0")
    io = torch.bfloat16 if cfg["io"] == "bf16" else torch.float32
    esz = 2 if io == torch.bfloat16 else 4
    print(f"[bench] generating {name} inputs", file=sys.stderr, flush=True)
    inp = W.make_conv_config(name)
    x = torch.from_numpy(inp["x"]).to(dev).to(io)
    dy = torch.from_numpy(inp["dy"]).to(dev).to(io)
    w = torch.from_numpy(inp["w"]).to(dev)
    bias = torch.from_numpy(inp["bias"]).to(dev)
    bsz, L, D = x.shape
    K = w.shape[1]
    y = torch.empty_like(x)
    grads = {"dx": torch.empty_like(x), "dw": torch.empty_like(w), "dbias": torch.empty_like(bias),
             "dring0": None}

    def fwd(timer=None):
        ssm.ssm_conv1d_fwd(x, w, bias, y=y, timing=timer)

    def bwd(timer=None):
        ssm.ssm_conv1d_bwd(x, w, bias, dy, out=grads, timing=timer)

    if args.copy_probe:
        copy_probe(dev)
    copy_gbps = copy_bandwidth(dev)

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    # Flushed: a cache flush before each of the two passes, outside its events,
    # so that neither reads what the other (or the previous step) left in the
    # caches, as in a model where other layers run between a layer's forward
    # and its backward.
    flush = CacheFlush(dev)
    timers = [ssm.LaunchTimer() for _ in range(args.steps)]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush()
        ev[i][0].record()
        fwd(timers[i])
        ev[i][1].record()
        flush()
        ev[i][2].record()
        bwd(timers[i])
        ev[i][3].record()
    torch.cuda.synchronize()
    ms_fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    ms_bwd = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    ms = ms_fwd + ms_bwd
    # Unflushed: the same passes back to back (the backward then finds part of x
    # in the Infinity Cache, and the next forward part of what the backward read).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        fwd()
        bwd()
    e1.record()
    torch.cuda.synchronize()
    ms_hot = e0.elapsed_time(e1) / args.steps
    del flush
    per_kernel = {}
    for tm in timers:
        for kname, kms in tm.results():
            per_kernel.setdefault(kname, []).append(kms)
        tm.close()
    kavg = {k: float(np.mean(v)) for k, v in per_kernel.items()}
    btd = bsz * L * D
    # compulsory bytes: forward reads x, writes y; backward reads x, dy, writes dx
    kbytes = {"k_conv_fwd": btd * esz * 2 + 4 * D * (K + 1),
              "k_conv_bwd": btd * esz * 3 + 4 * D * (K + 1)}
    dominant = max(kbytes, key=lambda k: kavg.get(k, 0.0))
    gbps = kbytes[dominant] / (kavg[dominant] * 1e-3) / 1e9
    traffic = measured_traffic(dominant, "conv1d")
    line = {
        "metric": "causal depthwise conv1d+SiLU fwd+bwd elements(B\u00b7L\u00b7D)/s and achieved HBM GB/s",
        "value": btd / (ms * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{name}: batch={bsz} seqlen={L} d_inner={D} d_conv={K}, {cfg['io']} "
                               f"activations, f32 weights and arithmetic, fwd+bwd",
                   "batch": bsz, "seqlen": L, "d_inner": D, "d_conv": K, "io_dtype": cfg["io"]},
        "timing": {"ms_per_step_flushed": round(ms, 4), "ms_fwd_flushed": round(ms_fwd, 4),
                   "ms_bwd_flushed": round(ms_bwd, 4), "ms_per_step_unflushed": round(ms_hot, 4),
                   "flush": "512 MiB read before the forward and before the backward, outside their events"},
        "achieved_hbm_GBps": round(sum(kbytes.values()) / (ms * 1e-3) / 1e9, 1),
        "kernels_ms": {k: round(v, 4) for k, v in sorted(kavg.items())},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": dominant,
                     "kernel_ms": round(kavg[dominant], 4), "algorithmic_bytes_per_launch": kbytes[dominant],
                     "traffic_over_algorithmic": None if traffic is None else round(traffic / kbytes[dominant], 3),
                     "copy_GBps": round(copy_gbps, 1), "frac_of_copy": round(gbps / copy_gbps, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        # The whole workload (one batch row at a time), repeated until about 10 s of host work.
        passes, sec = 0, 0.0
        while passes < 20 and sec < 10.0:
            for r in range(bsz):
                sub = {k: np.ascontiguousarray(inp[k][r:r + 1]).astype(np.float64) for k in ("x", "dy")}
                t0 = time.perf_counter()
                oracle.conv_fwd(sub["x"], inp["w"], inp["bias"])
                oracle.conv_bwd(sub["x"], inp["w"], inp["bias"], sub["dy"])
                sec += time.perf_counter() - t0
            passes += 1
        el = passes * btd
        line["cpu_baseline"] = {"value": el / sec, "unit": "elements/s", "cores": oracle.num_threads(),
                                "kind": "oracle",
                                "sample": f"the whole workload ({bsz} x {L} x {D}), one batch row per call, "
                                          f"fwd+bwd in f64, {passes} passes ({el} elements, {sec:.1f} s, "
                                          "f64 conversion of each row outside the timing)",
                                **host_cpu()}
    s = json.dumps(line)
    print(s, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(s + "\n")


def decode_bench(args):
    """1024 consecutive ssm_scan_step calls from a zero state (batch 256, d_inner
    5120, f32 with bf16-representable values): timed eagerly, and as one captured
    HIP graph of all 1024 launches, whose every replay is checked against the
    eager result."""
    import numpy as np
    import torch

    import selective_state_space_04_amd as ssm
    import workloads as W

    name = "c5_decode_step"
    cfg = W.CONFIGS[name]
    dev = torch.device("cuda:0")
    B, L, D, N = cfg["batch"], cfg["seqlen"], cfg["d_inner"], cfg["d_state"]
    print(f"[bench] generating {name} inputs", file=sys.stderr, flush=True)
    inp = W.make_config(name, with_dy=False)
    # time-major on the device, so that every step reads contiguous [batch, ...] slices
    tm = {k: torch.from_numpy(inp[k]).to(dev).transpose(0, 1).contiguous() for k in ("x", "z", "dt", "B", "C")}
    del inp["x"], inp["z"], inp["dt"]
    A_log, Dp, bias = (torch.from_numpy(inp[k]).to(dev) for k in ("A_log", "D", "dt_bias"))
    h = torch.zeros(B, D, N, device=dev)
    ys = torch.empty(L, B, D, device=dev)
    if args.copy_probe:
        copy_probe(dev)

    def run():
        for t in range(L):
            ssm.ssm_scan_step(h, tm["x"][t], tm["dt"][t], tm["B"][t], tm["C"][t], tm["z"][t], A_log, Dp, bias,
                              y=ys[t])

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        out = []
        for _ in range(reps):
            h.zero_()
            torch.cuda.synchronize()
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return float(np.median(out))

    copy_gbps = copy_bandwidth(dev)
    h.zero_()
    run()  # warm-up
    torch.cuda.synchronize()
    eager_ms = timed(run, max(1, min(args.steps, 5)))
    y_ref, h_ref = ys.clone(), h.clone()
    # one step kernel per launch, timed by the library's own events over 16 steps
    tmr = ssm.LaunchTimer()
    h.zero_()
    for t in range(tmr.capacity):
        ssm.ssm_scan_step(h, tm["x"][t], tm["dt"][t], tm["B"][t], tm["C"][t], tm["z"][t], A_log, Dp, bias,
                          y=ys[t], timing=tmr)
    torch.cuda.synchronize()
    kernel_ms = float(np.mean([ms for _, ms in tmr.results()]))
    tmr.close()
    # the whole 1024-step loop as one graph; every replay must reproduce the eager run
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        h.zero_()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    replays = []
    for _ in range(3):
        h.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replays.append(bool(torch.equal(ys, y_ref) and torch.equal(h, h_ref)))
    graph_ms = timed(graph.replay, max(1, min(args.steps, 5)))
    if not all(replays) or not (torch.equal(ys, y_ref) and torch.equal(h, h_ref)):
        raise SystemExit("graph replay differs from the eager decode loop")
    elems = B * D * N * L
    per_step = B * D * N * 4 * 2 + 4 * B * D * 4 + 2 * B * N * 4 + 4 * D * (N + 2)
    gbps = per_step / (kernel_ms * 1e-3) / 1e9
    traffic = measured_traffic("k_step", "decode")
    line = {
        "metric": "selective-scan decode elements(B\u00b7D\u00b7N per token)/s and achieved HBM GB/s",
        "value": elems / (eager_ms * 1e-3), "unit": "elements/s", "n_gpus": 1, "steps": L, "warmup": 1,
        "ms_per_step": round(eager_ms / L, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{name}: batch={B} d_inner={D} d_state={N}, {L} consecutive steps from a zero "
                               f"state, f32 (bf16-representable values)", "batch": B, "steps": L,
                   "d_inner": D, "d_state": N, "io_dtype": "f32"},
        "total_ms": {"eager": round(eager_ms, 3), "graph": round(graph_ms, 3)},
        "graph": {"value": elems / (graph_ms * 1e-3), "replays_bitwise_equal_eager": replays},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": "k_step",
                     "kernel_ms": round(kernel_ms, 4), "algorithmic_bytes_per_launch": per_step,
                     "copy_GBps": round(copy_gbps, 1), "frac_of_copy": round(gbps / copy_gbps, 4),
                     "cache_resident": "the 84 MB state (batch 256 x 5120 x 16 f32) fits the 256 MB "
                                       "Infinity Cache and is not flushed between steps (decode keeps it "
                                       "hot by design); byte counters count traffic past L2, which "
                                       "includes Infinity Cache hits, so this rate is not proof of HBM "
                                       "bandwidth"},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        rows = 96  # about 10 s of host work for the 1024 steps
        hs = np.zeros((rows, D, N))
        t0 = time.perf_counter()
        steps = 0
        while steps < L and time.perf_counter() - t0 < 20.0:
            sl = {k: tm[k][steps, :rows].cpu().numpy() for k in ("x", "z", "dt", "B", "C")}
            oracle.step(hs, sl["x"], sl["dt"], sl["B"], sl["C"], sl["z"], inp["A_log"], inp["D"], inp["dt_bias"])
            steps += 1
        sec = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": rows * D * N * steps / sec, "unit": "elements/s",
                                "cores": oracle.num_threads(), "kind": "oracle",
                                "sample": f"batch rows 0..{rows - 1}, all {D} channels, the first {steps} steps "
                                          f"of the same workload in f64 ({sec:.1f} s, host copies included)",
                                **host_cpu()}
    out = json.dumps(line)
    print(out, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(out + "\n")


MFMA_BF16_PEAK_TFLOPS = 2500.0


def block_bench(args):
    """One Mamba block, forward (training) + backward, 4 x 8192 tokens at d_model
    2560, d_inner 5120, dt_rank 160, d_conv 4, bf16 activations and projection
    weights."""
    import numpy as np
    import torch

    import selective_state_space_04_amd as ssm
    import workloads as W

    name = "block_mamba2p8b_bf16"
    cfg = W.BLOCK_CONFIGS[name]
    dev = torch.device("cuda:0")
    print(f"[bench] generating {name} inputs", file=sys.stderr, flush=True)
    X, p, dY = W.make_block_config(name)
    io = torch.bfloat16
    Xd, dYd = torch.from_numpy(X).to(dev).to(io), torch.from_numpy(dY).to(dev).to(io)
    pd = {k: torch.from_numpy(v).to(dev).to(io if k in ("W_in", "W_x", "W_dt", "W_out") else torch.float32)
          for k, v in p.items()}
    ctx = ssm.BlockContext()
    Y = torch.empty_like(Xd)
    grads = {}

    def step(timer=None):
        _, saved = ssm.ssm_block_fwd(ctx, Xd, pd, Y=Y, timing=timer)
        ssm.ssm_block_bwd(ctx, Xd, pd, saved, dYd, out=grads, timing=timer)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # every launch of the step (this library's kernels and each hipBLASLt GEMM,
    # logged as block_gemm) timed by events on the launch stream
    timers = [ssm.LaunchTimer() for _ in range(min(args.steps, 5))]
    for tm in timers:
        step(tm)
    torch.cuda.synchronize()
    per_kernel = {}
    nlaunch = []
    for tm in timers:
        res = tm.results()
        nlaunch.append(len(res))
        for kname, kms in res:
            per_kernel.setdefault(kname, []).append(kms)
        tm.close()
    if max(nlaunch) >= ssm.TIMING_MAX:
        raise SystemExit("the block step has more launches than the launch log holds")
    kavg = {k: float(np.sum(v)) / len(timers) for k, v in per_kernel.items()}
    gemm_ms = kavg.pop("block_gemm")
    ngemm = len(per_kernel["block_gemm"]) // len(timers)
    own_ms = sum(kavg.values())
    B, L, dm, di, R, N = cfg["batch"], cfg["seqlen"], cfg["d_model"], cfg["d_inner"], cfg["dt_rank"], cfg["d_state"]
    T = B * L
    P = R + 2 * N
    fwd_macs = T * (2 * di * dm + P * di + di * R + dm * di)
    gemm_flops = 2 * fwd_macs * 3  # forward, data gradients, weight gradients
    tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12
    line = {
        "metric": "Mamba block fwd+bwd tokens/s",
        "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{name}: batch={B} seqlen={L} d_model={dm} d_inner={di} d_state={N} "
                               f"dt_rank={R} d_conv={cfg['d_conv']}, bf16 activations and projection weights, "
                               f"f32 accumulation and scan state, fwd+bwd",
                   "batch": B, "seqlen": L, "d_model": dm, "d_inner": di, "dt_rank": R},
        "kernels_ms": {k: round(v, 4) for k, v in sorted(kavg.items())},
        "launch_sum_ms": {"own_kernels": round(own_ms, 4), "gemms": round(gemm_ms, 4),
                          "gaps": round(ms - own_ms - gemm_ms, 4)},
        "gemm": {"ms": round(gemm_ms, 4), "flops": gemm_flops,
                 "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                              "traffic": None,
                              "kernel": f"hipBLASLt GEMMs ({ngemm} per step, aggregate of their own launch "
                                        "times, HIP events on the launch stream)"}},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        from oracle.block import block_bwd
        # a prefix of batch row 0, doubled until one run takes at least 8 s
        Lp = 256
        while True:
            t0 = time.perf_counter()
            block_bwd(np.ascontiguousarray(X[:1, :Lp]), p, np.ascontiguousarray(dY[:1, :Lp]))
            sec = time.perf_counter() - t0
            if sec >= 8.0 or 2 * Lp > L:
                break
            Lp *= 2
        line["cpu_baseline"] = {"value": Lp / sec, "unit": "tokens/s", "cores": oracle.num_threads(),
                                "kind": "oracle",
                                "sample": f"batch row 0, the first {Lp} tokens of the same workload, forward "
                                          f"and backward in f64 ({sec:.1f} s)", **host_cpu()}
    ctx.close()
    out = json.dumps(line)
    print(out, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(out + "\n")


def train_bench(args):
    """Training steps/s of a one-block model (d_model = --dim, d_inner = 2 dim,
    d_state 16, dt_rank ceil(dim/16), d_conv 4, f32): each step gathers a batch of
    16 sequences x 128 tokens from a synthetic four-regime corpus, runs the block
    forward, the next-step MSE loss and its gradient, the block backward and one
    Adam update of all nine parameter tensors.  The block's forward and backward
    are this library's calls; the loss and Adam are plain PyTorch ops."""
    import numpy as np
    import torch

    import selective_state_space_04_amd as ssm
    import workloads as W

    dim, bsz, L, nseq = args.dim, 16, 128, 256
    di, R = 2 * dim, -(-dim // 16)
    dev = torch.device("cuda:0")
    Xc, Yc = W.make_regime_corpus(nseq, L, dim, seed=0)
    _, p0, _ = W.make_block_inputs(1, 1, dim, di, 16, R, 4, seed=1)
    params = {k: torch.from_numpy(v).to(dev).clone() for k, v in p0.items()}
    opt = torch.optim.Adam(list(params.values()), lr=2e-3, foreach=True)
    Xd, Yd = torch.from_numpy(Xc).to(dev), torch.from_numpy(Yc).to(dev)
    nsteps = args.warmup + args.steps
    order = torch.from_numpy(np.random.default_rng(2).integers(0, nseq, (nsteps, bsz))).to(dev)
    ctx = ssm.BlockContext()
    losses = []

    def step(i):
        xb, yb = Xd[order[i]], Yd[order[i]]
        Y, saved = ssm.ssm_block_fwd(ctx, xb, params)
        diff = Y - yb
        losses.append((diff * diff).mean())
        g = ssm.ssm_block_bwd(ctx, xb, params, saved, diff * (2.0 / diff.numel()))
        for k, t in params.items():
            t.grad = g["d" + k]
        opt.step()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.warmup, nsteps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    mse = [float(v) for v in losses]
    line = {
        "metric": "one-block training steps/s", "value": 1e3 / ms, "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"one Mamba block, d_model={dim} d_inner={di} d_state=16 dt_rank={R} d_conv=4, "
                               f"batch {bsz} x {L} tokens of a synthetic four-regime corpus, next-step MSE, "
                               f"Adam lr 2e-3, f32",
                   "d_model": dim, "batch": bsz, "seqlen": L},
        "mse_first": round(mse[0], 6), "mse_last": round(mse[-1], 6),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        from oracle.block import block_bwd
        idx = order[0].cpu().numpy()
        xb = np.ascontiguousarray(Xc[idx])
        dY = np.ones_like(xb) * np.float32(2.0 / xb.size)
        reps, t0 = 0, time.perf_counter()
        while reps < 500 and time.perf_counter() - t0 < 10.0:
            block_bwd(xb, p0, dY)  # forward and backward of one step's batch in f64
            reps += 1
        sec = (time.perf_counter() - t0) / reps
        line["cpu_baseline"] = {"value": 1.0 / sec, "unit": "steps/s", "cores": oracle.num_threads(),
                                "kind": "oracle",
                                "sample": f"{reps} block forward+backward passes of one step's batch in f64, "
                                          f"no optimizer ({sec * 1e3:.1f} ms each)", **host_cpu()}
    ctx.close()
    out = json.dumps(line)
    print(out, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(out + "\n")


MFMA_F32_PEAK_TFLOPS = 157.3


def gdn2_bench(args):
    """Gated DeltaNet-2 forward over batch 4 x 16 heads x 4096 tokens, k_dim =
    v_dim = 128, f32 (inputs resident on the GPU): the chunked WY form on MFMA
    (default) or, with --gdn2-form recurrent, the token recurrence."""
    import math

    import numpy as np
    import torch

    import selective_state_space_04_amd as ssm
    import workloads as W

    name = "gdn2_b4h16t4096"
    c = W.GDN2_CONFIGS[name]
    B, H, L, K, V = c["batch"], c["heads"], c["seqlen"], c["k_dim"], c["v_dim"]
    chunked = args.gdn2_form == "chunked"
    dev = torch.device("cuda:0")
    print(f"[bench] generating {name} inputs", file=sys.stderr, flush=True)
    inp = W.make_gdn2_config(name)
    names = ("q", "k", "v", "g", "b", "w")
    t = {n: torch.from_numpy(inp[n]).to(dev) for n in names}
    scale = 1.0 / math.sqrt(K)
    o = torch.empty(B, H, L, V, dtype=torch.float32, device=dev)
    fwd = ssm.ssm_gdn2_fwd_chunked if chunked else ssm.ssm_gdn2_fwd

    def step(timer=None):
        fwd(*[t[n] for n in names], None, scale=scale, o=o, return_state=False, timing=timer)

    if args.copy_probe:
        copy_probe(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timers = [ssm.LaunchTimer() for _ in range(args.steps)]
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(timers[i])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    per = {}
    for tm in timers:
        for kn, km in tm.results():
            per.setdefault(kn, []).append(km)
        tm.close()
    kavg = {kn: float(np.mean(v)) for kn, v in per.items()}
    ht = B * H * L                       # head-tokens
    nbytes = 4.0 * (4 * K + 3 * V) * ht  # q, k, g, b read; v, w read; o written (f32)
    if chunked:
        # MFMA work of the state pass as issued: per 64-token chunk and 16 columns,
        # 16x16x4 products for -BKe S and Qe S (4 K/4 each), M^-1 X and P vn (the 40
        # lower-triangular tiles each) and Kd^T vn (K/16 x 16), 2048 flops each
        dom = "k_gdn2_state"
        mfmas = (8 * (K // 4) + 80 + K) * (L // 64) * (V // 16) * B * H
        flops = 2048.0 * mfmas
        tflops = flops / (kavg[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_F32_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / MFMA_F32_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(dom, "gdn2_chunked"), "kernel": dom,
                "kernel_ms": round(kavg[dom], 4), "flops_per_launch": flops,
                "key_side_traffic": measured_traffic("k_gdn2_wy", "gdn2_chunked"),
                "note": "f32 MFMA (v_mfma_f32_16x16x4f32) work of the state pass as issued; traffic = "
                        "counted HBM bytes per launch of the state pass (key side beside it)"}
        form = "chunked WY form, 64-token chunks, products on MFMA"
    else:
        dom = "k_gdn2_fwd"
        flops = 7.0 * K * V * ht  # decay mul, erase-read, write and output FMAs per state element
        tflops = flops / (kavg[dom] * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": round(tflops, 2), "peak": 78.6, "unit": "TFLOP/s",
                "frac": round(tflops / 78.6, 4), "traffic": measured_traffic("k_gdn2_fwd", "gdn2"), "kernel": dom,
                "kernel_ms": round(kavg[dom], 4),
                "note": "f32 vector FMA peak without packed math (256 CUs x 64 lanes x 2 flops x 2.4 GHz)"}
        form = "token-by-token recurrence"
    line = {
        "metric": "GDN2 forward tokens/s", "value": B * L / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{name}: batch={B} heads={H} seqlen={L} k_dim={K} v_dim={V}, f32, forward "
                               f"(gated delta rule, {form})",
                   "batch": B, "heads": H, "seqlen": L, "k_dim": K, "v_dim": V},
        "kernels_ms": {kn: round(v, 4) for kn, v in sorted(kavg.items())},
        "roofline": roof,
        "hbm": {"algorithmic_bytes": nbytes, "achieved_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "frac": round(nbytes / (ms * 1e-3) / 8e12, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        from oracle import gdn2
        # whole (batch, head) sequences one after another, until at least 10 s
        npairs, sec = 0, 0.0
        while npairs < 10000 and sec < 10.0:
            bi, hi = (npairs // H) % B, npairs % H
            sub = [inp[n][bi:bi + 1, hi:hi + 1] for n in names]
            t0 = time.perf_counter()
            gdn2.recurrent(*sub, None, scale)
            sec += time.perf_counter() - t0
            npairs += 1
        line["cpu_baseline"] = {"value": npairs * L / H / sec, "unit": "tokens/s", "cores": oracle.num_threads(),
                                "kind": "oracle",
                                "sample": f"{npairs} whole (batch, head) sequences of {L} tokens in f64 "
                                          f"({sec:.1f} s), scaled to all {H} heads of a token", **host_cpu()}
    out = json.dumps(line)
    print(out, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(out + "\n")


def block_c_bench(args):
    """The block_mamba2p8b_bf16 workload (fwd+bwd) timed by tests/c_abi/block_from_c,
    a C++ program that calls libssmblock.so with no PyTorch in its process, so the
    projections run on the system ROCm hipBLASLt.  Its inputs are uniform random
    values of the same shapes and scales (its own generator)."""
    import subprocess

    import workloads as W

    exe = os.path.join(ROOT, "tests", "c_abi", "block_from_c")
    if not os.path.exists(exe):
        raise SystemExit(f"{exe} is missing: build the package first")
    res = subprocess.run([exe, "time", str(args.steps), str(args.warmup)], capture_output=True, text=True,
                         timeout=600)
    if res.returncode != 0:
        raise SystemExit(f"block_from_c failed ({res.returncode}): {res.stdout}{res.stderr}")
    ms = float(res.stdout.split()[-1])
    cfg = W.BLOCK_CONFIGS["block_mamba2p8b_bf16"]
    B, L = cfg["batch"], cfg["seqlen"]
    line = {
        "metric": "Mamba block fwd+bwd tokens/s (C caller, system ROCm libraries)",
        "value": B * L / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"block_mamba2p8b_bf16: batch={B} seqlen={L} d_model={cfg['d_model']} "
                               f"d_inner={cfg['d_inner']} d_state=16 dt_rank={cfg['dt_rank']} d_conv=4, bf16, "
                               f"fwd+bwd, driven from a C++ program",
                   "batch": B, "seqlen": L, "d_model": cfg["d_model"], "d_inner": cfg["d_inner"]},
        "cpu_baseline": None,
    }
    out = json.dumps(line)
    print(out, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(out + "\n")


# Algorithmic bytes per launch of the kernels that carry a pass's compulsory
# traffic (every input read once, every output written once); carries, chunk
# passes and reductions only add overhead on top of these.
def kernel_alg_bytes(kernel, cfg, esz):
    ab = algorithmic_bytes(cfg, esz)
    if kernel.startswith("k_fwd_main") or kernel.startswith("k_fwd_state"):
        return ab["fwd_main"]
    if kernel.startswith("k_bwd_main") or kernel.startswith("k_bwd_tile"):
        return ab["bwd_main"]
    return None


def host_cpu():
    """The host's CPU model and the cores this process may use."""
    model = None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "cores_available": avail}


class CacheFlush:
    """Reads 512 MiB (twice the 256 MB Infinity Cache) of unrelated data, so
    that what a timed pass reads comes from HBM.  A read, not a write: a
    written flush would leave the caches full of dirty lines that the timed
    pass then pays to write back."""

    def __init__(self, dev):
        import torch
        self.buf = torch.ones(1 << 27, dtype=torch.float32, device=dev)
        self.sink = torch.empty((), dtype=torch.float32, device=dev)

    def __call__(self):
        import torch
        torch.sum(self.buf, dim=0, out=self.sink)


def copy_bandwidth(dev, nbytes=1 << 30, reps=5):
    """Read+write GB/s of a plain device copy of nbytes (best of reps): the
    attainable-bandwidth reference the HBM fraction is also reported against."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del src, dst
    return 2 * nbytes / (best * 1e-3) / 1e9


def counted_valu(kernel, op="scan"):
    """(VALU lane instructions, transcendental lane instructions) per launch of
    `kernel` from the committed SQ counter summary, or None when it was taken on
    another kernel source."""
    import hashlib
    src_path, _ = TRAFFIC[op]
    path = os.path.join(ROOT, "profiles", "c4_mamba2p8b_bf16_valu.txt")
    try:
        lines = open(path).read().split("\n")
        src = hashlib.sha256(open(src_path, "rb").read()).hexdigest()
    except OSError:
        return None
    kv = {}
    for ln in lines:
        parts = ln.split()
        if len(parts) >= 2 and not ln.startswith("#"):
            kv[parts[0]] = parts[1:]
    if kv.get("source_sha256", [None])[0] != src or kernel not in kv:
        return None
    f = dict(p.split("=") for p in kv[kernel])
    return float(f["valu_wave_insts"]) * 64, float(f["trans_wave_insts"]) * 64


# One SIMD issues one wave64 VALU instruction per 4 cycles (16 lanes wide), so
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 3.93e13 lane instructions per second
# without packed FP32 (which this library does not use).
VALU_LANE_PEAK = 256 * 4 * 16 * 2.4e9


def cpu_scan_baseline(inp, cfg, passes, budget_s=12.0):
    """The oracle on the host cores: the whole workload when it fits the time
    budget (repeated when tiny), else the leading batch rows that fit."""
    import numpy as np

    import oracle
    bsz, L, D = inp["x"].shape
    N = cfg["d_state"]
    bwd = "bwd" in passes

    def run(rows):  # (seconds for the whole pass, seconds for its forward)
        sub = {k: inp[k][:rows] for k in ("x", "z", "dt", "B", "C") + (("dy",) if bwd else ())}
        t0 = time.perf_counter()
        oracle.fwd(sub["x"], sub["dt"], sub["B"], sub["C"], sub["z"], inp["A_log"], inp["D"], inp["dt_bias"])
        t1 = time.perf_counter()
        if bwd:
            oracle.bwd(sub["x"], sub["dt"], sub["B"], sub["C"], sub["z"], inp["A_log"], inp["D"], inp["dt_bias"],
                       sub["dy"])
        return time.perf_counter() - t0, t1 - t0

    per_row = max(run(1)[0], 1e-6)
    if per_row * bsz <= budget_s:
        # the whole workload, repeated until at least 10 s of host work
        reps, sec, fsec = 0, 0.0, 0.0
        while reps < 100000 and sec < 10.0:
            a, f = run(bsz)
            sec, fsec = sec + a, fsec + f
            reps += 1
        rows, what = bsz, f"the whole workload ({bsz} rows), {reps} run(s)"
    else:
        rows = max(1, min(bsz, int(budget_s / per_row)))
        reps = 1
        sec, fsec = run(rows)
        what = f"batch rows 0..{rows - 1} of {bsz}, all {L} tokens and {D} channels"
    elems = reps * rows * L * D * N
    out = {"value": elems / sec, "unit": "elements/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"{what}, {'fwd+bwd' if bwd else 'fwd'} in f64 ({elems} elements, {sec:.1f} s)",
           **host_cpu()}
    if bwd:  # the same runs' forward alone
        out["fwd_value"] = elems / fsec
    return out


def scan_bench(args):
    import numpy as np
    import torch

    import selective_state_space_04_amd as ssm
    import workloads as W

    cfg = W.CONFIGS[args.config]
    passes = cfg["passes"]
    bwd = "bwd" in passes
    dev = torch.device("cuda:0")
    io = torch.bfloat16 if cfg["io"] == "bf16" else torch.float32
    esz = 2 if io == torch.bfloat16 else 4
    print(f"[bench] generating {args.config} inputs", file=sys.stderr, flush=True)
    inp = W.make_config(args.config)
    t = {}
    for k in ("x", "z", "dt", "B", "C") + (("dy",) if bwd else ()):
        t[k] = torch.from_numpy(inp[k]).to(dev).to(io)
    for k in ("A_log", "D", "dt_bias"):
        t[k] = torch.from_numpy(inp[k]).to(dev)
    bsz, L, D = inp["x"].shape
    N = cfg["d_state"]
    grads = {"dx": torch.empty_like(t["x"]), "ddt": torch.empty_like(t["x"]), "dz": torch.empty_like(t["x"]),
             "dB": torch.empty_like(t["B"]), "dC": torch.empty_like(t["C"]),
             "dA_log": torch.empty_like(t["A_log"]), "dD": torch.empty_like(t["D"]),
             "ddt_bias": torch.empty_like(t["dt_bias"]), "dh0": None}
    y = torch.empty_like(t["x"])

    def step(timer=None, mid=None):
        _, _, ckpt = ssm.ssm_scan_fwd(t["x"], t["dt"], t["B"], t["C"], t["z"], t["A_log"], t["D"],
                                      t["dt_bias"], training=bwd, y=y, timing=timer)
        if mid is not None:
            mid.record()
        if bwd:
            ssm.ssm_scan_bwd(t["x"], t["dt"], t["B"], t["C"], t["z"], t["A_log"], t["D"], t["dt_bias"], ckpt,
                             t["dy"], out=grads, timing=timer)

    if args.copy_probe:
        copy_probe(dev)
    copy_gbps = copy_bandwidth(dev)
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Flushed: a cache flush between steps, outside each step's events, so that
    # every step starts from cold caches.
    flush = CacheFlush(dev)
    timers = [ssm.LaunchTimer() for _ in range(args.steps)]
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush()
        ev[i][0].record()
        step(timers[i], mid=ev[i][1])
        ev[i][2].record()
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(c) for a, _, c in ev]
    fwd_ms = [a.elapsed_time(m) for a, m, _ in ev]
    ms = float(np.mean(step_ms))
    # Unflushed: the same steps back to back.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_hot = e0.elapsed_time(e1) / args.steps
    del flush
    per_kernel = {}
    for tm in timers:
        for name, kms in tm.results():
            per_kernel.setdefault(name, []).append(kms)
    for tm in timers:
        tm.close()
    kavg = {k: float(np.mean(v)) for k, v in per_kernel.items()}
    kcount = {k: len(v) // args.steps for k, v in per_kernel.items()}
    dominant = max(kavg, key=lambda k: kavg[k] * kcount[k])
    ab = algorithmic_bytes(cfg, esz)
    step_bytes = ab["fwd"] + (ab["bwd"] if bwd else 0)
    elems = bsz * L * D * N
    dom_bytes = kernel_alg_bytes(dominant, cfg, esz)
    roof = valu = None
    if dom_bytes is not None:
        sec = kavg[dominant] * 1e-3
        # the committed byte counters were taken on the 2.8B-shaped workload only
        traffic = measured_traffic(dominant) if args.config == "c4_mamba2p8b_bf16" else None
        gbps = dom_bytes / sec / 1e9
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": dominant,
                "kernel_ms": round(kavg[dominant], 4), "algorithmic_bytes_per_launch": dom_bytes,
                "traffic_over_algorithmic": None if traffic is None else round(traffic / dom_bytes, 3),
                "copy_GBps": round(copy_gbps, 1), "frac_of_copy": round(gbps / copy_gbps, 4)}
        cv = counted_valu(dominant) if args.config == "c4_mamba2p8b_bf16" else None
        if cv is not None:
            lane, trans = cv
            valu = {"kernel": dominant, "lane_insts_per_element": round(lane / elems, 2),
                    "trans_lane_insts_per_element": round(trans / elems, 2),
                    "achieved_lane_insts_per_s": lane / sec, "peak_lane_insts_per_s": VALU_LANE_PEAK,
                    "frac": round(lane / sec / VALU_LANE_PEAK, 4),
                    "note": "SQ_INSTS_VALU x 64 from the committed counters; peak = one wave64 VALU "
                            "instruction per SIMD per 4 cycles at 2.4 GHz, no packed FP32"}
    work = "fwd+bwd" if bwd else "fwd (inference: no checkpoints)"
    line = {
        "metric": "selective-scan fwd+bwd elements(B\u00b7L\u00b7D\u00b7N)/s and achieved HBM GB/s",
        "value": elems / (ms * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: batch={bsz} seqlen={L} d_inner={D} d_state={N}, "
                               f"{cfg['io']} activations, f32 state, {work}",
                   "batch": bsz, "seqlen": L, "d_inner": D, "d_state": N, "io_dtype": cfg["io"], "passes": work},
        "timing": {"ms_per_step_flushed": round(ms, 4), "ms_per_step_unflushed": round(ms_hot, 4),
                   "ms_per_step_flushed_median": round(float(np.median(step_ms)), 4),
                   "ms_fwd_flushed": round(float(np.mean(fwd_ms)), 4),
                   "ms_bwd_flushed": round(float(np.mean([s - f for s, f in zip(step_ms, fwd_ms)])), 4)
                   if bwd else None,
                   "flush": "512 MiB read between timed steps, outside each step's events; the backward "
                            "follows its forward without a flush"},
        "inputs": {"generator": "numpy default_rng(seed) (PCG64)", "seed": 0, "numpy": np.__version__},
        "step_hbm": {"algorithmic_bytes": step_bytes, "achieved_GBps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
                     "frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "frac_of_copy": round(step_bytes / (ms * 1e-3) / 1e9 / copy_gbps, 4)},
        "kernels_ms": {k: round(v, 4) for k, v in sorted(kavg.items())},
        "roofline": roof,
        "valu": valu,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_scan_baseline(inp, cfg, passes)
    s = json.dumps(line)
    print(s, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(s + "\n")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the scan is measured on a "
              f"single MI355X and multi-GPU sharding is design-only.", file=sys.stderr)
        sys.exit(2)
    if args.op == "scan" and args.config == "c5_decode_step":
        args.op = "decode"
    ops = {"conv1d": conv_bench, "decode": decode_bench, "block": block_bench, "train": train_bench,
           "block-c": block_c_bench, "gdn2": gdn2_bench, "scan": scan_bench}
    ops[args.op](args)


if __name__ == "__main__":
    main()
