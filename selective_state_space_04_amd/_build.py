"""Compiles libssmscan.so (HIP, gfx950 only: the selective scan, the conv1d in
front of it and the Gated DeltaNet-2 forward) and libssmblock.so (one Mamba block: those kernels plus the
projections on hipBLASLt) in-tree with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", n)
        for n in ("ssm_scan.hip", "ssm_conv1d.hip", "ssm_gdn2.hip", "ssm_gdn2_chunk.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libssmscan.so")
BLOCK_SRC = os.path.join(HERE, "csrc", "ssm_block.hip")
BLOCK_LIB_PATH = os.path.join(HERE, "libssmblock.so")
ROCM_LIB = "/opt/rocm/lib"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",  # every fused multiply-add is written out explicitly
    # no packed-FP32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def _hipcc(cmd, out, verbose):
    tmp = out + ".tmp"
    cmd = cmd + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, out)


C_DRIVERS = [(os.path.join(ROOT, "tests", "c_abi", n + ".cpp"), os.path.join(ROOT, "tests", "c_abi", n), lib)
             for n, lib in (("scan_from_c", ["-lssmscan"]), ("block_from_c", ["-lssmblock", "-lssmscan"]))]


def build(verbose=False, extra=()):
    """libssmscan.so (scan, conv1d and GDN2 kernels), then libssmblock.so (the
    Mamba block on top of it and hipBLASLt), then the host-only test programs that
    drive the two libraries through their C ABI."""
    _hipcc([HIPCC, *FLAGS, *extra, "-I", INCLUDE, *SRCS], LIB_PATH, verbose)
    _hipcc([HIPCC, *FLAGS, *extra, "-I", INCLUDE, BLOCK_SRC, "-L", HERE, "-lssmscan",
            f"-L{ROCM_LIB}", "-lhipblaslt", "-Wl,-rpath,$ORIGIN", f"-Wl,-rpath,{ROCM_LIB}"],
           BLOCK_LIB_PATH, verbose)
    for src, out, lib in C_DRIVERS:
        _hipcc([HIPCC, "-O2", "-std=c++17", "-Wall", "-I", INCLUDE, src, "-L", HERE, *lib,
                "-Wl,-rpath,$ORIGIN/../../selective_state_space_04_amd", f"-Wl,-rpath,{ROCM_LIB}"],
               out, verbose)
    return LIB_PATH
