"""Build libsplash.so (HIP kernels for gfx950 + host mask compiler + C ABI)
and libsplash_probe.so (MFMA-throughput and HBM-read probes the benchmark reports
beside the nominal peaks; not part of the attention path).

Run `python -m block_sparse_attention_make_amd.build` (or call build()).  The
library lands in block_sparse_attention_make_amd/lib/, next to the binding
that loads it.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libsplash.so")
PROBE_PATH = os.path.join(LIB_DIR, "libsplash_probe.so")
SOURCES = ["splash_fwd.hip", "splash_bwd.hip", "splash_decode.hip", "lse_merge.hip", "capi.cpp", "mask_info.cpp"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def command(out_path=LIB_PATH, sources=SOURCES):
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-fvisibility=hidden",
        # packed-fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        *[os.path.join(CSRC, s) for s in sources],
        "-o", out_path,
    ]


def _run(out_path, sources, verbose):
    tmp = out_path + ".tmp"
    cmd = command(tmp, sources)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"{os.path.basename(out_path)} build failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    os.replace(tmp, out_path)
    if verbose:
        print(" ".join(cmd))


def build(verbose=False):
    os.makedirs(LIB_DIR, exist_ok=True)
    _run(LIB_PATH, SOURCES, verbose)
    _run(PROBE_PATH, ["mfma_probe.hip"], verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
