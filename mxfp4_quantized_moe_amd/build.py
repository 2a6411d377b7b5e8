"""Build libmxmoe.so (the C-ABI HIP library) in-tree for gfx950.

    python -m mxfp4_quantized_moe_amd.build

compiles every source under csrc/ with hipcc and links one shared library
next to this file.  hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxmoe.so")
SOURCES = ["moe_gemm.hip", "routing.hip", "api.hip", "codec.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 arithmetic stays off: its encodings are avoided on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


def _run(cmd, verbose: bool) -> str:
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=1800)
    except subprocess.TimeoutExpired as e:
        raise RuntimeError(f"hipcc did not finish within {e.timeout:.0f} s") from e
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel, one object each) and link the
    library; returns its path.  Raises on failure."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    inc = ["-I", os.path.join(HERE, "..", "include")]
    with tempfile.TemporaryDirectory(prefix="mxmoe_build_") as tmpdir:
        objs = [os.path.join(tmpdir, s + ".o") for s in SOURCES]
        cflags = [f for f in FLAGS if f != "-shared"]
        cmds = [[HIPCC, *cflags, *inc, "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as pool:
            errs = list(pool.map(lambda c: _run(c, verbose), cmds))
        tmp = LIB + ".tmp"
        errs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose))
    err = "\n".join(e for e in errs if e.strip())
    if verbose and err:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
