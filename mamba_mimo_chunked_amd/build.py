"""Build the HIP library ``libmimo_bwd_fwd.so`` for gfx950 with hipcc.

The library is built in-tree (``mamba_mimo_chunked_amd/_build/``) so that it
travels with the source tree; nothing is installed. ``python -m
mamba_mimo_chunked_amd.build`` (or ``__graft_entry__.build()``) rebuilds it.
"""

from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
SOURCES = (["mimo_bwd_fwd.hip"] + [f"b2_{t}.hip" for t in ("bf16", "f16", "f32")]
           + [f"tiles_f32_mt{m}.hip" for m in (32, 64, 128)]
           + [f"tiles_rp{r}_ct{c}.hip" for r, c in
              ((1, 1), (1, 2), (1, 4), (2, 1), (2, 2), (2, 4), (4, 1), (4, 2), (8, 1))])
INCLUDE = ROOT / "include"
OUT_DIR = PKG / "_build"
LIB = OUT_DIR / "libmimo_bwd_fwd.so"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed fp32 arithmetic (v_pk_{add,mul,fma}_f32) in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
]


def _check(res, what):
    if res.returncode != 0:
        # the host pass warns that it does not know the packed-fp32 feature; drop that noise
        err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc failed on {what} ({res.returncode}):\n{err}")


def build(verbose: bool = False) -> Path:
    """Compile the library (always): every translation unit in parallel, then
    link. Returns the path of the shared object."""
    OUT_DIR.mkdir(exist_ok=True)
    objs, procs = [], []
    for name in SOURCES:
        obj = OUT_DIR / (Path(name).stem + ".o")
        cmd = [HIPCC, *FLAGS, "-c", f"-I{INCLUDE}", str(CSRC / name), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((name, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    for name, pr in procs:
        out, err = pr.communicate()
        _check(subprocess.CompletedProcess(pr.args, pr.returncode, out, err), name)
    tmp = LIB.with_suffix(f".so.tmp{os.getpid()}")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    _check(subprocess.run(cmd, capture_output=True, text=True), "link")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
