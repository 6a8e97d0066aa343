"""Build the GPU test helpers (``tests/helpers/_build/liblds_fill.so``) for gfx950."""
import os
import subprocess
from pathlib import Path

HERE = Path(__file__).resolve().parent
LIB = HERE / "_build" / "liblds_fill.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> Path:
    LIB.parent.mkdir(exist_ok=True)
    tmp = LIB.with_suffix(f".so.tmp{os.getpid()}")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           str(HERE / "lds_fill.hip"), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc failed on lds_fill.hip ({res.returncode}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
