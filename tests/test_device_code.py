"""CPU check of the built device code: disassemble every gfx950 code object in
the library and assert that no instruction writes through the scalar data
cache (scalar stores, scalar atomics, scalar cache write-back or discard).
All writes of the kernels must be vector memory instructions."""

import re
import shutil
import subprocess
from pathlib import Path

import pytest

from mamba_mimo_chunked_amd._lib import LIB_PATH

LLVM = Path("/opt/rocm/llvm/bin")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
FORBIDDEN = re.compile(r"\bs_(store|scratch_store|buffer_store|atomic|buffer_atomic|dcache_wb|dcache_discard)\w*")


@pytest.mark.skipif(not (LLVM / "llvm-objdump").exists() or not LIB_PATH.exists(),
                    reason="ROCm LLVM tools or the built library missing")
def test_no_scalar_cache_writes(tmp_path):
    fb = tmp_path / "fatbin.bin"
    subprocess.run([str(LLVM / "llvm-objcopy"), f"--dump-section=.hip_fatbin={fb}", str(LIB_PATH),
                    str(tmp_path / "stripped.so")], check=True)
    data = fb.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    assert starts, "no offload bundles in the library"
    n_objects = 0
    for k, st in enumerate(starts):
        en = starts[k + 1] if k + 1 < len(starts) else len(data)
        part = tmp_path / f"b{k}.bin"
        part.write_bytes(data[st:en])
        co = tmp_path / f"c{k}.co"
        r = subprocess.run([str(LLVM / "clang-offload-bundler"), "--unbundle", "--type=o", f"--input={part}",
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        dis = subprocess.run([str(LLVM / "llvm-objdump"), "-d", str(co)], capture_output=True, text=True,
                             check=True).stdout
        hits = FORBIDDEN.findall(dis)
        assert not hits, f"code object {k}: scalar-cache writes {sorted(set(hits))}"
        n_objects += 1
    assert n_objects >= 10
