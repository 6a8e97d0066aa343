"""Host-side checks of the boundary (no GPU needed).

* the C library loads and exports every entry point include/mimo_bwd_fwd.h declares;
* the ctypes mirror of ``mimo_bwd_fwd_args`` has the C layout (gcc reports it);
* the workspace-size query validates shapes like the call does;
* the Python entry point raises the pages' errors, in the pages' order, before
  touching a device (the pages' three invalid-input tests use CPU tensors).
"""

import ctypes
import re
import subprocess
from pathlib import Path

import pytest
import torch

from mamba_mimo_chunked_amd import _lib, mamba_mimo_bwd_fwd, workspace_size
from synth.inputs import Case, api_args, make_inputs

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "mimo_bwd_fwd.h"


def test_library_exports_every_declared_symbol():
    decl = set(re.findall(r"^\w[\w\s\*]*?\b(mimo_\w+)\s*\(", HEADER.read_text(), re.M))
    assert decl == set(_lib.EXPORTED)
    L = _lib.lib()
    for name in decl:
        assert hasattr(L, name), name
    assert L.mimo_abi_version() == _lib.ABI_VERSION
    out = subprocess.run(["nm", "-D", "--defined-only", str(_lib.LIB_PATH)], capture_output=True,
                         text=True, check=True).stdout
    for name in decl:
        assert re.search(rf"\bT {name}$", out, re.M), name


@pytest.mark.parametrize("cls,cname", [(_lib.MimoBwdFwdArgs, "mimo_bwd_fwd_args"),
                                        (_lib.MimoFwdArgs, "mimo_fwd_args"),
                                        (_lib.MimoSisoFwdArgs, "mimo_siso_fwd_args"),
                                        (_lib.MimoBwdBwdArgs, "mimo_bwd_bwd_args")])
def test_struct_layout_matches_c(tmp_path, cls, cname):
    fields = [f[0] for f in cls._fields_]
    prog = ["#include <stddef.h>", "#include <stdio.h>", '#include "mimo_bwd_fwd.h"', "int main(void){",
            f'printf("%zu\\n", sizeof({cname}));']
    prog += [f'printf("%zu\\n", offsetof({cname}, {f}));' for f in fields]
    prog += ["return 0;}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(prog))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", f"-I{ROOT / 'include'}", str(src), "-o", str(exe)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(cls)
    for f, off in zip(fields, vals[1:]):
        assert getattr(cls, f).offset == off, f


def test_workspace_size_query():
    assert workspace_size(1, 16, 2, 1, 2, 16, 16, 16) == 0          # one chunk: no scratch
    assert workspace_size(1, 64, 2, 1, 2, 16, 16, 16) > 0
    big = workspace_size(1, 8192, 16, 1, 4, 64, 64, 16)
    assert big > 0 and big % 256 == 0
    with pytest.raises(ValueError, match="chunk_size"):
        workspace_size(1, 64, 2, 1, 16, 16, 16, 16)                   # C*R = 256
    with pytest.raises(ValueError, match="rotary"):
        workspace_size(1, 64, 2, 1, 2, 16, 16, 16, 3)
    with pytest.raises(ValueError, match="divisible by G"):
        workspace_size(1, 64, 3, 2, 2, 16, 16, 16)
    with pytest.raises(NotImplementedError, match="multiple of 16"):
        workspace_size(1, 64, 2, 1, 2, 24, 16, 16)
    with pytest.raises(NotImplementedError, match="chunk_size above 64"):
        workspace_size(1, 256, 1, 1, 1, 16, 16, 128)


def test_c_call_rejects_bad_arguments_without_a_device():
    """Argument errors are reported before the library looks at the device."""
    L = _lib.lib()
    a = _lib.MimoBwdFwdArgs()
    a.B, a.S, a.H, a.G, a.R, a.N, a.P = 1, 64, 2, 1, 2, 16, 16
    a.chunk_size, a.rotary_dim_divisor = 16, 4
    assert L.mimo_bwd_fwd(ctypes.byref(a), None) == _lib.MIMO_ERR_VALUE   # NULL inputs
    assert "NULL" in _lib.last_error()
    assert L.mimo_bwd_fwd(None, None) == _lib.MIMO_ERR_VALUE


def test_fp32_and_siso_argument_checks_without_a_device():
    """The fp32-intermediate and SISO entry points reject bad sizes before any device work."""
    L = _lib.lib()
    a = _lib.MimoBwdFwdArgs()
    a.B, a.S, a.H, a.G, a.R, a.N, a.P = 1, 300, 2, 1, 8, 128, 128
    a.chunk_size, a.rotary_dim_divisor = 16, 4
    n = ctypes.c_size_t(0)
    # the largest tiles of the range fit (K~ in scratch when the LDS cannot hold it)
    assert L.mimo_bwd_fwd_f32_workspace_size(ctypes.byref(a), ctypes.byref(n)) == _lib.MIMO_OK
    a.chunk_size = 32   # R * chunk_size = 256: outside the API's range
    assert L.mimo_bwd_fwd_f32_workspace_size(ctypes.byref(a), ctypes.byref(n)) == _lib.MIMO_ERR_VALUE
    assert "chunk_size * R" in _lib.last_error()
    a.chunk_size, a.N = 16, 144
    assert L.mimo_bwd_fwd_f32_workspace_size(ctypes.byref(a), ctypes.byref(n)) == _lib.MIMO_ERR_UNSUPPORTED
    assert "N must be" in _lib.last_error()
    a.R, a.N, a.P = 4, 64, 64
    assert L.mimo_bwd_fwd_f32_workspace_size(ctypes.byref(a), ctypes.byref(n)) == _lib.MIMO_OK
    assert L.mimo_bwd_fwd_f32(ctypes.byref(a), None) == _lib.MIMO_ERR_VALUE   # NULL inputs
    s = _lib.MimoSisoFwdArgs()
    s.B, s.S, s.Hq, s.H, s.K, s.V, s.A = 1, 128, 2, 4, 64, 96, 32
    for c, err in ((48, _lib.MIMO_ERR_VALUE), (32, _lib.MIMO_OK), (64, _lib.MIMO_OK)):
        s.chunk_size = c
        assert L.mimo_siso_fwd_workspace_size(ctypes.byref(s), ctypes.byref(n)) == err, c
    s.A = 33
    assert L.mimo_siso_fwd_workspace_size(ctypes.byref(s), ctypes.byref(n)) == _lib.MIMO_ERR_VALUE
    s.A, s.Hq = 32, 3
    assert L.mimo_siso_fwd_workspace_size(ctypes.byref(s), ctypes.byref(n)) == _lib.MIMO_ERR_VALUE
    s.Hq, s.dtype = 2, 7
    assert L.mimo_siso_fwd_workspace_size(ctypes.byref(s), ctypes.byref(n)) == _lib.MIMO_ERR_TYPE
    s.dtype = _lib.DTYPE_FP16
    assert L.mimo_siso_fwd(ctypes.byref(s), None) == _lib.MIMO_ERR_VALUE      # NULL inputs


def test_bwd_bwd_argument_checks_without_a_device():
    """The stage-2 entry point rejects shapes beyond its tiles and misaligned rows
    before any device work."""
    L = _lib.lib()
    a = _lib.MimoBwdBwdArgs()
    a.B, a.S, a.H, a.G, a.R, a.N, a.P = 1, 8192, 16, 1, 4, 64, 64
    a.chunk_size, a.rotary_dim_divisor = 16, 4
    n = ctypes.c_size_t(0)
    assert L.mimo_bwd_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n)) == _lib.MIMO_OK
    for field, val in (("N", 60), ("P", 60), ("N", 136), ("P", 136), ("R", 16)):
        old = getattr(a, field)
        setattr(a, field, val)
        if field == "R":
            a.chunk_size = 4
        assert L.mimo_bwd_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n)) == _lib.MIMO_ERR_UNSUPPORTED, field
        assert "multiples of 8" in _lib.last_error()
        setattr(a, field, old)
        a.chunk_size = 16
    # every pointer present, one input row start 8 bytes off
    for f, typ in _lib.MimoBwdBwdArgs._fields_:
        if typ is ctypes.c_void_p and f not in ("d", "dd", "workspace"):
            setattr(a, f, 1 << 20)
    a.S = 16                    # one chunk: no workspace
    a.q = (1 << 20) + 8
    assert L.mimo_bwd_bwd(ctypes.byref(a), None) == _lib.MIMO_ERR_VALUE
    assert "16-byte aligned" in _lib.last_error()


@pytest.mark.parametrize("chunk", [48, 0, True, 64.0, "64"])
def test_siso_invalid_chunk_size(chunk):
    """chunk_size must be the int 32 or 64 (not a bool, a float or another int)."""
    from mamba_mimo_chunked_amd import mamba3_siso_fwd
    from synth.inputs import SISO_CONFIGS, SISO_ORDER, make_siso_inputs
    inp = make_siso_inputs(SISO_CONFIGS["siso_example"])
    with pytest.raises(ValueError, match="chunk_size"):
        mamba3_siso_fwd(*[inp[n] for n in SISO_ORDER], chunk_size=chunk)


def test_siso_cpu_tensors_are_rejected():
    from mamba_mimo_chunked_amd import mamba3_siso_fwd
    from synth.inputs import SISO_CONFIGS, SISO_ORDER, make_siso_inputs
    inp = make_siso_inputs(SISO_CONFIGS["siso_example"])
    with pytest.raises(ValueError, match="GPU"):
        mamba3_siso_fwd(*[inp[n] for n in SISO_ORDER], chunk_size=64)


# -------------------------------------------------------------- the pages' invalid-input tests
def _args(**kw):
    inp = make_inputs(Case(1, 16, 1, 1, 64, 64, 4, 16, recipe="ut", has_z=False, has_d=False, **kw))
    return list(api_args(inp))


def test_invalid_q_shape():
    args = _args()
    args[1] = torch.randn((1, 16, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="q must have shape"):
        mamba_mimo_bwd_fwd(*args)


def test_invalid_empty_batch():
    args = list(api_args(make_inputs(Case(0, 16, 1, 1, 64, 64, 4, 16, recipe="ut", has_z=False,
                                          has_d=False))))
    with pytest.raises(ValueError, match="B, S, R and G must be positive"):
        mamba_mimo_bwd_fwd(*args)


def test_invalid_q_dtype():
    args = _args()
    args[1] = args[1].to(torch.float16)
    with pytest.raises(TypeError, match="torch.bfloat16"):
        mamba_mimo_bwd_fwd(*args)


def test_cpu_tensors_are_rejected():
    with pytest.raises(ValueError, match="GPU"):
        mamba_mimo_bwd_fwd(*_args())


def _stage1_args(S=64):
    """Stage-1 arguments with every pointer set to a fake, 256-byte aligned address:
    enough for the checks that come before any device work."""
    a = _lib.MimoBwdFwdArgs()
    a.B, a.S, a.H, a.G, a.R, a.N, a.P = 1, S, 2, 1, 2, 16, 16
    a.chunk_size, a.rotary_dim_divisor = 16, 4
    for f, typ in _lib.MimoBwdFwdArgs._fields_:
        if typ is ctypes.c_void_p and f not in ("workspace",):
            setattr(a, f, 1 << 20)
    return a


@pytest.mark.parametrize("field", ["dout", "q", "k", "v", "z", "states", "qk_dot", "dz"])
def test_c_call_rejects_misaligned_rows_without_a_device(field):
    L = _lib.lib()
    a = _stage1_args(S=16)      # one chunk: no workspace
    setattr(a, field, (1 << 20) + 8)
    assert L.mimo_bwd_fwd(ctypes.byref(a), None) == _lib.MIMO_ERR_VALUE
    assert "16-byte aligned" in _lib.last_error()
    assert L.mimo_bwd_fwd_f32(ctypes.byref(a), None) == _lib.MIMO_ERR_VALUE
    assert "16-byte aligned" in _lib.last_error()


def test_c_call_rejects_small_or_misaligned_workspace_without_a_device():
    L = _lib.lib()
    a = _stage1_args(S=300)
    need = ctypes.c_size_t(0)
    assert L.mimo_bwd_fwd_workspace_size(ctypes.byref(a), ctypes.byref(need)) == _lib.MIMO_OK
    assert need.value > 0
    a.workspace, a.workspace_bytes = 1 << 24, need.value - 1
    assert L.mimo_bwd_fwd(ctypes.byref(a), None) == _lib.MIMO_ERR_VALUE
    assert "workspace too small" in _lib.last_error()
    a.workspace, a.workspace_bytes = None, need.value
    assert L.mimo_bwd_fwd(ctypes.byref(a), None) == _lib.MIMO_ERR_VALUE
    assert "workspace too small" in _lib.last_error()
    a.workspace = (1 << 24) + 128
    assert L.mimo_bwd_fwd(ctypes.byref(a), None) == _lib.MIMO_ERR_VALUE
    assert "256-byte aligned" in _lib.last_error()


def test_binding_checks_caller_outputs_and_workspace():
    """Caller-supplied outputs and workspace are checked before they reach the library
    (CPU tensors stand in for device ones here: the checks are device-agnostic)."""
    from mamba_mimo_chunked_amd import api
    dev = torch.device("cpu")
    dims = (1, 40, 2, 1, 2, 16, 16, 16, 4)   # B, S, H, G, R, N, P, C, rd
    table = api._output_table(*dims, reduce_o=True, has_z=False)
    good = api._outputs(table, None, dev)
    assert good["dz"] is None and good["dmimo_z"] is None
    assert tuple(good["states"].shape) == (1, 2, 3, 16, 16)
    assert api._outputs(table, dict(good), dev)["qk_dot"] is good["qk_dot"]
    bad_cases = [
        (dict(good, states=good["states"].float()), TypeError, "dtype"),
        (dict(good, qk_dot=good["qk_dot"][:, :1]), ValueError, "shape"),
        (dict(good, dz=torch.empty((1, 40, 2, 16), dtype=torch.bfloat16)), ValueError, "must be None"),
        ({k: v for k, v in good.items() if k != "states"}, ValueError, "required"),
        (dict(good, extra=good["states"]), ValueError, "unknown keys"),
    ]
    st = good["states"]
    nc_view = torch.empty((1, 2, 16, 3, 16), dtype=torch.bfloat16).transpose(2, 3)
    bad_cases.append((dict(good, states=nc_view), ValueError, "contiguous"))
    flat = torch.empty(st.numel() + 8, dtype=torch.bfloat16)
    off = flat[1:1 + st.numel()].view(st.shape)       # starts 2 bytes into an allocation
    bad_cases.append((dict(good, states=off), ValueError, "16-byte aligned"))
    for out, exc, msg in bad_cases:
        with pytest.raises(exc, match=msg):
            api._outputs(table, out, dev)
    assert api._workspace(None, 0, dev) is None
    assert api._workspace(None, 100, dev).numel() == 100
    with pytest.raises(TypeError, match="uint8"):
        api._workspace(torch.empty(100, dtype=torch.float32), 100, dev)
    with pytest.raises(ValueError, match="too small"):
        api._workspace(torch.empty(99, dtype=torch.uint8), 100, dev)
    with pytest.raises(ValueError, match="contiguous"):
        api._workspace(torch.empty((100, 2), dtype=torch.uint8).t(), 100, dev)
    # inputs: views that start inside a row are copied to an aligned buffer
    x = torch.arange(72, dtype=torch.float32).to(torch.bfloat16)[1:65]
    assert x.data_ptr() % 16 and api._aligned(x).data_ptr() % 16 == 0
    assert torch.equal(api._aligned(x), x)


def test_noalloc_refuses_calls_beyond_its_scratch_without_a_device():
    """The no-allocation entry point checks the call's workspace against its fixed
    scratch before any device work."""
    L = _lib.lib()
    a = _stage1_args(S=47000)      # the planner leaves about 69 MB of segment state here
    a.B, a.H, a.G, a.R, a.N, a.P = 1, 4, 1, 4, 128, 128
    need = ctypes.c_size_t(0)
    assert L.mimo_bwd_fwd_workspace_size(ctypes.byref(a), ctypes.byref(need)) == _lib.MIMO_OK
    assert need.value > _lib.NOALLOC_SCRATCH_BYTES
    assert L.mimo_bwd_fwd_noalloc(ctypes.byref(a), None) == _lib.MIMO_ERR_UNSUPPORTED
    assert "fixed scratch" in _lib.last_error()
    a.chunk_size = 0
    assert L.mimo_bwd_fwd_noalloc(ctypes.byref(a), None) == _lib.MIMO_ERR_VALUE
