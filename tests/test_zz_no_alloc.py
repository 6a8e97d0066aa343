"""The entry point that allocates nothing (mimo_bwd_fwd_noalloc), through the C ABI.

Its scratch is a fixed device array inside the library. On two calls in a row,
the second one smaller, its outputs must equal those of mimo_bwd_fwd with a
caller workspace bit for bit (the same kernels run on the same inputs), and
meet the oracle bar. A call whose workspace would not fit the array is refused.
"""

import ctypes

import numpy as np
import pytest
import torch

from mamba_mimo_chunked_amd import _lib
from mamba_mimo_chunked_amd.api import _make_args
from synth.inputs import API_ORDER, Case, make_inputs

from ._parity import NAMES, compare, log, oracle

pytestmark = pytest.mark.gpu


def _outputs(case, dev):
    B, S, H, R, N, P = case.B, case.S, case.H, case.R, case.N, case.P
    nc = case.nchunks
    return {
        "dmimo_o": torch.full((B, H, R, P), float("nan"), device=dev) if case.reduce_o else None,
        "states": torch.full((B, H, nc, N, P), float("nan"), device=dev, dtype=torch.bfloat16),
        "dz": torch.full((B, S, H, P), float("nan"), device=dev, dtype=torch.bfloat16) if case.has_z else None,
        "dmimo_z": torch.full((B, H, R, P), float("nan"), device=dev) if case.has_z else None,
        "qk_dot": torch.full((B, H, S, R, R), float("nan"), device=dev, dtype=torch.bfloat16),
    }


def _call(case, d, noalloc):
    L = _lib.lib()
    dev = d["q"].device
    out = _outputs(case, dev)
    args = _make_args(case.B, case.S, case.H, case.G, case.R, case.N, case.P, case.C, case.rd, d, out)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if noalloc:
        st = L.mimo_bwd_fwd_noalloc(ctypes.byref(args), stream)
    else:
        need = ctypes.c_size_t(0)
        assert L.mimo_bwd_fwd_workspace_size(ctypes.byref(args), ctypes.byref(need)) == _lib.MIMO_OK
        ws = torch.empty(max(int(need.value), 256), dtype=torch.uint8, device=dev)
        args.workspace, args.workspace_bytes = ws.data_ptr(), int(need.value)
        st = L.mimo_bwd_fwd(ctypes.byref(args), stream)
    assert st == _lib.MIMO_OK, _lib.last_error()
    torch.cuda.synchronize()
    return tuple(out[n] for n in NAMES)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    _lib.lib()


def test_noalloc_matches_workspace_entry_point_twice():
    # first a call that fills most of the scratch, then a smaller one
    for case in (Case(1, 8192, 16, 1, 64, 64, 4, 16, name="noalloc_perf_shape"),
                 Case(1, 300, 3, 1, 64, 64, 4, 16, name="noalloc_small")):
        log(f"[noalloc] {case.name}")
        inp = make_inputs(case)
        d = {n: (None if inp[n] is None else inp[n].cuda()) for n in API_ORDER}
        ref = _call(case, d, noalloc=False)
        got = _call(case, d, noalloc=True)
        for n, a, b in zip(NAMES, ref, got):
            if a is None:
                assert b is None
                continue
            assert torch.isfinite(b.float()).all(), n
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), n
        if case.S <= 300:
            compare(got, oracle(inp), label=f"{case.name}: ")
