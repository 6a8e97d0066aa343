"""Shared helpers of the GPU parity tests: run the HIP path through its Python
binding (which calls the C ABI) and the CPU oracle O1 on the same seeded
inputs, and compare output by output."""

from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import o1
from synth.inputs import API_ORDER

NAMES = ("dmimo_o", "states", "dz", "dmimo_z", "qk_dot")
# The parity bar: RMS(actual - ref) / RMS(ref) < 1e-3 on every output.
TOL = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp: dict, device="cuda"):
    out = dict(inp)
    for n in API_ORDER:
        if inp[n] is not None:
            out[n] = inp[n].to(device)
    return out


def run_gpu(dinp: dict, **kw):
    from mamba_mimo_chunked_amd import mamba_mimo_bwd_fwd
    args = [dinp[n] for n in API_ORDER]
    res = mamba_mimo_bwd_fwd(*args, dinp["chunk_size"], dinp["rotary_dim_divisor"], **kw)
    torch.cuda.synchronize()
    return res


def rel_rms(actual, ref) -> float:
    a = np.asarray(actual, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    nr = np.sqrt(np.mean(r * r))
    return float(np.sqrt(np.mean((a - r) ** 2)) / (nr if nr > 0 else 1.0))


def compare(gpu_out, ref_out, *, tol=TOL, label=""):
    """Assert per-output parity; returns {name: rel_rms}."""
    errs = {}
    dtypes = (torch.float32, torch.bfloat16, torch.bfloat16, torch.float32, torch.bfloat16)
    for name, g, r, dt in zip(NAMES, gpu_out, ref_out, dtypes):
        if r is None:
            assert g is None, f"{label}{name}: expected None"
            continue
        assert g is not None, f"{label}{name}: missing"
        assert g.dtype == dt, f"{label}{name}: dtype {g.dtype}"
        gv = g.detach().float().cpu().numpy()
        assert gv.shape == r.shape, f"{label}{name}: shape {gv.shape} vs {r.shape}"
        assert np.isfinite(gv).all(), f"{label}{name}: non-finite values"
        e = rel_rms(gv, r)
        errs[name] = e
        assert e < tol, f"{label}{name}: rel RMS {e:.3e} >= {tol}"
    return errs


def oracle(inp: dict):
    return o1.run_inputs(inp)
