"""Python front end of O1, the contract oracle (``o1_contract.c``).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.

The C oracle is compiled with gcc (OpenMP, ``-ffp-contract=off`` so that no
multiply-add is fused behind the pages' separate fp32 rounding steps) into
``oracle/_build/libo1.so``.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np
import torch

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "o1_contract.c"
_LIB = _HERE / "_build" / "libo1.so"
_lib = None


def build(force: bool = True) -> Path:
    """Compile the C oracle (always, when ``force``)."""
    _LIB.parent.mkdir(exist_ok=True)
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(f".so.tmp{os.getpid()}")
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", str(_SRC), "-o", str(tmp), "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
            build(force=True)
        lib = ctypes.CDLL(str(_LIB))
        i64, dp = ctypes.c_int64, ctypes.POINTER(ctypes.c_double)
        lib.o1_bwd_fwd.restype = ctypes.c_int
        lib.o1_bwd_fwd.argtypes = [i64] * 9 + [ctypes.c_int] * 4 + [dp] * 22
        lib.o1_fwd.restype = ctypes.c_int
        lib.o1_fwd.argtypes = [i64] * 9 + [ctypes.c_int] * 4 + [dp] * 18
        lib.o1_set_skip.restype = ctypes.c_int
        lib.o1_set_skip.argtypes = [ctypes.c_uint64]
        lib.o1_round_bf16.restype = None
        lib.o1_round_bf16.argtypes = [ctypes.POINTER(ctypes.c_float)] * 2 + [i64]
        _lib = lib
    return _lib


def _dbl(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


# The contract's bf16 rounding places of intermediate values, in the order of the
# C enum (o1_contract.c). Each is one place the page's BF16-boundary reference
# rounds to bf16.
ROUNDING_SITES = (
    "Q_BIAS", "K_BIAS", "Q0", "K0", "QK", "QROT", "KROT", "MIMO_V", "PSI",
    "DT_G", "DT_B", "BETA", "FACTOR", "KT", "KAP", "A", "SB",
    "DPROD", "DSUM", "DGAM", "Y", "MIMO_O", "G_IN", "G_OUT", "G_NR", "DZ",
)


@contextlib.contextmanager
def skipping(*sites: str):
    """Test hook: within the block, contract-mode runs leave out the named bf16
    roundings (those values stay fp32). Used to show which outputs each
    rounding reaches; never by a parity reference."""
    mask = 0
    for s in sites:
        mask |= 1 << ROUNDING_SITES.index(s)
    n = _load().o1_set_skip(mask)
    assert n == len(ROUNDING_SITES), "rounding-place list out of step with o1_contract.c"
    try:
        yield
    finally:
        _load().o1_set_skip(0)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """The oracle's own bf16 round-to-nearest-even of float32 values."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    y = np.empty_like(x)
    fp = ctypes.POINTER(ctypes.c_float)
    _load().o1_round_bf16(x.ctypes.data_as(fp), y.ctypes.data_as(fp), x.size)
    return y


def _mode(exact, fp32):
    if exact and fp32:
        raise ValueError("exact and fp32 are exclusive")
    return 1 if exact else (2 if fp32 else 0)


def _width(angles, N, rotary_dim_divisor):
    """Rotated column pairs: the angles' last axis (N / rotary_dim_divisor when given)."""
    W = int(angles.shape[-1])
    if rotary_dim_divisor is not None and W != N // rotary_dim_divisor:
        raise ValueError(f"angles width {W} != N / rotary_dim_divisor")
    return W


def run(dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs, da_cs_rev,
        dt, trap, d, segsum, chunk_size, rotary_dim_divisor=4, *, exact=False, fp32=False):
    """Run O1. Inputs are tensors or arrays in the operator's shapes (any dtype;
    converted to float64 exactly). Returns float64 numpy arrays
    (dmimo_o, states, dz, dmimo_z, qk_dot); inactive outputs are None.
    ``exact``: no rounding at all; ``fp32``: fp32 intermediates (the pages' FP32
    reference), outputs rounded to their dtypes."""
    q = _dbl(q)
    B, S, R, G, N = q.shape
    v = _dbl(v)
    H, P = v.shape[2], v.shape[3]
    C = int(chunk_size)
    nc = (S + C - 1) // C
    reduce_o = mimo_o is not None
    has_z = z is not None
    has_d = d is not None
    arrs = [_dbl(x) for x in (dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles,
                              da_cs, da_cs_rev, dt, trap, d, segsum)]
    dmimo_o = np.zeros((B, H, R, P)) if reduce_o else None
    dmimo_z = np.zeros((B, H, R, P)) if has_z else None
    states = np.zeros((B, H, nc, N, P))
    dz = np.zeros((B, S, H, P)) if has_z else None
    qk_dot = np.zeros((B, H, S, R, R))
    W = _width(arrs[10], N, rotary_dim_divisor)
    rc = _load().o1_bwd_fwd(B, S, H, G, R, N, P, C, W, _mode(exact, fp32),
                            int(reduce_o), int(has_z), int(has_d),
                            *[_ptr(a) for a in arrs],
                            _ptr(dmimo_o), _ptr(states), _ptr(dz), _ptr(dmimo_z), _ptr(qk_dot))
    if rc != 0:
        raise ValueError("o1_bwd_fwd rejected the shape")
    return dmimo_o, states, dz, dmimo_z, qk_dot


def run_fwd(q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs, da_cs_rev,
            dt, trap, d, segsum, chunk_size, rotary_dim_divisor=4, *, exact=False, fp32=False):
    """Layer output of the same chunk walk (no dout): float64 ``o`` of shape
    [B,S,H,P] when ``mimo_o`` is given, else [B,S,R,H,P] (see ``o1_contract.c``)."""
    q = _dbl(q)
    B, S, R, G, N = q.shape
    v = _dbl(v)
    H, P = v.shape[2], v.shape[3]
    reduce_o = mimo_o is not None
    arrs = [_dbl(x) for x in (q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles,
                              da_cs, da_cs_rev, dt, trap, d, segsum)]
    o = np.zeros((B, S, H, P)) if reduce_o else np.zeros((B, S, R, H, P))
    W = _width(arrs[9], N, rotary_dim_divisor)
    rc = _load().o1_fwd(B, S, H, G, R, N, P, int(chunk_size), W, _mode(exact, fp32),
                        int(reduce_o), int(z is not None), int(d is not None),
                        *[_ptr(a) for a in arrs], _ptr(o), None)
    if rc != 0:
        raise ValueError("o1_fwd rejected the shape")
    return o


def run_fwd_inputs(inp: dict, *, exact=False, exact_controls=False, fp32=False):
    """``run_fwd`` on a ``synth.inputs.make_inputs`` dict (dout is not used)."""
    cs, rev, seg = inp["da_cs"], inp["da_cs_rev"], inp["segsum"]
    if exact_controls:
        cs, rev, seg = inp["da_cs64"], inp["da_cs_rev64"], inp["segsum64"]
    return run_fwd(inp["q"], inp["k"], inp["v"], inp["q_bias"], inp["k_bias"], inp["mimo_v"],
                   inp["mimo_o"], inp["z"], inp["mimo_z"], inp["angles"], cs, rev, inp["dt"],
                   inp["trap"], inp["d"], seg, inp["chunk_size"], inp["rotary_dim_divisor"],
                   exact=exact, fp32=fp32)


def run_inputs(inp: dict, *, exact=False, exact_controls=False, fp32=False):
    """Run O1 on a ``synth.inputs.make_inputs`` dict. With ``exact_controls`` the
    float64 controls built from da are used instead of their float32 copies."""
    cs, rev, seg = inp["da_cs"], inp["da_cs_rev"], inp["segsum"]
    if exact_controls:
        cs, rev, seg = inp["da_cs64"], inp["da_cs_rev64"], inp["segsum64"]
    return run(inp["dout"], inp["q"], inp["k"], inp["v"], inp["q_bias"], inp["k_bias"],
               inp["mimo_v"], inp["mimo_o"], inp["z"], inp["mimo_z"], inp["angles"], cs, rev,
               inp["dt"], inp["trap"], inp["d"], seg, inp["chunk_size"],
               inp["rotary_dim_divisor"], exact=exact, fp32=fp32)


def slice_heads(inp: dict, b: int, h: int) -> dict:
    """Inputs of one (batch, head) pair as a B=1, H=1, G=1 problem. Heads are
    independent, so the oracle's result on the slice equals the corresponding
    slice of its result on the whole input."""
    H = inp["v"].shape[2]
    G = inp["q"].shape[3]
    g = h // (H // G)
    out = dict(inp)
    bs, hs, gs = slice(b, b + 1), slice(h, h + 1), slice(g, g + 1)
    out["q"] = inp["q"][bs, :, :, gs]
    out["k"] = inp["k"][bs, :, :, gs]
    out["v"] = inp["v"][bs, :, hs]
    if inp["mimo_o"] is not None:
        out["dout"] = inp["dout"][bs, :, hs]
    else:
        out["dout"] = inp["dout"][bs, :, :, hs]
    out["z"] = None if inp["z"] is None else inp["z"][bs, :, hs]
    for name in ("q_bias", "k_bias", "mimo_v", "mimo_o", "mimo_z"):
        out[name] = None if inp[name] is None else inp[name][hs]
    out["d"] = None if inp["d"] is None else inp["d"][hs]
    out["angles"] = inp["angles"][bs, :, hs]
    for name in ("da_cs", "da_cs_rev", "dt", "trap", "da_cs64", "da_cs_rev64", "da"):
        if name in inp and inp[name] is not None:
            out[name] = inp[name][bs, hs]
    for name in ("segsum", "segsum64"):
        if name in inp and inp[name] is not None:
            out[name] = inp[name][bs, hs]
    return out


def slice_batch(inp: dict, b: int) -> dict:
    """Inputs of batch b as a B=1 problem (batches are independent)."""
    out = dict(inp)
    bs = slice(b, b + 1)
    for name in ("dout", "q", "k", "v", "z", "angles", "da_cs", "da_cs_rev", "dt", "trap",
                 "segsum", "da_cs64", "da_cs_rev64", "segsum64", "da"):
        if name in inp and inp[name] is not None:
            out[name] = inp[name][bs]
    return out
