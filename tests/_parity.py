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


def _ulp_key(x):
    """Monotonic integer key of bf16 values held as floats (one step per bf16 ulp)."""
    u = (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.int64)
    mag = u & 0x7FFF
    return np.where(u & 0x8000, -mag, mag)


def check_elements(name, gv, r, *, bf16: bool, label="", ulp_frac=0.999):
    """Element-wise bars next to the whole-tensor one, so that a few wrong
    elements in a large tensor cannot hide under the RMS:
    * bf16 outputs: at least 99.9 % of the elements within one bf16 ulp of the
      oracle, or, in tensors too small for 0.1 % to hold a cascade, at most 32
      elements off by more or all of them inside at most 4 rows (a row: the
      values along the last axis, e.g. one token's dz of one head). The hardware
      sine and cosine differ from the oracle's correctly rounded ones by up to
      ~3e-7, so now and then one rotated q or k value rounds to the other bf16
      neighbour; that reaches the dz row of its token, the rows of the later
      tokens of its chunk whose causal-block entry it changes, and the states
      after the chunk, through the bf16 chains. A wrong index or term is off in
      most rows instead. And every element within 2^-5 |ref| + 2^-3 RMS(ref): a
      rank-ordered bf16 chain (dz over up to 8 ranks) can cancel from partial
      sums many times its result, where one tie broken the other way is one ulp
      of the partial sum; a wrong element is off by the order of RMS(ref);
    * fp32 outputs (sums over tokens of products with bf16 y, where one y may sit
      one ulp apart because a rounding tie broke the other way; with few tokens one
      such term moves an element by up to ~1 %): every element within
      2^-6 (|ref| + RMS(ref)); a wrong element is off by the order of itself.
    ``ulp_frac`` replaces the 99.9 % (random shapes with drawn angles, whose long
    chains let one such flip reach more than 0.1 % of a small tensor).
    Returns the fraction of bf16 elements within one ulp (1.0 for fp32)."""
    a = np.asarray(gv, np.float64)
    r = np.asarray(r, np.float64)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    dev = np.abs(a - r)
    if bf16:
        far_mask = np.abs(_ulp_key(a) - _ulp_key(r)) > 1
        far = int(far_mask.sum()) if r.size else 0
        rows = int(np.any(far_mask.reshape(-1, r.shape[-1]), axis=1).sum()) if r.size else 0
        within = 1.0 - far / r.size if r.size else 1.0
        assert within >= ulp_frac or far <= 32 or rows <= 4, \
            f"{label}{name}: only {within:.5f} of the elements within 1 bf16 ulp ({far} beyond, in {rows} rows)"
        bound = 2.0 ** -5 * np.abs(r) + 2.0 ** -3 * rms
    else:
        within = 1.0
        bound = 2.0 ** -6 * (np.abs(r) + rms)
    bad = dev > bound
    if bad.any():
        i = np.unravel_index(int(np.argmax(dev - bound)), r.shape)
        raise AssertionError(f"{label}{name}: {int(bad.sum())} element(s) off, worst at {i}: "
                             f"{a[i]!r} vs {r[i]!r}")
    return within


def per_head(name, x):
    """View of an output with (batch, head) as its two leading axes."""
    x = np.asarray(x)
    return np.swapaxes(x, 1, 2) if name == "dz" else x   # dz is [B,S,H,P]


def compare(gpu_out, ref_out, *, tol=TOL, label="", ulp_frac=0.999):
    """Assert per-output parity: the stated bar (relative RMS < tol over the whole
    tensor), a per-(batch, head) bar, and the element-wise bars of check_elements.
    Returns {name: rel_rms}."""
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
        # every (batch, head) slice: a wrong head shows a relative RMS of order one; the
        # bar sits at 4 x tol because a head's dmimo slice holds R*P sums of as few as S
        # terms, where one bf16 tie of y broken the other way moves it by ~1e-3 at S ~ 20
        gh, rh = per_head(name, gv), per_head(name, r)
        for b in range(rh.shape[0]):
            for h in range(rh.shape[1]):
                eh = rel_rms(gh[b, h], rh[b, h])
                assert eh < 4 * tol, f"{label}{name}: rel RMS {eh:.3e} >= {4 * tol} at batch {b}, head {h}"
        check_elements(name, gv, r, bf16=(dt == torch.bfloat16), label=label, ulp_frac=ulp_frac)
    return errs


def oracle(inp: dict):
    return o1.run_inputs(inp)
