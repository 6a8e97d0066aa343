"""SISO forward oracle (mamba3_siso_fwd_kernel).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may use it.

Source: the Triton-Ascend mamba3_siso_fwd_kernel migration page ("operator
introduction", "inputs" and "implementation principle" sections): bias and
rotary on q/k, gamma and the look-ahead weight from dt and sigmoid(trap),
the strictly causal QK score times the decay derived from adt inside each
chunk, the previous chunk's state contribution, the same-token QK skip term,
the optional D skip and SiLU(z) gating, then the cross-chunk state update.
That is the rank-1 case of the MIMO chunk walk of O1 with PsiV = v (unit
projection), the gate silu(z) (unit gate projection) and no output
projection, in exact arithmetic (the page measures against a float64 golden).

adt [B,H,S] is the per-token log decay. Inside chunk c (tokens c0..last) with
cs_t = sum_{u=c0..t} adt_u:
  da_cs[t] = cs_t,   da_cs_rev[t] = cs_last - cs_t,   segsum[t][s] = cs_t - cs_s.
q/k heads map to value heads by h -> h / (H/Hq), the MIMO operator's map.
"""

from __future__ import annotations

import numpy as np

from . import o1


def _np(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def controls(adt, chunk_size):
    """float64 (da_cs, da_cs_rev, segsum) of the chunks from the per-token log decay."""
    a = _np(adt)
    B, H, S = a.shape
    C = int(chunk_size)
    nc = (S + C - 1) // C
    pad = np.zeros((B, H, nc * C))
    pad[..., :S] = a                       # zero log decay past the end changes no sum
    cs = np.cumsum(pad.reshape(B, H, nc, C), axis=-1)
    last = np.zeros((B, H, nc, 1))
    for c in range(nc):
        cl = min(C, S - c * C)
        last[:, :, c, 0] = cs[:, :, c, cl - 1]
    da_cs = cs.reshape(B, H, nc * C)[..., :S]
    da_cs_rev = (last - cs).reshape(B, H, nc * C)[..., :S]
    segsum = cs[..., :, None] - cs[..., None, :]
    return da_cs, da_cs_rev, segsum


def run(q, k, v, adt, dt, trap, q_bias, k_bias, angles, d=None, z=None, chunk_size=64):
    """float64 output [B,S,H,V] of the SISO forward in exact arithmetic.
    q, k [B,S,Hq,K]; v, z [B,S,H,V]; adt, dt, trap [B,H,S]; q_bias, k_bias [H,K];
    angles [B,S,H,A] (A <= K/2 rotated pairs); d [H]."""
    q, k, v = _np(q), _np(k), _np(v)
    H, V = v.shape[2], v.shape[3]
    cs, rev, seg = controls(adt, chunk_size)
    ones = np.ones((H, 1, V))
    o = o1.run_fwd(q[:, :, None], k[:, :, None], v, _np(q_bias)[:, None], _np(k_bias)[:, None], ones,
                   None, z, None if z is None else ones, angles, cs, rev, dt, trap, d, seg,
                   chunk_size, None, exact=True)
    return o[:, :, 0]
