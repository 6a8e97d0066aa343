"""Pins of the stage-2 backward oracle (``oracle.bwd2``) against an independent
formulation: float64 autograd of the unchunked token-by-token recurrence
(``oracle.o2_torch``), fed the same inputs, with the first stage's caches
(states, qk_dot) computed exactly. The chunked oracle's outputs are partial
derivatives with respect to the chunk controls (da_cs, da_cs_rev, segsum, the
factor and gamma), so they are mapped to the per-token log decay da, to dt and
to trap by the chain rule of the controls' definitions; q, k (summed over the
heads of a group), v, mimo_v and d (summed over the batch) and the angles
compare directly. Also: the heads of a group sum to the group's gradient, the
caches' values are what enters (not recomputed), and zero outputs where a
quantity is unused.
"""

import numpy as np
import pytest
import torch

from oracle import bwd2, o1, o2_torch
from synth.inputs import Case, make_inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


CASES = [
    Case(1, 40, 2, 1, 8, 8, 2, 8, name="small"),
    Case(2, 37, 4, 2, 8, 6, 3, 6, name="gqa_tail_r3"),
    Case(1, 33, 2, 1, 8, 8, 2, 16, reduce_o=False, has_z=False, has_d=False, name="nonreduced_nod"),
    Case(1, 20, 1, 1, 8, 8, 1, 1, name="c1_r1"),
    Case(1, 25, 2, 1, 8, 8, 2, 4, rd=2, name="rd2"),
]


def _exact_caches(inp):
    _, states, _, _, qk = o1.run_inputs(inp, exact=True, exact_controls=True)
    return states, qk


def _chunked(inp, states, qk):
    return bwd2.run(inp["dout"], inp["q"], inp["k"], inp["v"], inp["q_bias"], inp["k_bias"], inp["mimo_v"],
                    states, qk, inp["da_cs64"], inp["da_cs_rev64"], inp["dt"], inp["trap"], inp["segsum64"],
                    inp["angles"], inp["mimo_o"], inp["d"], inp["chunk_size"])


def _to_da(g, S, C):
    """d L / d da_u from the partials with respect to the chunk controls."""
    B, H = g["DDA_CS"].shape[:2]
    out = np.zeros((B, H, S))
    for c0 in range(0, S, C):
        cl = min(C, S - c0)
        cs, rev = g["DDA_CS"][..., c0:c0 + cl], g["DDA_CS_REV"][..., c0:c0 + cl]
        seg = g["DSSDA"][:, :, c0 // C, :cl, :cl]
        state = g["DDA"][..., c0 + cl - 1]
        for u in range(cl):
            v = cs[..., u:].sum(-1) + rev[..., :u].sum(-1) + seg[..., u:, :u].sum((-1, -2)) + state
            out[..., c0 + u] = v
    return out


def _to_dt_trap(g, dt, trap):
    dt, trap = torch.as_tensor(dt).double().numpy(), torch.as_tensor(trap).double().numpy()
    sg = 1.0 / (1.0 + np.exp(-trap))
    dsg = sg * (1.0 - sg)
    dgam = g["DGAMMA"] + g["DFACTOR"]          # gamma enters the diagonal and the factor
    dbeta = g["DFACTOR"]
    ddt = dgam * sg
    dtr = dgam * dt * dsg
    ddt[..., 1:] += dbeta[..., :-1] * (1.0 - sg[..., 1:])
    dtr[..., 1:] -= dbeta[..., :-1] * dt[..., 1:] * dsg[..., 1:]
    return ddt, dtr


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_bwd2_equals_sequential_autograd(case):
    inp = make_inputs(case, want_exact=True)
    states, qk = _exact_caches(inp)
    g = _chunked(inp, states, qk)
    ref = o2_torch.grads(inp["dout"], inp["q"], inp["k"], inp["v"], inp["q_bias"], inp["k_bias"],
                         inp["mimo_v"], inp["angles"], inp["da"], inp["dt"], inp["trap"], inp["mimo_o"], inp["d"])
    B, S, R, G, N = inp["q"].shape
    H = inp["v"].shape[2]
    hpg = H // G
    dq = g["DQ"].reshape(B, S, R, G, hpg, N).sum(4)
    dk = g["DK"].reshape(B, S, R, G, hpg, N).sum(4)
    assert rel(dq, ref["q"]) < 1e-10
    assert rel(dk, ref["k"]) < 1e-10
    assert rel(g["DV"], ref["v"]) < 1e-10
    assert rel(g["DMIMO_V"].sum(0), ref["mimo_v"]) < 1e-10
    assert rel(g["DANGLES"], ref["angles"]) < 1e-10
    if case.has_d:
        assert rel(g["DD"].sum(0), ref["d"]) < 1e-10
    else:
        assert g["DD"] is None
    assert rel(_to_da(g, S, case.C), ref["da"]) < 1e-9
    ddt, dtr = _to_dt_trap(g, inp["dt"], inp["trap"])
    assert rel(ddt, ref["dt"]) < 1e-9
    assert rel(dtr, ref["trap"]) < 1e-9


def test_bwd2_shapes_and_unused_entries():
    case = Case(1, 21, 2, 1, 8, 8, 2, 8, name="shapes")
    inp = make_inputs(case, want_exact=True)
    states, qk = _exact_caches(inp)
    g = _chunked(inp, states, qk)
    B, S, H, N, P, R, C = 1, 21, 2, 8, 8, 2, 8
    assert g["DQ"].shape == (B, S * R, H, N) and g["DK"].shape == (B, S * R, H, N)
    assert g["DV"].shape == (B, S, H, P) and g["DMIMO_V"].shape == (B, H, R, P)
    assert g["DANGLES"].shape == (B, S, H, N // 4) and g["DD"].shape == (B, H)
    assert g["DSSDA"].shape == (B, H, 3, C, C)
    for name in ("DFACTOR", "DGAMMA", "DDA", "DDA_CS_REV", "DDA_CS"):
        assert g[name].shape == (B, H, S)
    # the state decay is used at each chunk's last real token only; chunk 0's decay
    # multiplies the zero initial state and the last chunk's outgoing state is never
    # read, so only chunk 1's entry is nonzero
    last = [7, 15]
    mask = np.zeros(S, bool)
    mask[last] = True
    assert np.all(g["DDA"][..., ~mask] == 0) and np.all(g["DDA"][..., 20] == 0)
    assert np.all(g["DDA"][..., 7] == 0) and np.all(g["DDA"][..., 15] != 0)
    # segsum entries on or above the diagonal, and past the tail, get no gradient
    for c in range(3):
        assert np.all(np.triu(g["DSSDA"][0, 0, c]) == 0)
    assert np.all(g["DSSDA"][:, :, 2, 5:, :] == 0) and np.all(g["DSSDA"][:, :, 2, :, 5:] == 0)


def test_bwd2_uses_the_cached_values():
    """The caches' values enter the result: replacing states by other values changes
    DQ (through the inter term) but leaves DV and DK, which do not read S, unchanged."""
    case = Case(1, 32, 2, 1, 8, 8, 2, 8, name="cache")
    inp = make_inputs(case, want_exact=True)
    states, qk = _exact_caches(inp)
    a = _chunked(inp, states, qk)
    b = _chunked(inp, states * 1.5, qk)
    assert rel(a["DQ"], b["DQ"]) > 1e-3
    assert rel(a["DV"], b["DV"]) < 1e-13 and rel(a["DK"], b["DK"]) < 1e-13
    c = _chunked(inp, states, qk * 2.0)
    assert rel(a["DGAMMA"], c["DGAMMA"]) > 1e-3
