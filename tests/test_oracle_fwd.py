"""Pins of the oracle's layer output (``o1.run_fwd``) against things other than itself.

* exact algebra: O1's chunked forward with every rounding off equals the output
  built from the y of the unchunked recurrence O2 and of the brute-force
  quadratic form O3;
* the backward's own definition: dmimo_o, dz and dmimo_z of the pages' gating
  branches are the gradients of sum(o * dout) with respect to mimo_o, z and
  mimo_z, so central differences of the exact forward must reproduce the exact
  backward oracle (this pins the projection and the silu gate of the forward
  against the pages' gradient formulas);
* bit-for-bit invariants of the bf16 contract mode: causality and the rounding
  points of the rank-1 projection;
* calibration: the contract's distance from exact arithmetic.
"""

import numpy as np
import pytest
import torch

from oracle import o1, o2_sequential as o2, o3_bruteforce as o3
from synth.inputs import Case, make_inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


FWD_CASES = [
    Case(1, 64, 2, 1, 16, 16, 2, 16, name="tiny"),
    Case(1, 37, 2, 1, 16, 8, 2, 8, name="tail_c8"),
    Case(2, 23, 4, 2, 8, 12, 3, 6, name="gqa_r3_c6"),
    Case(1, 17, 1, 1, 12, 8, 2, 2, rd=2, name="rd2_c2"),
    Case(1, 29, 2, 1, 16, 16, 4, 16, reduce_o=False, has_z=True, has_d=False, name="nr_z"),
    Case(1, 29, 2, 1, 16, 16, 4, 16, reduce_o=False, has_z=False, has_d=False, name="nr_noz"),
    Case(1, 29, 2, 1, 16, 16, 4, 16, reduce_o=True, has_z=False, has_d=True, name="r_noz"),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: c.name)
def test_exact_fwd_equals_sequential_and_bruteforce(case):
    inp = make_inputs(case, want_exact=True)
    got = o1.run_fwd_inputs(inp, exact=True, exact_controls=True)
    y2 = o2.run_inputs(inp)[5]
    y3 = o3.run_inputs(inp)[5]
    want2 = o2.forward(y2, inp["mimo_o"], inp["z"], inp["mimo_z"])
    want3 = o2.forward(y3, inp["mimo_o"], inp["z"], inp["mimo_z"])
    assert got.shape == want2.shape
    assert rel(got, want2) < 1e-10
    assert rel(got, want3) < 1e-10


def _f(inp, dout):
    """sum(o * dout) of the exact forward."""
    o = o1.run_fwd_inputs(inp, exact=True, exact_controls=True)
    return float((o * dout).sum())


@pytest.mark.parametrize("reduce_o", [True, False], ids=["reduced", "not_reduced"])
def test_fwd_gradients_are_the_backward(reduce_o):
    """Central differences of sum(o * dout) equal the exact backward oracle's
    dmimo_o (summed over batch), dz and dmimo_z."""
    case = Case(2, 21, 2, 1, 8, 8, 3, 8, reduce_o=reduce_o, has_z=True, has_d=True, name="grad")
    inp = make_inputs(case, want_exact=True)
    dmo, _, dz, dmz, _ = o1.run_inputs(inp, exact=True, exact_controls=True)
    dout = inp["dout"].double().numpy()
    rng = np.random.default_rng(5)
    B, S, H, P = inp["v"].shape
    R = inp["q"].shape[2]

    def central(name, idx, h):
        x = inp[name].double().clone()
        x[idx] += h
        fp = _f(dict(inp, **{name: x}), dout)
        x[idx] -= 2 * h
        fm = _f(dict(inp, **{name: x}), dout)
        return (fp - fm) / (2 * h)

    if reduce_o:
        # o is linear in mimo_o: a unit step is exact up to rounding
        for _ in range(4):
            hh, r, p = rng.integers(H), rng.integers(R), rng.integers(P)
            g = central("mimo_o", (hh, r, p), 1.0)
            want = dmo[:, hh, r, p].sum()
            assert abs(g - want) <= 1e-9 * (1 + abs(want)), (hh, r, p, g, want)
    for _ in range(6):
        b, t, hh, p = rng.integers(B), rng.integers(S), rng.integers(H), rng.integers(P)
        g = central("z", (b, t, hh, p), 1e-5)
        want = dz[b, t, hh, p]
        assert abs(g - want) <= 1e-6 * (1 + abs(want)), ("z", b, t, hh, p, g, want)
    for _ in range(4):
        hh, r, p = rng.integers(H), rng.integers(R), rng.integers(P)
        g = central("mimo_z", (hh, r, p), 1e-5)
        want = dmz[:, hh, r, p].sum()
        assert abs(g - want) <= 1e-6 * (1 + abs(want)), ("mimo_z", hh, r, p, g, want)


@pytest.mark.parametrize("t0", [0, 8, 13, 40])
def test_fwd_causality_bitwise(t0):
    """Changing every per-token input from token t0 on leaves o before t0 unchanged,
    bit for bit, in the contract mode."""
    case = Case(1, 48, 2, 1, 16, 16, 2, 16, name="causal")
    inp = make_inputs(case)
    ref = o1.run_fwd_inputs(inp)
    g = torch.Generator().manual_seed(11)
    mod = dict(inp)
    for name in ("q", "k", "v", "z", "angles"):
        x = inp[name].clone()
        x[:, t0:] = torch.randn(x[:, t0:].shape, generator=g).to(x.dtype)
        mod[name] = x
    for name in ("dt", "trap"):
        x = inp[name].clone()
        x[:, :, t0:] = (torch.rand(x[:, :, t0:].shape, generator=g) * 0.5).to(x.dtype)
        mod[name] = x
    out = o1.run_fwd_inputs(mod)
    assert np.array_equal(out[:, :t0], ref[:, :t0])
    if t0 < 48:
        assert not np.array_equal(out[:, t0:], ref[:, t0:])


def test_fwd_rank1_projection_rounding_points():
    """With R = 1 and no z, the reduced output is bf16(y * bf16(mimo_o)) where y is
    the non-reduced output, bit for bit."""
    case = Case(1, 33, 2, 1, 16, 16, 1, 16, reduce_o=True, has_z=False, has_d=True, name="r1")
    inp = make_inputs(case)
    o_red = o1.run_fwd_inputs(inp)
    y = o1.run_fwd_inputs(dict(inp, mimo_o=None))[:, :, 0]            # [B,S,H,P]
    mo = o1.round_bf16(inp["mimo_o"].float().numpy())[:, 0]            # [H,P]
    want = o1.round_bf16((y.astype(np.float32) * mo[None, None]).astype(np.float32))
    assert np.array_equal(o_red, want.astype(np.float64))


@pytest.mark.parametrize("reduce_o,has_z", [(True, True), (False, True), (True, False)])
def test_fwd_contract_distance_from_exact(reduce_o, has_z):
    case = Case(1, 96, 2, 1, 32, 32, 4, 16, reduce_o=reduce_o, has_z=has_z, name="cal")
    inp = make_inputs(case, want_exact=True)
    c = o1.run_fwd_inputs(inp)
    e = o1.run_fwd_inputs(inp, exact=True, exact_controls=True)
    d = rel(c, e)
    assert 1e-5 < d < 2e-2, d
