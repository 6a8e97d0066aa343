"""Pins of the contract oracle's bf16 rounding placement.

Exact-mode pins make every rounding the identity and the bitwise invariants
hold wherever the roundings sit, so two further checks tie O1's contract mode
(``oracle/o1_contract.c``) to the page's BF16-boundary reference:

* O4 (``oracle/o4_matrix.py``), a second implementation written independently
  in chunk-matrix form (numpy arrays, rank-major rows, torch's bf16 conversion,
  float64-accumulated contractions), must agree with O1 output by output:
  bf16 outputs bit-equal on at least 99.9 % of the elements and within one bf16
  ulp everywhere, fp32 outputs within 1e-6 relative. In practice they agree bit
  for bit.
* Rounding witnesses: each of O1's 26 bf16 rounding places, switched off on its
  own, must change exactly the outputs that the reference's dataflow lets it
  reach, and leave every other output bit-identical. The same switch also
  plays the mutation check: with any single place left out, O1 no longer meets
  the O4 bar above.
"""

import numpy as np
import pytest

from oracle import o1, o4_matrix as o4
from synth.inputs import ATK_CASES, CONFIGS, Case, UT_CASES, make_inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

NAMES = ("dmimo_o", "states", "dz", "dmimo_z", "qk_dot")
BF16_OUT = {"states", "dz", "qk_dot", "o"}

CASES = [
    CONFIGS["tiny"],
    Case(1, 37, 2, 1, 16, 8, 2, 8, name="tail_c8"),
    Case(2, 23, 4, 2, 8, 12, 3, 6, name="gqa_r3_c6"),
    Case(1, 20, 2, 2, 8, 8, 1, 1, name="c1_r1"),
    Case(1, 17, 1, 1, 12, 8, 2, 2, rd=2, name="rd2_c2"),
    Case(1, 70, 1, 1, 8, 8, 2, 64, name="c64_tail"),
    Case(1, 29, 2, 1, 16, 16, 4, 16, reduce_o=False, has_z=True, has_d=False, name="nr_z"),
    Case(1, 29, 2, 1, 16, 16, 4, 16, reduce_o=False, has_z=False, has_d=False, name="nr_noz"),
    Case(1, 29, 2, 1, 16, 16, 4, 16, reduce_o=True, has_z=False, has_d=True, name="r_noz"),
    Case(1, 48, 2, 1, 32, 64, 8, 8, name="r8_c8"),
] + UT_CASES + ATK_CASES[:2]


def _ulp_key(x):
    """Monotonic integer key of bf16 values held as floats (one step per bf16 ulp)."""
    u = (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.int64)
    mag = u & 0x7FFF
    return np.where(u & 0x8000, -mag, mag)


def disagreement(name, a, b):
    """None when a and b meet the O1-vs-O4 bar for output ``name``, else a reason."""
    if a is None or b is None:
        return None if (a is None and b is None) else "presence differs"
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if name in BF16_OUT:
        if a.size == 0:
            return None
        eq = np.mean(a == b)
        ulp = int(np.max(np.abs(_ulp_key(a) - _ulp_key(b))))
        if eq < 0.999 or ulp > 1:
            return f"{name}: bit-equal {eq:.5f}, max {ulp} ulp"
        return None
    nb = np.linalg.norm(b)
    r = np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)
    return f"{name}: rel {r:.2e}" if r > 1e-6 else None


@pytest.mark.parametrize("fp32", [False, True], ids=["contract", "fp32"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_o1_equals_o4(case, fp32):
    inp = make_inputs(case)
    r1 = o1.run_inputs(inp, fp32=fp32)
    r4 = o4.run_inputs(inp, fp32=fp32)
    bad = [disagreement(n, a, b) for n, a, b in zip(NAMES, r1, r4)]
    assert not any(bad), bad


@pytest.mark.parametrize("fp32", [False, True], ids=["contract", "fp32"])
@pytest.mark.parametrize("case", [c for c in CASES if c.recipe == "configs"][:7], ids=lambda c: c.name)
def test_o1_equals_o4_layer_output(case, fp32):
    inp = make_inputs(case)
    assert disagreement("o", o1.run_fwd_inputs(inp, fp32=fp32), o4.run_fwd_inputs(inp, fp32=fp32)) is None


# ---------------------------------------------------------------- rounding witnesses
# Which outputs each rounding place can reach, read off the reference's dataflow:
# qk_dot uses only the biased, unrotated q and k; the states use the k path
# (bias, rotation, factor and its dt/trap inputs, kappa) and Psi, never q; y uses
# everything before it; dmimo_o uses y only; the gate gradient G adds bf(mimo_o)
# and its own two roundings (dz, dmimo_z); the dz chain reaches dz alone.
QK_SITES = {"Q_BIAS", "K_BIAS", "Q0", "K0"}
STATE_SITES = {"K_BIAS", "K0", "KROT", "MIMO_V", "PSI", "DT_G", "DT_B", "BETA", "FACTOR", "KT", "KAP"}
Y_SITES = QK_SITES | STATE_SITES | {"QK", "QROT", "A", "SB", "DPROD", "DSUM", "DGAM", "Y"}
G_SITES = {"MIMO_O", "G_IN", "G_OUT"}


def expected_reach(site, reduce_o):
    reach = set()
    if site in QK_SITES:
        reach.add("qk_dot")
    if site in STATE_SITES:
        reach.add("states")
    if site in Y_SITES:
        reach |= {"dz", "dmimo_z"} | ({"dmimo_o"} if reduce_o else set())
    if reduce_o and site in G_SITES:
        reach |= {"dz", "dmimo_z"}
    if not reduce_o and site == "G_NR":
        reach |= {"dz", "dmimo_z"}
    if site == "DZ":
        reach.add("dz")
    return reach


# two full chunks and a tail, every gating branch that has a G
WITNESS_CASES = [
    Case(1, 40, 2, 1, 16, 16, 4, 16, name="reduced_z_d"),
    Case(1, 40, 2, 1, 16, 16, 4, 16, reduce_o=False, has_z=True, has_d=True, name="per_rank_z_d"),
]


@pytest.mark.parametrize("case", WITNESS_CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("site", o1.ROUNDING_SITES)
def test_rounding_reaches_exactly_its_dataflow(case, site):
    inp = make_inputs(case)
    base = o1.run_inputs(inp)
    with o1.skipping(site):
        alt = o1.run_inputs(inp)
    changed = {n for n, a, b in zip(NAMES, base, alt) if a is not None and not np.array_equal(a, b)}
    assert changed == expected_reach(site, case.reduce_o), (site, changed)
    # the entry state of chunk 0 is zero, so neither kappa nor the bf16 state copy
    # used by the inter term can reach the first chunk's y (dz rows of chunk 0)
    if site in ("KAP", "SB"):
        C = case.C
        assert np.array_equal(base[2][:, :C], alt[2][:, :C]), site
        assert not np.array_equal(base[2][:, C:], alt[2][:, C:]), site
    if site == "KAP":
        assert np.array_equal(base[1][:, :, :1], alt[1][:, :, :1])   # states[0] = 0
        assert not np.array_equal(base[1][:, :, 1:2], alt[1][:, :, 1:2])   # chunk 0's kappa


@pytest.mark.parametrize("site", o1.ROUNDING_SITES)
def test_each_rounding_is_caught_by_o4(site):
    """Mutation check: O1 with any one rounding place left out fails the O4 bar."""
    case = WITNESS_CASES[1] if site == "G_NR" else WITNESS_CASES[0]
    inp = make_inputs(case)
    ref = o4.run_inputs(inp)
    with o1.skipping(site):
        mutated = o1.run_inputs(inp)
    bad = [disagreement(n, a, b) for n, a, b in zip(NAMES, mutated, ref)]
    assert any(bad), f"O1 without the {site} rounding still meets the O4 bar"
