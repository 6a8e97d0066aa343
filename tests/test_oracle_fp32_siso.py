"""Pins of the oracle's fp32-intermediate mode (the pages' FP32 reference) and
of the SISO forward oracle, against things other than themselves.

fp32 mode: every intermediate is fp32, so it must agree with exact arithmetic
(O1 exact on the same fp32 controls, itself pinned to O2/O3) to fp32 accuracy
on the fp32 outputs, and bit for bit, up to rare rounding-boundary flips, on
the bf16 outputs rounded from the exact values; it must sit far closer to
exact arithmetic than the bf16 contract does.

SISO: the rank-1 chunk walk with controls built from adt equals the unchunked
recurrence O2 fed the per-token log decay directly and the brute-force
quadratic form O3, is invariant to the chunk size, and maps GQA heads like
the expanded-head problem.
"""

import numpy as np
import pytest
import torch

from oracle import o1, o2_sequential as o2, o3_bruteforce as o3, siso
from synth.inputs import Case, SisoCase, make_inputs, make_siso_inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

NAMES = ("dmimo_o", "states", "dz", "dmimo_z", "qk_dot")
BF16_OUT = ("states", "dz", "qk_dot")


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


FP32_CASES = [
    Case(1, 64, 2, 1, 16, 16, 2, 16, name="tiny"),
    Case(2, 45, 4, 2, 16, 16, 3, 8, name="gqa_r3_tail"),
    Case(1, 29, 2, 1, 16, 16, 4, 16, reduce_o=False, has_z=True, has_d=False, name="nr_z"),
    Case(1, 29, 2, 1, 16, 16, 4, 16, reduce_o=True, has_z=False, has_d=True, name="r_noz"),
]


@pytest.mark.parametrize("case", FP32_CASES, ids=lambda c: c.name)
def test_fp32_mode_is_exact_arithmetic_to_fp32_accuracy(case):
    inp = make_inputs(case)
    f = o1.run_inputs(inp, fp32=True)
    e = o1.run_inputs(inp, exact=True)
    for name, a, b in zip(NAMES, f, e):
        if b is None:
            assert a is None, name
            continue
        if name in BF16_OUT:
            rb = o1.round_bf16(b.astype(np.float32)).astype(np.float64)
            assert np.array_equal(a, o1.round_bf16(a.astype(np.float32))), f"{name} not bf16"
            same = np.mean(a == rb)
            assert same > 0.97, (name, same)
            assert rel(a, rb) < 1e-3, name
        else:
            assert rel(a, b) < 1e-5, (name, rel(a, b))


@pytest.mark.parametrize("case", FP32_CASES[:2], ids=lambda c: c.name)
def test_fp32_mode_far_closer_to_exact_than_contract(case):
    inp = make_inputs(case)
    f = o1.run_inputs(inp, fp32=True)
    c = o1.run_inputs(inp)
    e = o1.run_inputs(inp, exact=True)
    for i in (0, 3):            # dmimo_o, dmimo_z (fp32 outputs)
        assert rel(f[i], e[i]) * 50 < rel(c[i], e[i]), NAMES[i]


def test_fp32_mode_forward():
    case = Case(1, 70, 2, 1, 16, 16, 4, 16, name="fwd")
    inp = make_inputs(case)
    f = o1.run_fwd_inputs(inp, fp32=True)
    e = o1.run_fwd_inputs(inp, exact=True)
    rb = o1.round_bf16(e.astype(np.float32)).astype(np.float64)
    assert np.mean(f == rb) > 0.97
    assert rel(f, e) < 4e-3          # bf16 output rounding only


# ---------------------------------------------------------------- SISO oracle
SISO_SMALL = [
    SisoCase(1, 128, 2, 4, 16, 24, 64, name="example_like"),
    SisoCase(2, 70, 1, 2, 16, 8, 32, A=4, name="tail_a4_c32"),
    SisoCase(1, 50, 2, 2, 8, 8, 32, has_z=False, has_d=False, name="no_z_no_d"),
]


def _siso_via_o2(inp):
    q, k = inp["q"], inp["k"]
    B, S, Hq, K = q.shape
    H, V = inp["v"].shape[2:]
    ones = np.ones((H, 1, V))
    z = inp["z"]
    y = o2.run(np.zeros((B, S, 1, H, V)), q[:, :, None], k[:, :, None], inp["v"],
               inp["q_bias"][:, None], inp["k_bias"][:, None], ones, None, z,
               None if z is None else ones, inp["angles"], inp["adt"], inp["dt"], inp["trap"],
               inp["d"], inp["chunk_size"], None)[5]
    return o2.forward(y, None, z, None if z is None else ones)[:, :, 0]


def _siso_via_o3(inp):
    q, k = inp["q"], inp["k"]
    B, S, Hq, K = q.shape
    H, V = inp["v"].shape[2:]
    ones = np.ones((H, 1, V))
    z = inp["z"]
    y = o3.run(np.zeros((B, S, 1, H, V)), q[:, :, None], k[:, :, None], inp["v"],
               inp["q_bias"][:, None], inp["k_bias"][:, None], ones, None, z,
               None if z is None else ones, inp["angles"], inp["adt"], inp["dt"], inp["trap"],
               inp["d"], inp["chunk_size"], None)[5]
    return o2.forward(y, None, z, None if z is None else ones)[:, :, 0]


def _siso(inp, C=None):
    return siso.run(*[inp[n] for n in ("q", "k", "v", "adt", "dt", "trap", "q_bias", "k_bias",
                                       "angles", "d", "z")], chunk_size=C or inp["chunk_size"])


@pytest.mark.parametrize("case", SISO_SMALL, ids=lambda c: c.name)
def test_siso_equals_sequential_and_bruteforce(case):
    inp = make_siso_inputs(case)
    got = _siso(inp)
    assert got.shape == tuple(inp["v"].shape)
    assert rel(got, _siso_via_o2(inp)) < 1e-10
    assert rel(got, _siso_via_o3(inp)) < 1e-10


@pytest.mark.parametrize("C", [1, 7, 32])
def test_siso_chunk_size_invariance(C):
    inp = make_siso_inputs(SisoCase(1, 100, 2, 2, 16, 16, 64, name="inv"))
    assert rel(_siso(inp, C), _siso(inp, 64)) < 1e-12


def test_siso_gqa_equals_expanded_heads():
    case = SisoCase(1, 40, 2, 4, 16, 8, 32, name="gqa")
    inp = make_siso_inputs(case)
    a = _siso(inp)
    exp = dict(inp, q=inp["q"].repeat_interleave(2, dim=2), k=inp["k"].repeat_interleave(2, dim=2))
    b = _siso(exp)
    assert rel(a, b) < 1e-14


def test_siso_controls_from_adt():
    """da_cs restarts at each chunk; rev is what remains to the chunk's last real
    token; segsum is the pairwise difference."""
    adt = torch.tensor([[[1.0, 2.0, 4.0, 8.0, 16.0]]])
    cs, rev, seg = siso.controls(adt, 2)
    assert np.allclose(cs[0, 0], [1, 3, 4, 12, 16])
    assert np.allclose(rev[0, 0], [2, 0, 8, 0, 0])
    assert np.allclose(seg[0, 0, 1], [[0, -8], [8, 0]])
