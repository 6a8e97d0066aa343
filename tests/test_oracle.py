"""Pins of the CPU oracle against things other than itself.

* exact algebra: O1 with every rounding off equals the unchunked recurrence
  O2 and the quadratic brute force O3 (three independent implementations);
* special cases that reduce to library routines (numpy matmul prefix sums,
  strictly causal linear attention, torch's bf16 conversion);
* invariants of the method that hold bit for bit in the bf16 contract mode
  (causality, power-of-two scaling, tail padding, reduced vs non-reduced
  dout, GQA vs expanded heads, head slicing, chunk-size invariance in exact
  mode);
* calibration: the contract's distance from exact arithmetic.
"""

import math

import numpy as np
import pytest
import torch

from oracle import o1, o2_sequential as o2, o3_bruteforce as o3
from synth.inputs import CONFIGS, Case, make_inputs, UT_CASES

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

NAMES = ("dmimo_o", "states", "dz", "dmimo_z", "qk_dot")


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def same(a, b):
    """Bitwise equality of two optional float arrays (NaN == NaN)."""
    if a is None or b is None:
        return a is None and b is None
    return np.array_equal(np.asarray(a), np.asarray(b), equal_nan=True)


SMALL = [
    Case(1, 64, 2, 1, 16, 16, 2, 16, name="tiny"),
    Case(1, 37, 2, 1, 16, 8, 2, 8, name="tail_c8"),
    Case(2, 23, 4, 2, 8, 12, 3, 6, name="gqa_r3_c6"),
    Case(1, 20, 2, 2, 8, 8, 1, 1, name="c1_r1"),
    Case(1, 17, 1, 1, 12, 8, 2, 2, rd=2, name="rd2_c2"),
    Case(1, 70, 1, 1, 8, 8, 2, 64, name="c64_tail"),
    Case(1, 29, 2, 1, 16, 16, 4, 16, reduce_o=False, has_z=True, has_d=False, name="nr_z"),
    Case(1, 29, 2, 1, 16, 16, 4, 16, reduce_o=False, has_z=False, has_d=False, name="nr_noz"),
    Case(1, 29, 2, 1, 16, 16, 4, 16, reduce_o=True, has_z=False, has_d=True, name="r_noz"),
]


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    special = np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, 1e-40, -1e-40, 1.17e-38,
                        float("inf"), float("-inf"), 1.00390625, 1.01171875, 1.0078125 + 2**-9],
                       dtype=np.float32)
    # exact ties: upper half odd / even with lower half 0x8000
    ties = (np.array([0x3f808000, 0x3f818000, 0xbf808000, 0x00018000, 0x7f7f8000], dtype=np.uint32)
            .view(np.float32))
    x = np.concatenate([x, special, ties])
    ours = o1.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours, ref, equal_nan=True)


# ---------------------------------------------------------------- exact algebra
@pytest.mark.parametrize("case", SMALL, ids=lambda c: c.name)
def test_exact_o1_equals_sequential_and_bruteforce(case):
    inp = make_inputs(case, want_exact=True)
    r1 = o1.run_inputs(inp, exact=True, exact_controls=True)
    r2 = o2.run_inputs(inp)
    r3 = o3.run_inputs(inp)
    for i, n in enumerate(NAMES):
        if r2[i] is None:
            assert r1[i] is None and r3[i] is None, n
            continue
        assert rel(r1[i], r2[i]) < 1e-10, n
        assert rel(r3[i], r2[i]) < 1e-10, n


@pytest.mark.parametrize("case", SMALL[:4], ids=lambda c: c.name)
def test_exact_o1_with_fp32_controls(case):
    """The float32 copies of the controls move the exact result by ~1e-7 only."""
    inp = make_inputs(case, want_exact=True)
    r1 = o1.run_inputs(inp, exact=True, exact_controls=False)
    r2 = o2.run_inputs(inp)
    for i, n in enumerate(NAMES):
        if r2[i] is not None:
            assert rel(r1[i], r2[i]) < 1e-4, n


def test_states_are_entry_states():
    """states[c] is the state before chunk c: the first one is exactly zero, and
    with C = 1 state c is the recurrence's state after token c-1."""
    case = Case(1, 9, 2, 1, 8, 8, 2, 1)
    inp = make_inputs(case, want_exact=True)
    r1 = o1.run_inputs(inp)
    assert not np.any(r1[1][:, :, 0])
    r1e = o1.run_inputs(inp, exact=True, exact_controls=True)
    r2 = o2.run_inputs(inp)
    assert rel(r1e[1], r2[1]) < 1e-12


@pytest.mark.parametrize("C", [1, 2, 4, 8, 16, 32])
def test_chunk_size_invariance_exact(C):
    """Exact mode: every chunk size gives the same y-derived outputs and qk_dot,
    and states agree at shared chunk boundaries."""
    base = Case(1, 32, 2, 1, 8, 8, 2, 32)
    ref_inp = make_inputs(base, want_exact=True)
    ref = o1.run_inputs(ref_inp, exact=True, exact_controls=True)
    inp = make_inputs(base.with_(C=C), want_exact=True)
    out = o1.run_inputs(inp, exact=True, exact_controls=True)
    for i in (0, 2, 3, 4):
        assert rel(out[i], ref[i]) < 1e-12, NAMES[i]
    # states at C and at C' = 8 (boundaries every lcm)
    other = o1.run_inputs(make_inputs(base.with_(C=8), want_exact=True), exact=True,
                          exact_controls=True)
    L = math.lcm(C, 8)
    for t0 in range(0, 32, L):
        assert rel(out[1][:, :, t0 // C], other[1][:, :, t0 // 8]) < 1e-12


# ---------------------------------------------------------------- special cases
def _prep_numpy(inp):
    """Biased / rotated / scaled q, k and PsiV for B=1,H=1,G=1 inputs with
    angles = 0 (no rotation): plain definitions, float64."""
    q = inp["q"].double().numpy()[0, :, :, 0]              # [S,R,N]
    k = inp["k"].double().numpy()[0, :, :, 0]
    qb, kb = inp["q_bias"].double().numpy()[0], inp["k_bias"].double().numpy()[0]
    q0, k0 = q + qb, k + kb
    dt = inp["dt"].double().numpy()[0, 0]
    tr = inp["trap"].double().numpy()[0, 0]
    sig = lambda x: 1 / (1 + np.exp(-x))
    gam = dt * sig(tr)
    beta = np.append(dt[1:] * sig(-tr[1:]), 0.0)
    kt = k0 * (gam + beta)[:, None, None]
    psi = inp["v"].double().numpy()[0, :, 0][:, None, :] * inp["mimo_v"].double().numpy()[0]
    return q0, k0, kt, psi, gam


def test_no_decay_states_are_prefix_gemms():
    """da = 0: states[c] = K~[:cC]^T Psi[:cC], a plain matrix product."""
    case = Case(1, 40, 1, 1, 8, 6, 2, 8)
    inp = make_inputs(case, want_exact=True)
    inp["angles"] = torch.zeros_like(inp["angles"])
    for n in ("da_cs64", "da_cs_rev64", "segsum64"):
        inp[n] = torch.where(torch.isinf(inp[n]), inp[n], torch.zeros_like(inp[n]))
    _, _, kt, psi, _ = _prep_numpy(inp)
    st = o1.run_inputs(inp, exact=True, exact_controls=True)[1][0, 0]
    S, R, N = kt.shape
    for c in range(case.nchunks):
        e = c * case.C
        ref = kt[:e].reshape(e * R, N).T @ psi[:e].reshape(e * R, psi.shape[-1])
        assert np.allclose(st[c], ref, rtol=1e-12, atol=1e-12)


def test_no_decay_rank1_is_causal_linear_attention():
    """da = 0, R = 1: y = strict_tril(Q K~^T) Psi + gamma * diag(Q0 K0^T) Psi + d Psi,
    unnormalised causal linear attention. y rows are read through dmimo_o with a
    one-hot dout (no z)."""
    case = Case(1, 24, 1, 1, 8, 6, 1, 8, has_z=False, has_d=True)
    inp = make_inputs(case, want_exact=True)
    inp["angles"] = torch.zeros_like(inp["angles"])
    for n in ("da_cs64", "da_cs_rev64", "segsum64"):
        inp[n] = torch.where(torch.isinf(inp[n]), inp[n], torch.zeros_like(inp[n]))
    q0, k0, kt, psi, gam = _prep_numpy(inp)
    Q, K, Kt, Ps = q0[:, 0], k0[:, 0], kt[:, 0], psi[:, 0]
    d = inp["d"].double().numpy()[0]
    y = np.tril(Q @ Kt.T, -1) @ Ps + (gam * np.diag(Q @ K.T))[:, None] * Ps + d * Ps
    for t in (0, 5, 13, 23):
        onehot = torch.zeros_like(inp["dout"], dtype=torch.float64)
        onehot[0, t, 0, :] = 1.0
        inp2 = dict(inp, dout=onehot)
        dmo = o1.run_inputs(inp2, exact=True, exact_controls=True)[0][0, 0, 0]
        assert np.allclose(dmo, y[t], rtol=1e-12, atol=1e-12)


def test_zero_angles_rotary_divisor_irrelevant():
    """angles = 0 leaves q and k unrotated, in contract mode too: rd = 2 and rd = 4
    give bit-identical outputs."""
    case = Case(1, 33, 2, 1, 16, 8, 2, 8, rd=4)
    inp4 = make_inputs(case)
    inp4["angles"] = torch.zeros_like(inp4["angles"])
    inp2 = dict(inp4, rotary_dim_divisor=2, angles=torch.zeros(1, 33, 2, 8))
    a, b = o1.run_inputs(inp4), o1.run_inputs(inp2)
    for i in range(5):
        assert same(a[i], b[i]), NAMES[i]


# ---------------------------------------------------------------- contract-mode invariants
@pytest.fixture(scope="module")
def base_case():
    case = Case(1, 45, 2, 1, 16, 16, 2, 8)
    inp = make_inputs(case)
    return case, inp, o1.run_inputs(inp)


def test_qk_dot_independent_of_other_inputs(base_case):
    case, inp, ref = base_case
    g = torch.Generator().manual_seed(7)
    inp2 = dict(inp)
    for n in ("v", "dout", "z", "angles", "da_cs", "da_cs_rev", "dt", "segsum"):
        inp2[n] = (torch.randn(inp[n].shape, generator=g)).to(inp[n].dtype)
    out = o1.run_inputs(inp2)
    assert same(out[4], ref[4])


def test_power_of_two_scaling_bitwise(base_case):
    case, inp, ref = base_case
    out = o1.run_inputs(dict(inp, v=inp["v"] * 2))
    for i in (0, 1, 2, 3):
        assert same(out[i], 2 * ref[i]), NAMES[i]
    assert same(out[4], ref[4])
    out = o1.run_inputs(dict(inp, dout=inp["dout"] * 2))
    for i in (0, 2, 3):
        assert same(out[i], 2 * ref[i]), NAMES[i]
    assert same(out[1], ref[1]) and same(out[4], ref[4])


@pytest.mark.parametrize("t0", [0, 8, 13, 40])
def test_causality_bitwise(base_case, t0):
    """Changing inputs at tokens >= t0 changes no output before t0; states[c] with
    c*C <= t0 keep their value (dt/trap at t0 itself feed the state before it)."""
    case, inp, ref = base_case
    g = torch.Generator().manual_seed(t0 + 1)
    inp2 = dict(inp)
    for n in ("q", "k", "v", "dout", "z", "angles"):
        x = inp[n].clone()
        x[:, t0:] = torch.randn(x[:, t0:].shape, generator=g).to(x.dtype)
        inp2[n] = x
    for n in ("da_cs", "da_cs_rev"):
        x = inp[n].clone()
        x[..., t0:] = torch.randn(x[..., t0:].shape, generator=g).to(x.dtype)
        inp2[n] = x
    for n in ("dt", "trap"):
        x = inp[n].clone()
        x[..., t0 + 1:] = torch.rand(x[..., t0 + 1:].shape, generator=g).to(x.dtype)
        inp2[n] = x
    seg = inp["segsum"].clone().view(1, 2, -1, case.C)          # rows of the chunk tiles
    rows = torch.arange(case.nchunks * case.C)
    seg[:, :, rows >= t0] = torch.randn(seg[:, :, rows >= t0].shape, generator=g)
    inp2["segsum"] = seg.view_as(inp["segsum"])
    out = o1.run_inputs(inp2)
    assert same(out[4][:, :, :t0], ref[4][:, :, :t0])
    assert same(out[2][:, :t0], ref[2][:, :t0])
    ncs = t0 // case.C + 1                                      # chunks starting at <= t0
    assert same(out[1][:, :, :ncs], ref[1][:, :, :ncs])


def test_dt_trap_lookahead_reaches_state_only(base_case):
    """beta_t uses dt/trap of token t+1: changing them at t0 = cC changes the state
    entering chunk c but no y (hence no dz) before t0."""
    case, inp, ref = base_case
    t0 = 2 * case.C
    inp2 = dict(inp)
    dt = inp["dt"].clone()
    dt[..., t0] *= 3.0
    inp2["dt"] = dt
    out = o1.run_inputs(inp2)
    assert same(out[2][:, :t0], ref[2][:, :t0])
    assert same(out[1][:, :, :2], ref[1][:, :, :2])
    assert not same(out[1][:, :, 2], ref[1][:, :, 2])


@pytest.mark.parametrize("S", [17, 20, 23, 24])
def test_tail_equals_zero_padded_crop(S):
    """A partial last chunk gives the crop of the run on inputs zero-padded to a
    whole number of chunks (the pages' own tail handling)."""
    case = Case(1, S, 2, 1, 16, 8, 2, 8)
    inp = make_inputs(case)
    Sp = case.nchunks * case.C
    pad = dict(inp)
    for n in ("q", "k", "v", "dout", "z", "angles"):
        x = inp[n]
        pad[n] = torch.cat([x, torch.zeros((x.shape[0], Sp - S) + tuple(x.shape[2:]), dtype=x.dtype)], 1)
    for n in ("da_cs", "da_cs_rev", "dt", "trap"):
        x = inp[n]
        pad[n] = torch.cat([x, torch.zeros(x.shape[:2] + (Sp - S,), dtype=x.dtype)], 2)
    a, b = o1.run_inputs(inp), o1.run_inputs(pad)
    assert same(a[0], b[0]) and same(a[3], b[3])
    assert same(a[1], b[1])
    assert same(a[2], b[2][:, :S]) and same(a[4], b[4][:, :, :S])


def test_reduced_equals_nonreduced_with_projected_dout():
    case = Case(1, 30, 2, 1, 16, 16, 3, 8)
    inp = make_inputs(case)
    ref = o1.run_inputs(inp)
    mo = inp["mimo_o"].to(torch.bfloat16).float()                    # [H,R,P]
    dnr = (inp["dout"].float()[:, :, None] * mo.permute(1, 0, 2)[None, None]).to(torch.bfloat16)
    nr = dict(inp, dout=dnr, mimo_o=None)
    out = o1.run_inputs(nr)
    assert out[0] is None
    assert same(out[2], ref[2]) and same(out[3], ref[3])
    assert same(out[1], ref[1]) and same(out[4], ref[4])


def test_gqa_equals_expanded_heads_and_head_permutation():
    case = Case(2, 21, 4, 2, 8, 8, 2, 8)
    inp = make_inputs(case)
    ref = o1.run_inputs(inp)
    exp = dict(inp, q=inp["q"].repeat_interleave(2, dim=3), k=inp["k"].repeat_interleave(2, dim=3))
    out = o1.run_inputs(exp)
    for i in range(5):
        assert same(out[i], ref[i]), NAMES[i]
    # permuting heads (with their parameters) permutes the outputs
    perm = torch.tensor([2, 0, 3, 1])
    pin = dict(exp)
    for n in ("v", "dout", "z"):
        pin[n] = exp[n][:, :, perm]
    pin["q"], pin["k"] = exp["q"][:, :, :, perm], exp["k"][:, :, :, perm]
    for n in ("q_bias", "k_bias", "mimo_v", "mimo_o", "mimo_z", "d"):
        pin[n] = exp[n][perm]
    pin["angles"] = exp["angles"][:, :, perm]
    for n in ("da_cs", "da_cs_rev", "dt", "trap", "segsum"):
        pin[n] = exp[n][:, perm]
    out = o1.run_inputs(pin)
    p = perm.numpy()
    assert same(out[0], ref[0][:, p]) and same(out[1], ref[1][:, p])
    assert same(out[2], ref[2][:, :, p]) and same(out[3], ref[3][:, p])
    assert same(out[4], ref[4][:, p])


def test_head_slice_equals_full_run():
    case = Case(2, 19, 4, 2, 8, 8, 2, 8)
    inp = make_inputs(case)
    ref = o1.run_inputs(inp)
    for b, h in ((0, 0), (1, 3), (1, 2)):
        out = o1.run_inputs(o1.slice_heads(inp, b, h))
        assert same(out[0][0, 0], ref[0][b, h]) and same(out[1][0, 0], ref[1][b, h])
        assert same(out[2][0, :, 0], ref[2][b, :, h]) and same(out[3][0, 0], ref[3][b, h])
        assert same(out[4][0, 0], ref[4][b, h])


def test_unused_segsum_entries_are_ignored(base_case):
    """Entries on and above the diagonal of each segsum tile, and the padded rows
    and columns of the tail tile, never reach an output."""
    case, inp, ref = base_case
    seg = inp["segsum"].clone()
    C = case.C
    seg[..., torch.ones(C, C, dtype=torch.bool).triu()] = float("nan")
    last = case.S - (case.nchunks - 1) * C
    seg[:, :, -1, last:, :] = float("nan")
    seg[:, :, -1, :, last:] = float("nan")
    out = o1.run_inputs(dict(inp, segsum=seg))
    for i in range(5):
        assert same(out[i], ref[i]), NAMES[i]


# ---------------------------------------------------------------- calibration
def test_contract_distance_from_exact():
    """The bf16 contract sits ~1e-3..1e-2 (relative RMS) away from exact arithmetic:
    dropping its roundings is a detectable mistake at the 1e-3 parity gate."""
    inp = make_inputs(CONFIGS["tiny"], want_exact=True)
    c = o1.run_inputs(inp)
    e = o2.run_inputs(inp)
    for i, n in enumerate(NAMES):
        r = rel(c[i], e[i])
        assert 5e-4 < r < 3e-2, (n, r)


@pytest.mark.parametrize("case", UT_CASES, ids=lambda c: c.name)
def test_ut_recipe_runs_finite(case):
    """The pages' own unit-test input formulas (independent random controls)."""
    out = o1.run_inputs(make_inputs(case))
    for i, n in enumerate(NAMES):
        if out[i] is not None:
            assert np.isfinite(out[i]).all(), n
    assert (out[0] is None) == (not case.reduce_o)
    assert (out[2] is None) == (not case.has_z)
