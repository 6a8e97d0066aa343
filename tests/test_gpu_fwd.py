"""GPU parity of the layer output ``mamba_mimo_fwd`` (through the C ABI) against
the CPU oracle's ``o1.run_fwd`` on the same seeded inputs.

Bar: RMS(gpu - oracle) / RMS(oracle) < 1e-3, bf16 dtype, right shape. Cases:
the perf workload shape on every head, shapes that span several tiles,
segments and ragged tails (GQA, C=64, R=8, R=3/C=6/rd=2, reduced and
per-rank outputs, with and without z and d), the larger workloads on sampled
heads. Bit-for-bit checks: shape-exact vs generic kernel instances, every
element written, determinism, and the forward's y against the backward's
(dmimo_o with a one-hot dout reads y out of the backward kernel).
"""

import numpy as np
import pytest
import torch

from oracle import o1
from synth.inputs import API_ORDER, CONFIGS, Case, make_inputs

from ._parity import TOL, check_elements, log, rel_rms, run_gpu, to_device

pytestmark = pytest.mark.gpu

FWD_ORDER = [n for n in API_ORDER if n != "dout"]

FWD_CASES = [
    Case(1, 300, 3, 1, 64, 64, 4, 16, name="fwd_segments_tail"),
    Case(2, 777, 4, 2, 32, 64, 2, 16, name="fwd_gqa_tail_r2"),
    Case(1, 1000, 2, 1, 128, 64, 2, 64, name="fwd_c64_n128"),
    Case(1, 500, 2, 1, 128, 128, 8, 16, name="fwd_r8_n128_p128"),
    Case(1, 333, 2, 2, 64, 32, 4, 16, reduce_o=False, has_z=True, has_d=True, name="fwd_perrank_z"),
    Case(2, 257, 4, 4, 64, 64, 4, 16, reduce_o=False, has_z=False, has_d=False, name="fwd_perrank_noz"),
    Case(1, 200, 2, 1, 64, 64, 4, 16, reduce_o=True, has_z=False, has_d=True, name="fwd_reduced_noz"),
    Case(1, 130, 2, 1, 16, 16, 8, 8, name="fwd_r8_c8_small"),
    Case(1, 95, 1, 1, 32, 48, 3, 6, rd=2, name="fwd_r3_c6_rd2_p48"),
    Case(1, 64, 1, 1, 64, 64, 1, 64, name="fwd_r1_c64"),
    Case(1, 1, 1, 1, 64, 64, 4, 16, name="fwd_one_token"),
    # per-rank output whose R*C rows of P values do not fit the staging tile: the
    # epilogue's direct 2-byte stores
    Case(1, 300, 2, 1, 32, 64, 4, 16, reduce_o=False, has_z=True, has_d=True, name="fwd_perrank_p_gt_n"),
]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from mamba_mimo_chunked_amd import _lib
    _lib.lib()


def run_fwd(dinp: dict, **kw):
    from mamba_mimo_chunked_amd import mamba_mimo_fwd
    args = [dinp[n] for n in FWD_ORDER]
    o = mamba_mimo_fwd(*args, dinp["chunk_size"], dinp["rotary_dim_divisor"], **kw)
    torch.cuda.synchronize()
    return o


def _cmp(got, ref, label, ulp_frac=0.999):
    assert got.dtype == torch.bfloat16, f"{label}: dtype {got.dtype}"
    g = got.float().cpu().numpy()
    assert g.shape == ref.shape, f"{label}: shape {g.shape} vs {ref.shape}"
    assert np.isfinite(g).all(), f"{label}: non-finite values"
    e = rel_rms(g, ref)
    log(f"    {label}: o={e:.2e}")
    assert e < TOL, f"{label}: rel RMS {e:.3e} >= {TOL}"
    check_elements("o", g, ref, bf16=True, label=f"{label}: ", ulp_frac=ulp_frac)
    return e


def _check(case, *, zero_angles=False, ulp_frac=0.999):
    log(f"[fwd] {case.name} B={case.B} S={case.S} H={case.H} G={case.G} N={case.N} P={case.P} "
        f"R={case.R} C={case.C} reduce_o={case.reduce_o} z={case.has_z}" + (" (zero angles)" if zero_angles else ""))
    inp = make_inputs(case)
    if zero_angles:
        inp["angles"] = torch.zeros_like(inp["angles"])
    ref = o1.run_fwd_inputs(inp)
    got = run_fwd(to_device(inp))
    return _cmp(got, ref, case.name, ulp_frac)


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: c.name)
def test_fwd_shapes(case):
    _check(case)


@pytest.mark.parametrize("k", range(96))
def test_fwd_random_shapes(k):
    """Seeded random shapes (the same draw as the backward's random parity cases) for
    the layer output against the oracle, with zero angles at the full bars and with
    the drawn angles at 99.5 % of elements within one ulp (as the backward's random
    cases); an LDS refusal must say so."""
    from .test_gpu_parity import _random_case
    case = _random_case(k)
    try:
        _check(case, zero_angles=True)
        _check(case, ulp_frac=0.995)
    except NotImplementedError as e:
        assert "bytes of LDS" in str(e), e
        pytest.skip(f"{case.name}: {e}")


def test_fwd_tiny_config():
    _check(CONFIGS["tiny"].with_(name="fwd_tiny"))


def test_fwd_perf_shape_all_heads():
    """The shape the benchmark times (shape-exact kernel instances), every head."""
    _check(CONFIGS["perf_s8192"].with_(seed=7, name="fwd_perf_s8192"))


@pytest.mark.parametrize("name,heads", [("gqa_tail_nonreduced", [(0, 0), (1, 31)]),
                                        ("wide_chunk_n128", [(0, 0), (3, 31)]),
                                        ("max_rank_tile", [(1, 15)])])
def test_fwd_full_sizes_sampled_heads(name, heads):
    case = CONFIGS[name].with_(seed=321)
    log(f"[fwd-full] {name}: generating inputs")
    inp = make_inputs(case)
    got = run_fwd(to_device(inp))
    for b, h in heads:
        ref = o1.run_fwd_inputs(o1.slice_heads(inp, b, h))
        sl = got[b:b + 1, :, h:h + 1] if case.reduce_o else got[b:b + 1, :, :, h:h + 1]
        _cmp(sl, ref, f"{name} b={b} h={h}")


def test_fwd_determinism_and_every_element_written():
    case = Case(1, 300, 3, 1, 64, 64, 4, 16)
    d = to_device(make_inputs(case))
    a = run_fwd(d)
    b = torch.full_like(a, float("nan"))
    run_fwd(d, out=b)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("case", [Case(1, 300, 2, 1, 64, 64, 4, 16, name="ex_r4_c16"),
                                  Case(1, 190, 2, 1, 32, 32, 2, 32, name="ex_r2_c32")],
                         ids=lambda c: c.name)
def test_fwd_shape_exact_and_generic_kernels_agree(case, monkeypatch):
    d = to_device(make_inputs(case))
    ex = run_fwd(d)
    monkeypatch.setenv("MIMO_FORCE_GENERIC", "1")
    gen = run_fwd(d)
    monkeypatch.delenv("MIMO_FORCE_GENERIC")
    assert torch.equal(ex.view(torch.int16), gen.view(torch.int16))
    _cmp(ex, o1.run_fwd_inputs(make_inputs(case)), case.name)


@pytest.mark.parametrize("t", [0, 5, 137, 299])
def test_fwd_y_equals_backward_y_bitwise(t):
    """Without z and with a one-hot dout at token t, the backward's dmimo_o[r,p] is
    y[t,r,p] (one nonzero product, exact sums); the per-rank forward output
    without z is bf16 y itself. Both must agree bit for bit."""
    case = Case(1, 300, 2, 1, 64, 64, 4, 16, reduce_o=False, has_z=False, has_d=True, name="y")
    inp = make_inputs(case)
    d = to_device(inp)
    o = run_fwd(d)                                            # [B,S,R,H,P]
    dout = torch.zeros((1, 300, 2, 64), dtype=torch.bfloat16, device="cuda")
    dout[:, t] = 1.0
    mimo_o = torch.ones((2, 4, 64), dtype=torch.float32, device="cuda")
    bw = run_gpu(dict(d, dout=dout, mimo_o=mimo_o))
    y_bwd = bw.dmimo_o[0]                                     # [H,R,P] fp32 = y
    y_fwd = o[0, t].permute(1, 0, 2).float()                  # [H,R,P]
    assert torch.equal(y_bwd, y_fwd)
