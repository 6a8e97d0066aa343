"""GPU parity of the fp32-intermediate kernels (through the C ABI).

* ``mamba_mimo_bwd_fwd_fp32`` / ``mamba_mimo_fwd_fp32`` against the oracle's
  fp32-intermediate mode (the pages' FP32 reference): relative RMS < 2e-4 on
  every output (a fifth of the operator's 1e-3 bar: with no intermediate bf16
  rounding the two sides differ only by fp32 summation order and by rare
  bf16 rounding flips of the outputs), dtypes as the bf16 operator's.
* ``mamba3_siso_fwd`` against the float64 SISO oracle: relative RMS below the
  SISO page's thresholds (2^-8 for bf16, 2^-11 for fp16 outputs) and below 1e-3
  against the oracle rounded to the output dtype.
Cases span several tiles, segments and ragged tails, GQA, both dtypes, both
chunk sizes, the branch combinations, the perf shapes, and the 128-row tiles
whose K~ tile lives in scratch (R * C > 64 with N or P = 128: small shapes on
every head, the two 128-wide workloads at full size on sampled heads).
"""

import numpy as np
import pytest
import torch

from oracle import o1, siso
from synth.inputs import (API_ORDER, CONFIGS, SISO_CONFIGS, SISO_ORDER, Case, SisoCase, make_inputs,
                          make_siso_inputs)

from ._parity import compare, log, rel_rms, to_device

TOL32 = 2e-4

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from mamba_mimo_chunked_amd import _lib
    _lib.lib()


def run_bwd32(dinp):
    from mamba_mimo_chunked_amd import mamba_mimo_bwd_fwd_fp32
    res = mamba_mimo_bwd_fwd_fp32(*[dinp[n] for n in API_ORDER], dinp["chunk_size"], dinp["rotary_dim_divisor"])
    torch.cuda.synchronize()
    return res


def run_fwd32(dinp):
    from mamba_mimo_chunked_amd import mamba_mimo_fwd_fp32
    o = mamba_mimo_fwd_fp32(*[dinp[n] for n in API_ORDER if n != "dout"], dinp["chunk_size"],
                            dinp["rotary_dim_divisor"])
    torch.cuda.synchronize()
    return o


BWD32_CASES = [
    Case(1, 64, 2, 1, 16, 16, 2, 16, name="f32_tiny"),
    Case(1, 300, 3, 1, 64, 64, 4, 16, name="f32_segments_tail"),
    Case(2, 777, 4, 2, 32, 64, 2, 16, name="f32_gqa_tail_r2"),
    Case(1, 1000, 2, 1, 64, 64, 1, 64, name="f32_r1_c64"),
    Case(1, 1000, 2, 1, 64, 32, 2, 32, name="f32_r2_c32"),
    Case(1, 333, 2, 2, 64, 32, 4, 16, reduce_o=False, has_z=True, has_d=True, name="f32_nonreduced_z"),
    Case(2, 257, 4, 4, 64, 64, 4, 16, reduce_o=False, has_z=False, has_d=False, name="f32_nonreduced_noz"),
    Case(1, 200, 2, 1, 64, 64, 4, 16, reduce_o=True, has_z=False, has_d=True, name="f32_reduced_noz"),
    Case(1, 130, 2, 1, 16, 16, 8, 8, name="f32_r8_c8"),
    Case(1, 95, 1, 1, 32, 48, 3, 6, rd=2, name="f32_r3_c6_rd2_p48"),
    Case(1, 500, 2, 1, 128, 64, 4, 16, name="f32_n128_r4"),
    Case(1, 400, 2, 1, 64, 128, 2, 16, name="f32_p128_r2"),
    Case(1, 300, 1, 1, 64, 64, 8, 16, name="f32_r8_c16_mt128"),
    # calls without y (states and qk_dot only) on other tiles
    Case(1, 200, 2, 2, 32, 64, 2, 32, reduce_o=False, has_z=False, name="f32_noy_r2_c32"),
    Case(1, 150, 2, 1, 64, 32, 3, 16, reduce_o=False, has_z=False, has_d=False, name="f32_noy_r3_p32"),
]


@pytest.mark.parametrize("case", BWD32_CASES, ids=lambda c: c.name)
def test_bwd_fwd_fp32(case):
    log(f"[fp32] {case.name} B={case.B} S={case.S} H={case.H} G={case.G} N={case.N} P={case.P} "
        f"R={case.R} C={case.C}")
    inp = make_inputs(case)
    ref = o1.run_inputs(inp, fp32=True)
    got = run_bwd32(to_device(inp))
    errs = compare(got, ref, tol=TOL32, label=f"{case.name}: ")
    log("    " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("case", [Case(1, 300, 3, 1, 64, 64, 4, 16, name="f32_exact_reduced_z"),
                                  Case(2, 257, 4, 4, 64, 64, 4, 16, reduce_o=False, has_z=False, has_d=False,
                                       name="f32_exact_nonreduced")], ids=lambda c: c.name)
def test_bwd_fwd_fp32_shape_exact_and_generic_agree(case, monkeypatch):
    """R=4, C=16, N=P=64 with rotary divisor 4 runs the shape-exact fp32 instances
    (sizes as constants); the generic ones (forced through MIMO_FORCE_GENERIC) must give
    the same bits, and both meet the oracle bar. The layer output likewise."""
    log(f"[fp32 exact-vs-generic] {case.name}")
    inp = make_inputs(case)
    d = to_device(inp)
    ex, ex_o = run_bwd32(d), run_fwd32(d)
    monkeypatch.setenv("MIMO_FORCE_GENERIC", "1")
    gen, gen_o = run_bwd32(d), run_fwd32(d)
    monkeypatch.delenv("MIMO_FORCE_GENERIC")
    ref = o1.run_inputs(inp, fp32=True)
    compare(ex, ref, tol=TOL32, label=f"{case.name} exact: ")
    compare(gen, ref, tol=TOL32, label=f"{case.name} generic: ")
    for a, b in zip(ex, gen):
        if a is None or b is None:
            assert a is None and b is None
            continue
        assert torch.equal(a, b), "shape-exact and generic fp32 instances differ"
    assert torch.equal(ex_o, gen_o), "shape-exact and generic fp32 layer outputs differ"


def test_bwd_fwd_fp32_perf_shape_all_heads():
    case = CONFIGS["perf_s8192"].with_(seed=5)
    log("[fp32] perf_s8192 (all heads)")
    inp = make_inputs(case)
    got = run_bwd32(to_device(inp))
    errs = compare(got, o1.run_inputs(inp, fp32=True), tol=TOL32, label="perf_s8192 fp32: ")
    log("    " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_bwd_fwd_fp32_gqa_tail_nonreduced_sampled():
    case = CONFIGS["gqa_tail_nonreduced"].with_(seed=9)
    log("[fp32] gqa_tail_nonreduced (sampled heads)")
    inp = make_inputs(case)
    got = run_bwd32(to_device(inp))
    for b, h in [(0, 0), (1, 31)]:
        ref = o1.run_inputs(o1.slice_heads(inp, b, h), fp32=True)
        sl = (None, got.states[b:b + 1, h:h + 1], None, None, got.qk_dot[b:b + 1, h:h + 1])
        compare(sl, ref, tol=TOL32, label=f"gqa b={b} h={h}: ")


@pytest.mark.parametrize("k", range(96))
def test_bwd_fwd_fp32_random_shapes(k):
    """Seeded random shapes (the same draw as the bf16 path's random parity cases) for
    the fp32-intermediate variant against the oracle in fp32 mode; shapes beyond the
    variant's LDS and scratch tiles must be refused as such."""
    from .test_gpu_parity import _random_case
    case = _random_case(k)
    log(f"[fp32 random] {case}")
    inp = make_inputs(case)
    try:
        got = run_bwd32(to_device(inp))
    except NotImplementedError as e:
        pytest.skip(f"{case.name}: {e}")
    compare(got, o1.run_inputs(inp, fp32=True), tol=TOL32, label=f"{case.name} fp32: ")


def test_fp32_is_closer_to_exact_than_bf16_contract():
    """The fp32 variant's dmimo outputs sit far closer to exact arithmetic than the
    bf16-contract operator's (both on the GPU, the same inputs)."""
    from mamba_mimo_chunked_amd import mamba_mimo_bwd_fwd
    case = Case(1, 512, 2, 1, 64, 64, 4, 16, name="closer")
    inp = make_inputs(case)
    d = to_device(inp)
    f32 = run_bwd32(d)
    b16 = mamba_mimo_bwd_fwd(*[d[n] for n in API_ORDER], 16, 4)
    e = o1.run_inputs(inp, exact=True)
    for i in (0, 3):
        ef = rel_rms(f32[i].cpu().numpy(), e[i])
        eb = rel_rms(b16[i].cpu().numpy(), e[i])
        log(f"    output {i}: fp32 {ef:.2e}  bf16 contract {eb:.2e}")
        assert ef * 20 < eb


KG_CASES = [
    Case(1, 300, 2, 1, 128, 128, 8, 16, name="kg_n128_p128_r8"),
    Case(1, 300, 2, 1, 128, 64, 2, 64, name="kg_n128_c64"),
    Case(2, 150, 4, 2, 64, 128, 4, 32, reduce_o=False, has_z=True, has_d=True, name="kg_p128_nonreduced_z"),
    Case(1, 77, 2, 1, 128, 32, 3, 24, reduce_o=True, has_z=False, has_d=False, name="kg_n128_p32_r3_c24"),
    Case(1, 150, 2, 2, 128, 128, 8, 16, reduce_o=False, has_z=False, name="kg_noy_n128_p128_r8"),
]


@pytest.mark.parametrize("case", KG_CASES, ids=lambda c: c.name)
def test_bwd_fwd_fp32_k_tile_in_scratch(case):
    """128-row tiles beyond the LDS with all tiles in it: K~ in scratch."""
    log(f"[fp32] {case.name} B={case.B} S={case.S} H={case.H} G={case.G} N={case.N} P={case.P} "
        f"R={case.R} C={case.C}")
    inp = make_inputs(case)
    got = run_bwd32(to_device(inp))
    errs = compare(got, o1.run_inputs(inp, fp32=True), tol=TOL32, label=f"{case.name}: ")
    log("    " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,heads", [("wide_chunk_n128", ((0, 0), (3, 31))), ("max_rank_tile", ((1, 9),))])
def test_bwd_fwd_fp32_wide_workloads_sampled(name, heads):
    """The two 128-wide workloads at full size; the oracle runs on sampled (batch,
    head) pairs, the per-head outputs compared on those heads and dmimo_o / dmimo_z
    on their (batch, head) entries."""
    case = CONFIGS[name].with_(seed=13)
    log(f"[fp32] {name} (sampled heads)")
    inp = make_inputs(case)
    got = run_bwd32(to_device(inp))
    for b, h in heads:
        ref = o1.run_inputs(o1.slice_heads(inp, b, h), fp32=True)
        pick = lambda x, dz=False: None if x is None else (x[b:b + 1, :, h:h + 1] if dz else x[b:b + 1, h:h + 1])
        sl = (pick(got[0]), pick(got[1]), pick(got[2], dz=True), pick(got[3]), pick(got[4]))
        errs = compare(sl, ref, tol=TOL32, label=f"{name} b={b} h={h}: ")
        log(f"    b={b} h={h} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("case", [Case(1, 300, 3, 1, 64, 64, 4, 16, name="fwd32_reduced"),
                                  Case(1, 200, 2, 1, 64, 32, 2, 16, reduce_o=False, has_z=True,
                                       name="fwd32_perrank"),
                                  Case(1, 150, 2, 1, 32, 64, 4, 16, reduce_o=True, has_z=False,
                                       name="fwd32_noz")],
                         ids=lambda c: c.name)
def test_fwd_fp32(case):
    inp = make_inputs(case)
    ref = o1.run_fwd_inputs(inp, fp32=True)
    got = run_fwd32(to_device(inp)).float().cpu().numpy()
    e = rel_rms(got, ref)
    log(f"    {case.name}: o={e:.2e}")
    assert got.shape == ref.shape and e < TOL32


# ---------------------------------------------------------------- SISO forward
def run_siso(dinp):
    from mamba_mimo_chunked_amd import mamba3_siso_fwd
    o = mamba3_siso_fwd(*[dinp[n] for n in SISO_ORDER], chunk_size=dinp["chunk_size"])
    torch.cuda.synchronize()
    return o


def _siso_dev(inp):
    return {n: (v.to("cuda") if torch.is_tensor(v) else v) for n, v in inp.items()}


def _round(x, dtype):
    return torch.from_numpy(x).to(dtype).double().numpy()


def _check_siso(case, heads=None):
    log(f"[siso] {case.name} B={case.B} S={case.S} Hq={case.Hq} H={case.H} K={case.K} V={case.V} "
        f"C={case.C} A={case.width} {case.dtype} z={case.has_z} d={case.has_d}")
    inp = make_siso_inputs(case)
    got = run_siso(_siso_dev(inp))
    dt = torch.float16 if case.dtype == "fp16" else torch.bfloat16
    assert got.dtype == dt and tuple(got.shape) == (case.B, case.S, case.H, case.V)
    g = got.double().cpu().numpy()
    assert np.isfinite(g).all()
    ref = siso.run(*[inp[n] for n in SISO_ORDER], chunk_size=case.C)
    gate = 2.0 ** -11 if case.dtype == "fp16" else 2.0 ** -8
    e64 = rel_rms(g, ref)
    er = rel_rms(g, _round(ref, dt))
    log(f"    vs float64 {e64:.2e} (gate {gate:.2e}); vs float64 rounded to {case.dtype} {er:.2e}")
    assert e64 < gate and er < 1e-3


SISO_CASES = [
    SISO_CONFIGS["siso_example"],
    SISO_CONFIGS["siso_example"].with_(dtype="bf16", name="example_bf16"),
    SisoCase(1, 200, 2, 4, 64, 64, 32, name="c32_tail"),
    SisoCase(2, 333, 1, 2, 128, 64, 64, A=16, name="k128_a16_tail"),
    SisoCase(1, 300, 2, 2, 64, 128, 64, dtype="fp16", name="v128_fp16"),
    SisoCase(1, 100, 4, 4, 32, 32, 32, has_z=False, has_d=False, name="no_z_no_d"),
    SisoCase(1, 64, 1, 1, 16, 16, 64, A=0, name="no_rotation"),
    SisoCase(1, 1, 1, 1, 64, 64, 64, name="one_token"),
]


def _random_siso(k):
    """A seeded random SISO shape: K and V multiples of 16 up to 128, chunks of 32 or
    64 tokens, an even rotated width up to K/2 (zero included), query heads dividing
    the value heads, bf16 or fp16, a ragged tail and random z/D flags."""
    rng = np.random.default_rng(5000 + k)
    K = int(rng.choice([16, 32, 48, 64, 96, 128]))
    V = int(rng.choice([16, 32, 48, 64, 96, 128]))
    C = int(rng.choice([32, 64]))
    A = 2 * int(rng.integers(0, K // 4 + 1))
    Hq = int(rng.choice([1, 2]))
    H = Hq * int(rng.choice([1, 2, 3]))
    S = int(rng.integers(1, 4 * C + 1))
    return SisoCase(1, S, Hq, H, K, V, C, A=A, dtype=str(rng.choice(["bf16", "fp16"])),
                    has_z=bool(rng.integers(2)), has_d=bool(rng.integers(2)), seed=k, name=f"siso_random_{k}")


@pytest.mark.parametrize("k", range(48))
def test_siso_random_shapes(k):
    """Seeded random SISO shapes against the SISO oracle; a shape beyond the tiles
    must be refused as such."""
    case = _random_siso(k)
    try:
        _check_siso(case)
    except NotImplementedError as e:
        pytest.skip(f"{case.name}: {e}")


@pytest.mark.parametrize("case", SISO_CASES, ids=lambda c: c.name)
def test_siso(case):
    _check_siso(case)


@pytest.mark.parametrize("name", ["siso_s8192_k128", "siso_s8192_k128_fp16"])
def test_siso_perf_shapes_all_heads(name):
    _check_siso(SISO_CONFIGS[name])


@pytest.mark.parametrize("case", [SisoCase(1, 300, 2, 4, 128, 64, 64, name="sx_bf16_tail"),
                                  SisoCase(2, 257, 3, 3, 128, 64, 64, dtype="fp16", has_z=False,
                                           name="sx_fp16_no_z")], ids=lambda c: c.name)
def test_siso_shape_exact_and_generic_agree(case, monkeypatch):
    """K=128, V=64, chunk 64 with every pair rotated runs the shape-exact SISO
    instances (sizes as constants); the generic ones (forced through
    MIMO_FORCE_GENERIC) must give the same bits, and both meet the oracle gates."""
    log(f"[siso exact-vs-generic] {case.name}")
    assert case.width == 64
    d = _siso_dev(make_siso_inputs(case))
    ex = run_siso(d)
    monkeypatch.setenv("MIMO_FORCE_GENERIC", "1")
    gen = run_siso(d)
    monkeypatch.delenv("MIMO_FORCE_GENERIC")
    assert torch.equal(ex.view(torch.int16), gen.view(torch.int16)), "shape-exact and generic SISO instances differ"
    _check_siso(case)


def test_siso_determinism_and_every_element_written():
    case = SisoCase(1, 300, 2, 2, 64, 64, 64, name="det")
    d = _siso_dev(make_siso_inputs(case))
    from mamba_mimo_chunked_amd import mamba3_siso_fwd
    a = mamba3_siso_fwd(*[d[n] for n in SISO_ORDER], chunk_size=64)
    b = torch.full_like(a, float("nan"))
    mamba3_siso_fwd(*[d[n] for n in SISO_ORDER], chunk_size=64, out=b)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
