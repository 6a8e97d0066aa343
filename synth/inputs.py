"""Seeded synthetic inputs for the Mamba-3 MIMO backward first stage.

This module only draws random tensors and lays them out in the operator's
input shapes and dtypes. It holds none of the operator's arithmetic; both the
HIP path (through the tests and the benchmark) and the CPU oracle consume what
it returns.

Two recipes are provided:

* ``"configs"`` -- the workload distributions of the benchmark shapes:
  q, k, v, dout, z ~ N(0,1) in bf16; q_bias, k_bias ~ 0.1*N(0,1);
  mimo_v/o/z ~ 0.5*N(0,1); angles ~ U(-pi, pi); dt = softplus(N(0,1) - 3);
  A_h ~ U(1, 16) and a per-token log-decay da = -A_h * dt; trap =
  sigmoid(N(0,1)) rounded to bf16; d ~ N(0,1). The chunked controls
  da_cs / da_cs_rev / segsum are built from da per chunk (inclusive cumsum,
  the remaining sum to the chunk's last token, and pairwise differences),
  in float64 and stored as float32. This is the one reading of the three
  undefined control tensors under which the chunked state update equals a
  token-by-token recurrence (the state update decays by exp(da_cs) at the
  chunk's last token; the stage-2 page rebuilds da_cs_rev and segsum from
  da_cs after extending it).
* ``"ut"`` -- the unit-test distributions printed on the operator's page
  (Triton-Ascend mamba_mimo_bwd_fwd, unit-test file, input builder): controls
  drawn independently of each other, so they are not consistent with one da.
  The API must accept any finite float32 controls.

Entries of segsum above the diagonal are never used by the method; the
"configs" recipe fills them with -inf.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

__all__ = ["Case", "make_inputs", "API_ORDER", "CONFIGS", "UT_CASES", "ATK_CASES", "SisoCase",
           "make_siso_inputs", "SISO_ORDER", "SISO_CONFIGS"]

# Positional order of the tensor arguments of mamba_mimo_bwd_fwd.
API_ORDER = (
    "dout", "q", "k", "v", "q_bias", "k_bias", "mimo_v", "mimo_o", "z", "mimo_z",
    "angles", "da_cs", "da_cs_rev", "dt", "trap", "d", "segsum",
)


@dataclass(frozen=True)
class Case:
    B: int
    S: int
    H: int
    G: int
    N: int
    P: int
    R: int
    C: int
    rd: int = 4
    reduce_o: bool = True
    has_z: bool = True
    has_d: bool = True
    seed: int = 123
    recipe: str = "configs"
    name: str = field(default="", compare=False)

    @property
    def nchunks(self) -> int:
        return (self.S + self.C - 1) // self.C

    def with_(self, **kw) -> "Case":
        return replace(self, **kw)


# The five workload shapes (tiny parity shape, the pages' performance shape,
# GQA + tail + non-reduced dout, wide chunk with large state, maximum rank tile).
CONFIGS = {
    "tiny": Case(1, 64, 2, 1, 16, 16, 2, 16, name="tiny"),
    "perf_s8192": Case(1, 8192, 16, 1, 64, 64, 4, 16, name="perf_s8192"),
    "gqa_tail_nonreduced": Case(2, 4100, 32, 4, 64, 64, 4, 16, reduce_o=False, has_z=False,
                                has_d=False, name="gqa_tail_nonreduced"),
    "wide_chunk_n128": Case(4, 16384, 32, 8, 128, 64, 2, 64, name="wide_chunk_n128"),
    "max_rank_tile": Case(2, 32768, 16, 2, 128, 128, 8, 16, name="max_rank_tile"),
}


def _ut(name, **kw):
    base = dict(B=1, S=32, H=1, G=1, N=64, P=64, R=4, C=16, reduce_o=True, has_z=False,
                has_d=False, seed=123, recipe="ut")
    base.update(kw)
    return Case(name=name, **base)


# The unit-test grid of the operator's page (branch combinations, GQA, tail seeds,
# batch/groups, non-power-of-two tail, tail chunk, and the shape sweep).
UT_CASES = [
    _ut("branch_TFF", reduce_o=True, has_z=False, has_d=False),
    _ut("branch_TTT", reduce_o=True, has_z=True, has_d=True),
    _ut("branch_FFT", reduce_o=False, has_z=False, has_d=True),
    _ut("branch_FTF", reduce_o=False, has_z=True, has_d=False),
    _ut("gqa", H=2, G=1, has_z=True, has_d=True),
    _ut("tail_seed0", seed=0, S=35, H=2, has_z=True, has_d=True),
    _ut("tail_seed1", seed=1, S=35, H=2, has_z=True, has_d=True),
    _ut("tail_seed42", seed=42, S=35, H=2, has_z=True, has_d=True),
    _ut("batch_groups", B=2, H=4, G=2, S=20, has_z=True, has_d=True),
    _ut("npot_tail", S=13, R=3, C=6, has_z=True, has_d=True),
    _ut("tail_chunk", S=20, has_z=True, has_d=True),
    _ut("shape_32_64_4_16", N=32, P=64, R=4, C=16, S=32),
    _ut("shape_128_32_4_16", N=128, P=32, R=4, C=16, S=32),
    _ut("shape_64_128_4_16", N=64, P=128, R=4, C=16, S=32),
    _ut("shape_128_64_8_8", N=128, P=64, R=8, C=8, S=16),
    _ut("shape_64_64_3_6", N=64, P=64, R=3, C=6, S=12),
    _ut("shape_64_64_1_64", N=64, P=64, R=1, C=64, S=128),
]

# The four shapes of the pages' ATK harness (B,S,H,G,N,P,R,C), all branches on.
ATK_CASES = [
    Case(1, 16, 1, 1, 64, 64, 4, 16, name="atk0"),
    Case(1, 32, 1, 1, 64, 64, 4, 16, name="atk1"),
    Case(1, 20, 1, 1, 64, 64, 4, 16, name="atk2"),
    Case(1, 32, 2, 1, 64, 64, 4, 16, name="atk3"),
]


def _controls_from_da(da: torch.Tensor, C: int):
    """Chunked controls from a per-token log decay da [B,H,S] (float64).

    da_cs[t]     = sum_{l=c0..t} da_l            (inclusive, restarts at each chunk)
    da_cs_rev[t] = sum_{l=t+1..last(c)} da_l     (what remains to the chunk's last token)
    segsum[c,i,j]= da_cs[c0+i] - da_cs[c0+j]     for i >= j, -inf above the diagonal.
    The tail chunk is extended with da = 0 past S.
    """
    B, H, S = da.shape
    nc = (S + C - 1) // C
    pad = nc * C - S
    dap = torch.cat([da, da.new_zeros(B, H, pad)], dim=2).view(B, H, nc, C)
    cs = dap.cumsum(dim=3)                                  # [B,H,nc,C]
    # remaining sum to the last *valid* token of each chunk
    valid = torch.arange(nc * C).view(nc, C) < S            # [nc,C]
    cs_last = torch.stack([cs[:, :, c, int(valid[c].sum()) - 1] for c in range(nc)], dim=2)
    rev = cs_last[..., None] - cs
    seg = cs[..., :, None] - cs[..., None, :]               # [B,H,nc,C,C]
    upper = torch.ones(C, C, dtype=torch.bool).triu(1)
    seg = seg.masked_fill(upper, float("-inf"))
    da_cs = cs.reshape(B, H, nc * C)[..., :S]
    da_cs_rev = rev.reshape(B, H, nc * C)[..., :S]
    return da_cs, da_cs_rev, seg


def make_inputs(case: Case, *, want_exact: bool = False):
    """Draw the operator's inputs for ``case`` on the CPU.

    Returns a dict holding every API tensor (``API_ORDER`` names; absent optional
    tensors are None), ``chunk_size`` and ``rotary_dim_divisor``, and, for the
    "configs" recipe, ``da`` (float64 [B,H,S] per-token log decay). With
    ``want_exact`` the float64 controls built from da are returned too, under
    ``da_cs64``, ``da_cs_rev64`` and ``segsum64``.
    """
    B, S, H, G, N, P, R, C = case.B, case.S, case.H, case.G, case.N, case.P, case.R, case.C
    g = torch.Generator().manual_seed(case.seed)
    bf16, f32 = torch.bfloat16, torch.float32
    W = N // case.rd
    nc = case.nchunks
    out = {}
    if case.recipe == "configs":
        out["q"] = torch.randn((B, S, R, G, N), generator=g).to(bf16)
        out["k"] = torch.randn((B, S, R, G, N), generator=g).to(bf16)
        out["v"] = torch.randn((B, S, H, P), generator=g).to(bf16)
        dshape = (B, S, H, P) if case.reduce_o else (B, S, R, H, P)
        out["dout"] = torch.randn(dshape, generator=g).to(bf16)
        out["z"] = torch.randn((B, S, H, P), generator=g).to(bf16) if case.has_z else None
        out["q_bias"] = 0.1 * torch.randn((H, R, N), generator=g)
        out["k_bias"] = 0.1 * torch.randn((H, R, N), generator=g)
        out["mimo_v"] = 0.5 * torch.randn((H, R, P), generator=g)
        out["mimo_o"] = 0.5 * torch.randn((H, R, P), generator=g) if case.reduce_o else None
        out["mimo_z"] = 0.5 * torch.randn((H, R, P), generator=g) if case.has_z else None
        out["angles"] = (torch.rand((B, S, H, W), generator=g) * 2 - 1) * math.pi
        out["dt"] = torch.nn.functional.softplus(torch.randn((B, H, S), generator=g) - 3.0)
        A = 1.0 + 15.0 * torch.rand((H,), generator=g, dtype=torch.float64)
        out["trap"] = torch.sigmoid(torch.randn((B, H, S), generator=g)).to(bf16)
        out["d"] = torch.randn((H,), generator=g) if case.has_d else None
        da = -A[None, :, None] * out["dt"].double()
        cs, rev, seg = _controls_from_da(da, C)
        out["da_cs"], out["da_cs_rev"], out["segsum"] = cs.to(f32), rev.to(f32), seg.to(f32)
        out["da"] = da
        if want_exact:
            out["da_cs64"], out["da_cs_rev64"], out["segsum64"] = cs, rev, seg
    elif case.recipe == "ut":
        torch.manual_seed(case.seed)
        q = torch.randn((B, S, R, G, N), dtype=bf16)
        out["q"] = q
        out["k"] = torch.randn_like(q)
        out["v"] = torch.randn((B, S, H, P), dtype=bf16)
        dshape = (B, S, H, P) if case.reduce_o else (B, S, R, H, P)
        out["dout"] = torch.randn(dshape, dtype=bf16)
        out["q_bias"] = torch.randn((H, R, N), dtype=f32) / 8
        out["k_bias"] = torch.randn_like(out["q_bias"])
        out["mimo_v"] = torch.randn((H, R, P), dtype=f32) / 4
        out["mimo_o"] = torch.randn((H, R, P), dtype=f32) / 4 if case.reduce_o else None
        out["z"] = torch.randn((B, S, H, P), dtype=bf16) if case.has_z else None
        out["mimo_z"] = torch.randn((H, R, P), dtype=f32) / 4 if case.has_z else None
        out["angles"] = torch.rand((B, S, H, N // 4), dtype=f32)
        out["da_cs"] = torch.randn((B, H, S), dtype=f32) / 8
        out["da_cs_rev"] = torch.randn_like(out["da_cs"]) / 8
        out["dt"] = torch.rand_like(out["da_cs"]) / 10 + 0.05
        out["trap"] = torch.randn((B, H, S), dtype=bf16)
        out["d"] = torch.randn((H,), dtype=f32) / 8 if case.has_d else None
        out["segsum"] = torch.randn((B, H, nc, C, C), dtype=f32) / 8
        if case.rd != 4:
            out["angles"] = torch.rand((B, S, H, N // case.rd), dtype=f32)
    else:
        raise ValueError(f"unknown recipe {case.recipe!r}")
    out["chunk_size"] = C
    out["rotary_dim_divisor"] = case.rd
    return out


def api_args(inputs: dict):
    """Positional argument tuple of mamba_mimo_bwd_fwd for an inputs dict."""
    return tuple(inputs[n] for n in API_ORDER) + (inputs["chunk_size"], inputs["rotary_dim_divisor"])


# ---------------------------------------------------------------- SISO forward
# Positional order of the tensor arguments of the SISO forward (mamba3_siso_fwd_kernel).
SISO_ORDER = ("q", "k", "v", "adt", "dt", "trap", "q_bias", "k_bias", "angles", "d", "z")


@dataclass(frozen=True)
class SisoCase:
    """SISO forward shape: q/k [B,S,Hq,K], v/z [B,S,H,V], angles [B,S,H,A]."""
    B: int
    S: int
    Hq: int
    H: int
    K: int
    V: int
    C: int = 64
    A: int = -1                # rotated pairs; -1 = K // 2
    dtype: str = "bf16"        # "bf16" or "fp16" for q, k, v, z
    has_z: bool = True
    has_d: bool = True
    seed: int = 123
    name: str = field(default="", compare=False)

    @property
    def width(self) -> int:
        return self.K // 2 if self.A < 0 else self.A

    def with_(self, **kw) -> "SisoCase":
        return replace(self, **kw)


# The page's usage example (fp16, Hq=2, H=4, K=64, V=96, chunk 64) and a long
# sequence in each dtype at the K=128 state size the page singles out.
SISO_CONFIGS = {
    "siso_example": SisoCase(1, 128, 2, 4, 64, 96, 64, dtype="fp16", name="siso_example"),
    "siso_s8192_k128": SisoCase(1, 8192, 16, 16, 128, 64, 64, name="siso_s8192_k128"),
    "siso_s8192_k128_fp16": SisoCase(1, 8192, 16, 16, 128, 64, 64, dtype="fp16",
                                     name="siso_s8192_k128_fp16"),
}


def make_siso_inputs(case: SisoCase):
    """Draw the SISO forward's inputs on the CPU with the distributions of the page's
    usage example: q, k, v, z ~ N(0,1) in the case's dtype; adt = -0.08 U(0,1);
    dt = 0.05 N(0,1); trap ~ N(0,1); q_bias, k_bias = 0.05 N(0,1); angles =
    0.25 U(0,1); d = 0.2 U(0,1) (numeric parameters float32). Returns a dict with
    the ``SISO_ORDER`` tensors (absent optional ones None) and ``chunk_size``."""
    B, S, Hq, H, K, V, A = case.B, case.S, case.Hq, case.H, case.K, case.V, case.width
    g = torch.Generator().manual_seed(case.seed)
    dt_ = torch.float16 if case.dtype == "fp16" else torch.bfloat16
    out = {
        "q": torch.randn((B, S, Hq, K), generator=g).to(dt_),
        "k": torch.randn((B, S, Hq, K), generator=g).to(dt_),
        "v": torch.randn((B, S, H, V), generator=g).to(dt_),
        "adt": -torch.rand((B, H, S), generator=g) * 0.08,
        "dt": torch.randn((B, H, S), generator=g) * 0.05,
        "trap": torch.randn((B, H, S), generator=g),
        "q_bias": torch.randn((H, K), generator=g) * 0.05,
        "k_bias": torch.randn((H, K), generator=g) * 0.05,
        "angles": torch.rand((B, S, H, A), generator=g) * 0.25,
        "d": torch.rand((H,), generator=g) * 0.2 if case.has_d else None,
        "z": torch.randn((B, S, H, V), generator=g).to(dt_) if case.has_z else None,
    }
    out["chunk_size"] = case.C
    return out
