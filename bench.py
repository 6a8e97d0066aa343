"""Benchmark of the Mamba-3 MIMO backward first stage (mamba_mimo_bwd_fwd) on
one MI355X.

One step = one call of the whole operation (all kernels) on one batch of
synthetic inputs already resident in device memory. Default workload: the
pages' performance shape B=1, S=8192, H=16, G=1, N=P=64, R=4, C=16 with
reduced dout and the D and Z branches on (seeded synthetic inputs).

Several input/output buffer sets are used in turn so that the data of one
call is not still sitting in the 256 MB Infinity Cache from the previous
call: the figures are device-memory (HBM) figures.

Other operations (``--op``), each on its own workload line:
  fwd           the layer output mamba_mimo_fwd (the forward whose gradients the
                backward stage computes), same workload;
  bwd_fwd_fp32  the backward stage with fp32 intermediates, same workload;
  siso          the SISO forward mamba3_siso_fwd, B=1, S=8192, H=Hq=16, K=128,
                V=64, chunk 64, bf16 (--config siso_s8192_k128_fp16 for fp16);
  bwd_bwd       the stage-2 backward mamba3_mimo_bwd_bwd on the same workload as
                the first stage, fed that stage's states and qk_dot.

Timing (the pages' protocol, NPU performance record of the operator document):
``--procs`` processes (default 3) each run ``--warmup`` calls and then
``--steps`` timed calls; an event recorded on the stream between consecutive
calls gives each call's device time. ``value`` is this process's ms per step
over its timed calls (bracketed by synchronisation); ``timing`` holds the
median, per-process medians, standard deviation and range over all processes,
and the synchronous wall time of the Python entry point with output and
workspace allocation included.

Prints progress on stderr and ONE JSON line on stdout.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import subprocess
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "mimo_bwd_fwd ms/call + HBM GB/s at B1 S8192 H16 G1 N=P=64 R4 C16"
FWD_METRIC = "mimo_fwd (layer output) ms/call + HBM GB/s at B1 S8192 H16 G1 N=P=64 R4 C16"
FP32_METRIC = "mimo_bwd_fwd_fp32 (fp32 intermediates) ms/call + HBM GB/s at B1 S8192 H16 G1 N=P=64 R4 C16"
SISO_METRIC = "mamba3_siso_fwd ms/call + HBM GB/s at B1 S8192 H=Hq=16 K128 V64 C64"
BWD2_METRIC = "mamba3_mimo_bwd_bwd (stage-2 backward) ms/call + HBM GB/s at B1 S8192 H16 G1 N=P=64 R4 C16"
MFMA_FP32_PEAK_TFLOPS = 157.3
PAGES_MS = 53.849475          # the pages' Ascend910_9382 median at this exact workload (context)
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0
# fp32 vector peak 157.3 TFLOP/s counts an FMA as two flops: 78.6 T fp32
# element operations per second (256 CUs x 4 SIMDs x 32 lane-ops x 2.4 GHz,
# i.e. with packed-fp32 dual issue). Without packed fp32 the issue ceiling is
# half of that, 39.3 T/s.
ALU_PEAK_TOPS = 256 * 4 * 32 * 2.4e9 / 1e12
ALU_NONPACKED_TOPS = ALU_PEAK_TOPS / 2

# The sources an operation's kernels and launch plan are built from (the shared kernel
# header, the host file, and the operation's own kernel header): a traffic record is
# used only while their hash is the one it was measured with.
_CSRC = ROOT / "mamba_mimo_chunked_amd" / "csrc"
_COMMON = [_CSRC / "mimo_kernels.hpp", _CSRC / "mimo_bwd_fwd.hip"]
KERNEL_SOURCES = {"bwd_fwd": _COMMON, "fwd": _COMMON,
                  "bwd_fwd_fp32": _COMMON + [_CSRC / "mimo_f32.hpp"], "siso": _COMMON + [_CSRC / "mimo_f32.hpp"],
                  "bwd_bwd": _COMMON + [_CSRC / "mimo_bwd2.hpp"]}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(c, fwd=False) -> int:
    """Bytes the operation must move at least once: every tensor its branches
    need, read or written once (q/k once although several heads share them).
    fwd: the layer output (no dout; o instead of states, qk_dot and gradients)."""
    B, S, H, G, R, N, P, C = c.B, c.S, c.H, c.G, c.R, c.N, c.P, c.C
    nc = (S + C - 1) // C
    if fwd:
        b = 2 * B * S * R * G * N * 2 + B * S * H * P * 2   # q, k, v
        if c.has_z:
            b += B * S * H * P * 2                          # z
        b += B * S * H * (N // c.rd) * 4                    # angles
        b += 3 * B * H * S * 4 + B * H * S * 2              # da_cs, da_cs_rev, dt, trap
        b += B * H * nc * C * C * 4                         # segsum
        b += 2 * H * R * N * 4 + (1 + c.reduce_o + c.has_z) * H * R * P * 4 + (H * 4 if c.has_d else 0)
        b += B * S * H * P * 2 * (1 if c.reduce_o else R)  # o
        return b
    need_y = c.reduce_o or c.has_z
    b = 2 * B * S * R * G * N * 2                       # q, k
    b += B * S * H * P * 2                              # v
    if c.reduce_o:
        b += B * S * H * P * 2                          # dout [B,S,H,P]
    elif c.has_z:
        b += B * S * R * H * P * 2                      # dout [B,S,R,H,P]
    if c.has_z:
        b += B * S * H * P * 2                          # z
    b += B * S * H * (N // c.rd) * 4                    # angles
    b += 3 * B * H * S * 4 + B * H * S * 2              # da_cs, da_cs_rev, dt, trap
    if need_y:
        b += B * H * nc * C * C * 4                     # segsum
    b += 2 * H * R * N * 4 + (1 + c.reduce_o + c.has_z) * H * R * P * 4 + (H * 4 if c.has_d else 0)
    b += B * H * nc * N * P * 2 + B * H * S * R * R * 2  # states, qk_dot
    if c.has_z:
        b += B * S * H * P * 2                          # dz
    b += (c.reduce_o + c.has_z) * B * H * R * P * 4     # dmimo_o, dmimo_z
    return b


def algorithmic_flops(c, fwd=False) -> int:
    """Multiply-adds (x2) the method needs: qk_dot, the state increment, and when
    y is needed the strictly causal pairs, the inter term and the diagonal."""
    B, S, H, R, N, P, C = c.B, c.S, c.H, c.R, c.N, c.P, c.C
    nc = (S + C - 1) // C
    f = 2 * S * R * R * N + 2 * S * R * N * P
    if fwd or c.reduce_o or c.has_z:
        pairs = nc * C * (C - 1) // 2
        f += pairs * R * R * 2 * (N + P) + 2 * S * R * N * P + 2 * S * R * R * P
    return B * H * f


def algorithmic_alu_ops(c, fwd=False) -> int:
    """Elementwise fp32 operations the bf16 contract prescribes (one per add,
    multiply, bf16 rounding, exponential, logistic or sin/cos of one element),
    excluding the contractions counted in algorithmic_flops. Per real token
    and head, with W = N/rd rotated column pairs:
      q, k bias + round            4RN      rotation of q, k (8 per pair)  16RW + 2W (cos, sin)
      K~ and kappa scale + round   4RN      PsiV                           2RP
    and, when y is needed,
      causal block scale + round   2 per strictly causal (token, rank) pair
      inter scale                  RP       y assembly and rounding        5RP
      rank-ordered diagonal        (4R + 2)RP
      gating (sigmoid, SiLU, projections, dz chain, dmimo sums)   24RP (Z) or 2RP (no Z);
    for the layer output (fwd) y is always needed and the gating is
      projection, pz, sigmoid, SiLU, gate product, rank sum  6RP (Z) or 2RP (no Z), plus P
      for the output rounding (reduced)."""
    B, S, H, R, N, P, C = c.B, c.S, c.H, c.R, c.N, c.P, c.C
    W = N // c.rd
    per_tok = 8 * R * N + 16 * R * W + 2 * W + 2 * R * P
    ops = S * per_tok
    if fwd or c.reduce_o or c.has_z:
        full, tail = S // C, S - (S // C) * C
        pairs = full * C * (C - 1) // 2 + tail * (tail - 1) // 2
        ops += 2 * pairs * R * R
        if fwd:
            gate = (6 if c.has_z else 2) * R * P + (P if c.reduce_o else 0)
        else:
            gate = (24 if c.has_z else 2) * R * P
        ops += S * (R * P + 5 * R * P + (4 * R + 2) * R * P + gate)
    return B * H * ops


def source_hash(op: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[op]:
        h.update(p.read_bytes())
    return h.hexdigest()


class HipEvents:
    """Raw HIP events (the library records them on the stream it launches on)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs.append(e)
        return evs

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")


def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def sync_api_samples(op, case, inp, dev, n, torch) -> list:
    """Synchronous wall time of n calls of the Python entry point, each allocating its
    outputs and workspace (the pages' timing boundary includes that allocation)."""
    from mamba_mimo_chunked_amd import mamba_mimo_bwd_fwd, mamba_mimo_bwd_fwd_fp32, mamba_mimo_fwd
    from synth.inputs import API_ORDER
    d = {k: (None if inp[k] is None else inp[k].to(dev)) for k in API_ORDER}
    if op == "fwd":
        fn, args = mamba_mimo_fwd, [d[k] for k in API_ORDER if k != "dout"]
    else:
        fn = mamba_mimo_bwd_fwd_fp32 if op == "bwd_fwd_fp32" else mamba_mimo_bwd_fwd
        args = [d[k] for k in API_ORDER]
    for _ in range(3):
        fn(*args, case.C, case.rd)
    torch.cuda.synchronize()
    out = []
    for _ in range(n):
        t0 = time.perf_counter()
        r = fn(*args, case.C, case.rd)
        torch.cuda.synchronize()
        out.append((time.perf_counter() - t0) * 1e3)
        del r
    return out


def bwd2_bytes(c) -> int:
    """Algorithmic bytes of the stage-2 backward: its inputs (dout, q, k, v, the caches,
    controls, segsum, angles, parameters) read once and its twelve outputs written once
    (DQ, DK, DV in bf16)."""
    B, S, H, G, R, N, P, C = c.B, c.S, c.H, c.G, c.R, c.N, c.P, c.C
    nc = (S + C - 1) // C
    W = N // c.rd
    b = B * S * H * P * 2 * (1 if c.reduce_o else R)          # dout
    b += 2 * B * S * R * G * N * 2 + B * S * H * P * 2          # q, k, v
    b += B * H * nc * N * P * 2 + B * H * S * R * R * 2         # states, qk_dot
    b += 3 * B * H * S * 4 + B * H * S * 2 + B * H * nc * C * C * 4 + B * S * H * W * 4
    b += 2 * H * R * N * 4 + (1 + c.reduce_o) * H * R * P * 4 + (H * 4 if c.has_d else 0)
    b += 2 * B * S * R * H * N * 2 + B * S * H * P * 2          # DQ, DK, DV
    b += B * H * R * P * 4 + B * S * H * W * 4 + 5 * B * H * S * 4 + B * H * nc * C * C * 4
    return b + (B * H * 4 if c.has_d else 0)


def bwd2_flops(c) -> int:
    """Multiply-adds (x2) of the stage-2 contractions: per chunk, over the strictly
    causal (token, rank) pairs, the causal block, dPhiO Psi^T and the three products
    with them (3N + 2P per pair), and the four products with a state ([C*R, N] x [N, P]:
    dPhiO S^T, Psi dS^T, kappa dS, the dS increment)."""
    B, S, H, R, N, P, C = c.B, c.S, c.H, c.R, c.N, c.P, c.C
    full, tail = S // C, S - (S // C) * C
    pairs = full * C * (C - 1) // 2 + tail * (tail - 1) // 2
    return B * H * 2 * (pairs * R * R * (3 * N + 2 * P) + 4 * S * R * N * P)


def siso_bytes(c) -> int:
    """Algorithmic bytes of the SISO forward: every input once, the output once."""
    B, S, Hq, H, K, V, A = c.B, c.S, c.Hq, c.H, c.K, c.V, c.width
    b = 2 * B * S * Hq * K * 2 + B * S * H * V * 2 * (2 if c.has_z else 1)   # q, k, v, z
    b += 3 * B * H * S * 4 + 2 * H * K * 4 + B * S * H * A * 4 + (H * 4 if c.has_d else 0)
    return b + B * S * H * V * 2                                                # out


def siso_flops(c) -> int:
    """Multiply-adds (x2) of the SISO forward (the rank-1 case of algorithmic_flops)."""
    B, S, H, K, V, C = c.B, c.S, c.H, c.K, c.V, c.C
    full, tail = S // C, S - (S // C) * C
    pairs = full * C * (C - 1) // 2 + tail * (tail - 1) // 2
    f = 2 * S * K + 2 * S * K * V + pairs * 2 * (K + V) + 2 * S * K * V + 2 * S * V
    return B * H * f


def siso_alu_ops(c) -> int:
    """Elementwise fp32 operations of the SISO forward per token and head: bias of q, k
    (2K), rotation (8A + 2A sin/cos), factor scale of k (K), the decay weights of the
    strictly causal pairs (2 per pair), the inter scale (V), y assembly (4V), and with z
    the gate (sigmoid, SiLU, product: 4V)."""
    B, S, H, K, V, C, A = c.B, c.S, c.H, c.K, c.V, c.C, c.width
    full, tail = S // C, S - (S // C) * C
    pairs = full * C * (C - 1) // 2 + tail * (tail - 1) // 2
    per_tok = 2 * K + 10 * A + K + V + 4 * V + (4 * V if c.has_z else 0)
    return B * H * (S * per_tok + 2 * pairs)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=None,
                    help="workload name (synth.inputs.CONFIGS; SISO_CONFIGS for --op siso)")
    ap.add_argument("--sets", type=int, default=0, help="rotating buffer sets (0: enough for > 512 MB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--mode", choices=("op", "copy"), default="op",
                    help="copy: a plain device copy of known size, for counter calibration")
    ap.add_argument("--op", choices=("bwd_fwd", "fwd", "bwd_fwd_fp32", "siso", "bwd_bwd"), default="bwd_fwd",
                    help="operation to time (default: the backward first stage)")
    ap.add_argument("--procs", type=int, default=3,
                    help="processes of the timing protocol (each: warm-up, then the timed calls)")
    ap.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if a.config is None:
        a.config = "siso_s8192_k128" if a.op == "siso" else "perf_s8192"

    # The other processes of the timing protocol run first, one after the other, as
    # children started before this process touches the GPU; each prints its samples.
    child_samples = []
    if not a.child and a.mode == "op":
        for k in range(1, max(1, a.procs)):
            log(f"timing process {k + 1} of {a.procs}")
            cmd = [sys.executable, str(ROOT / "bench.py"), "--child", "--op", a.op, "--config", a.config,
                   "--steps", str(a.steps), "--warmup", str(a.warmup), "--sets", str(a.sets)]
            res = subprocess.run(cmd, capture_output=True, text=True)
            sys.stderr.write(res.stderr)
            if res.returncode != 0:
                log(f"timing process {k + 1} failed with status {res.returncode}")
                sys.exit(res.returncode)
            child_samples.append(json.loads(res.stdout.strip().splitlines()[-1]))

    import torch
    from mamba_mimo_chunked_amd import _lib
    from mamba_mimo_chunked_amd.api import _make_args, _make_bwd2_args, _make_fwd_args, _make_siso_args
    from synth.inputs import API_ORDER, CONFIGS, SISO_CONFIGS, SISO_ORDER, make_inputs, make_siso_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if a.mode == "copy":
        n = 256 << 20                                          # 256 Mi fp32 = 1 GiB each way
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(a.warmup):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(a.steps):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / a.steps
        print(json.dumps({"mode": "copy", "bytes_read": 4 * n, "bytes_written": 4 * n, "ms": ms,
                          "GBps": 8 * n / ms / 1e6}))
        return

    op = a.op
    siso_op = op == "siso"
    case = SISO_CONFIGS[a.config] if siso_op else CONFIGS[a.config]
    log(f"op {op}, workload {a.config}: {case}")
    t = time.perf_counter()
    inp = make_siso_inputs(case) if siso_op else make_inputs(case)
    log(f"inputs generated in {time.perf_counter() - t:.1f}s")
    L = _lib.lib()
    bwd2_op = op == "bwd_bwd"
    fwd = op == "fwd"
    if siso_op:
        alg_bytes, alg_flops, alu_ops = siso_bytes(case), siso_flops(case), siso_alu_ops(case)
        mfma_peak, mfma_unit_dtype = MFMA_FP32_PEAK_TFLOPS, "fp32"
    elif bwd2_op:
        alg_bytes, alg_flops, alu_ops = bwd2_bytes(case), bwd2_flops(case), 0
        mfma_peak, mfma_unit_dtype = MFMA_FP32_PEAK_TFLOPS, "fp32"
    else:
        alg_bytes, alg_flops = algorithmic_bytes(case, fwd), algorithmic_flops(case, fwd)
        alu_ops = algorithmic_alu_ops(case, fwd)
        fp32 = op == "bwd_fwd_fp32"
        mfma_peak = MFMA_FP32_PEAK_TFLOPS if fp32 else MFMA_BF16_PEAK_TFLOPS
        mfma_unit_dtype = "fp32" if fp32 else "bf16"
    nsets = a.sets or max(2, math.ceil(512e6 / alg_bytes))

    # ---- buffer sets and argument structs
    sets = []
    if siso_op:
        B, S, H, V = case.B, case.S, case.H, case.V
        dims = (case.B, case.S, case.Hq, case.H, case.K, case.V, case.width, case.C)
        odt = torch.float16 if case.dtype == "fp16" else torch.bfloat16
        for _ in range(nsets):
            d = {n: (None if inp[n] is None else inp[n].to(dev)) for n in SISO_ORDER}
            sets.append((d, torch.empty((B, S, H, V), device=dev, dtype=odt)))
        probe = _make_siso_args(dims, odt, sets[0][0], sets[0][1])
        nbytes = ctypes.c_size_t(0)
        st = L.mimo_siso_fwd_workspace_size(ctypes.byref(probe), ctypes.byref(nbytes))
        if st != 0:
            raise RuntimeError(_lib.last_error())
        ws_bytes = int(nbytes.value)
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        cargs = [_make_siso_args(dims, odt, d, o, ws, ws_bytes) for d, o in sets]
        run_call, run_timed = L.mimo_siso_fwd, L.mimo_siso_fwd_timed
    elif bwd2_op:
        from mamba_mimo_chunked_amd import mamba_mimo_bwd_fwd
        B, S, H, G, R, N, P, C = case.B, case.S, case.H, case.G, case.R, case.N, case.P, case.C
        nc = case.nchunks
        W = N // case.rd
        d0 = {n: (None if inp[n] is None else inp[n].to(dev)) for n in API_ORDER}
        st1 = mamba_mimo_bwd_fwd(*[d0[n] for n in API_ORDER], C, case.rd)   # the caches
        torch.cuda.synchronize()
        caches = (st1.states, st1.qk_dot)
        f32 = torch.float32
        for _ in range(nsets):
            d = {n: (None if inp[n] is None else inp[n].to(dev)) for n in API_ORDER}
            d["states"], d["qk_dot"] = caches[0].clone(), caches[1].clone()
            outs = {"DQ": torch.empty((B, S * R, H, N), dtype=torch.bfloat16, device=dev),
                    "DK": torch.empty((B, S * R, H, N), dtype=torch.bfloat16, device=dev),
                    "DV": torch.empty((B, S, H, P), dtype=torch.bfloat16, device=dev),
                    "DMIMO_V": torch.empty((B, H, R, P), dtype=f32, device=dev),
                    "DANGLES": torch.empty((B, S, H, W), dtype=f32, device=dev),
                    "DSSDA": torch.empty((B, H, nc, C, C), dtype=f32, device=dev),
                    "DD": torch.empty((B, H), dtype=f32, device=dev) if case.has_d else None}
            for key in ("DFACTOR", "DGAMMA", "DDA", "DDA_CS_REV", "DDA_CS"):
                outs[key] = torch.empty((B, H, S), dtype=f32, device=dev)
            sets.append((d, outs))
        dims = (B, S, H, G, R, N, P)
        probe = _make_bwd2_args(dims, C, case.rd, _lib.DTYPE_BF16, _lib.DTYPE_BF16, sets[0][0], sets[0][1])
        nbytes = ctypes.c_size_t(0)
        st = L.mimo_bwd_bwd_workspace_size(ctypes.byref(probe), ctypes.byref(nbytes))
        if st != 0:
            raise RuntimeError(_lib.last_error())
        ws_bytes = int(nbytes.value)
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        cargs = [_make_bwd2_args(dims, C, case.rd, _lib.DTYPE_BF16, _lib.DTYPE_BF16, d, o, ws, ws_bytes)
                 for d, o in sets]
        run_call, run_timed = L.mimo_bwd_bwd, L.mimo_bwd_bwd_timed
    else:
        B, S, H, G, R, N, P, C = case.B, case.S, case.H, case.G, case.R, case.N, case.P, case.C
        nc = case.nchunks
        for _ in range(nsets):
            d = {n: (None if inp[n] is None or (fwd and n == "dout") else inp[n].to(dev)) for n in API_ORDER}
            if fwd:
                oshape = (B, S, H, P) if case.reduce_o else (B, S, R, H, P)
                sets.append((d, torch.empty(oshape, device=dev, dtype=torch.bfloat16)))
                continue
            out = {
                "dmimo_o": torch.empty((B, H, R, P), device=dev) if case.reduce_o else None,
                "states": torch.empty((B, H, nc, N, P), device=dev, dtype=torch.bfloat16),
                "dz": torch.empty((B, S, H, P), device=dev, dtype=torch.bfloat16) if case.has_z else None,
                "dmimo_z": torch.empty((B, H, R, P), device=dev) if case.has_z else None,
                "qk_dot": torch.empty((B, H, S, R, R), device=dev, dtype=torch.bfloat16),
            }
            sets.append((d, out))
        fn = {"bwd_fwd": "mimo_bwd_fwd", "fwd": "mimo_fwd", "bwd_fwd_fp32": "mimo_bwd_fwd_f32"}[op]
        mk = _make_fwd_args if fwd else _make_args
        probe = mk(B, S, H, G, R, N, P, C, case.rd, sets[0][0], sets[0][1])
        nbytes = ctypes.c_size_t(0)
        st = getattr(L, fn + "_workspace_size")(ctypes.byref(probe), ctypes.byref(nbytes))
        if st != 0:
            raise RuntimeError(_lib.last_error())
        ws_bytes = int(nbytes.value)
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        cargs = [mk(B, S, H, G, R, N, P, C, case.rd, d, out, ws, ws_bytes) for d, out in sets]
        run_call, run_timed = getattr(L, fn), getattr(L, fn + "_timed")
    stream = torch.cuda.current_stream(dev).cuda_stream

    def call(i):
        st = run_call(ctypes.byref(cargs[i % nsets]), ctypes.c_void_p(stream))
        if st != 0:
            raise RuntimeError(_lib.last_error())

    log(f"{nsets} buffer sets, workspace {ws_bytes} B; warmup {a.warmup}")
    hip = HipEvents()
    marks = hip.create(a.steps + 1)
    for i in range(a.warmup):
        call(i)
    torch.cuda.synchronize()
    # K timed calls bracketed by synchronisation; an event on the stream between
    # consecutive calls gives each call's device time
    t0 = time.perf_counter()
    hip.record(marks[0], stream)
    for i in range(a.steps):
        call(a.warmup + i)
        hip.record(marks[i + 1], stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / a.steps
    samples = [hip.elapsed_ms(marks[i], marks[i + 1]) for i in range(a.steps)]
    hip.destroy(marks)
    log(f"timed {a.steps} steps: {ms:.4f} ms/call (median call {statistics.median(samples):.4f} ms)")
    api_samples = sync_api_samples(op, case, inp, dev, a.steps, torch) if not (siso_op or bwd2_op) else []
    if a.child:
        print(json.dumps({"samples_ms": samples, "api_samples_ms": api_samples, "ms_per_step": ms}), flush=True)
        return

    # per-kernel durations, HIP events recorded by the library on its stream
    evs = [hip.create(_lib.TIMED_EVENTS) for _ in range(a.steps)]
    for i in range(a.steps):
        arr = (ctypes.c_void_p * _lib.TIMED_EVENTS)(*[e.value for e in evs[i]])
        st = run_timed(ctypes.byref(cargs[i % nsets]), ctypes.c_void_p(stream), arr)
        if st != 0:
            raise RuntimeError(_lib.last_error())
    torch.cuda.synchronize()
    f32_names = op in ("bwd_fwd_fp32", "siso")
    names = ("k_agg", "k_scan", "k_main", "k_finish")
    if f32_names:
        names = ("k_chunk32_agg", "k_scan", "k_chunk32_main", "k_finish")
    if bwd2_op:
        names = ("k_agg2", "k_scan_rev", "k_main2", "k_finish2")
    per = {n: 0.0 for n in names}
    for e in evs:
        for j, n in enumerate(names):
            per[n] += hip.elapsed_ms(e[j], e[j + 1]) / a.steps
        hip.destroy(e)
    log("per-kernel ms: " + ", ".join(f"{n}={v:.4f}" for n, v in per.items()))

    main_name = names[2]
    main_ms = per[main_name]
    all_samples = [samples] + [c["samples_ms"] for c in child_samples]
    flat = [x for ss in all_samples for x in ss]
    call_ms = statistics.median(flat)
    hbm_gbps_main = alg_bytes / (main_ms * 1e-3) / 1e9
    alu_tops = alu_ops / (main_ms * 1e-3) / 1e12
    mfma_tflops = alg_flops / (main_ms * 1e-3) / 1e12
    traffic, traffic_call, per_kernel_traffic = None, None, None
    tfile = ROOT / "profiles" / f"traffic_{op}_{a.config}.json"
    if tfile.exists():
        rec = json.loads(tfile.read_text())
        if rec.get("source_sha256") == source_hash(op) and rec.get("workload") == a.config:
            traffic = rec.get("bytes_per_launch")
            per_kernel_traffic = rec.get("per_kernel_bytes")
            if per_kernel_traffic:
                traffic_call = sum(per_kernel_traffic.values())
    # The binding roof: HBM (algorithmic bytes at 8 TB/s) or the matrix units at the
    # dtype the contractions run in, whichever has the longer ideal time. The
    # elementwise ALU work of the bf16 contract is reported beside it against the
    # issue ceiling of non-packed fp32 (packed fp32 is not used).
    roofs = {
        "hbm": (alg_bytes / (HBM_PEAK_GBS * 1e9), hbm_gbps_main, HBM_PEAK_GBS, "GB/s"),
        "mfma": (alg_flops / (mfma_peak * 1e12), mfma_tflops, mfma_peak, "TFLOP/s"),
    }
    bound = max(roofs, key=lambda k: roofs[k][0])
    _, achieved, peak, unit = roofs[bound]
    roofline = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic}
    roofline.update({
        "kernel": main_name, "kernel_ms": round(main_ms, 5),
        "algorithmic_bytes_per_launch": alg_bytes, "algorithmic_flops_per_launch": alg_flops,
        "mfma_dtype": mfma_unit_dtype,
        "hbm_frac": round(hbm_gbps_main / HBM_PEAK_GBS, 4),
        "mfma_frac": round(mfma_tflops / mfma_peak, 5),
        "call_ms": round(call_ms, 5),
        "call_hbm_frac": round(alg_bytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "traffic_call": traffic_call,
        "traffic_call_ratio": None if traffic_call is None else round(traffic_call / alg_bytes, 3),
        "traffic_per_kernel": per_kernel_traffic})
    if alu_ops:
        roofline["alu"] = {"ops_per_launch": alu_ops, "achieved_tops": round(alu_tops, 3),
                           "peak_tops_nonpacked": round(ALU_NONPACKED_TOPS, 2),
                           "frac_nonpacked": round(alu_tops / ALU_NONPACKED_TOPS, 4)}

    procs = len(all_samples)
    timing = {
        "protocol": (f"{procs} processes x ({a.warmup} warm-up + {a.steps} timed calls); each call's device "
                     f"time from HIP events on its stream; inputs resident, outputs preallocated"),
        "median_ms": round(call_ms, 5),
        "process_medians_ms": [round(statistics.median(ss), 5) for ss in all_samples],
        "stdev_ms": round(statistics.stdev(flat), 5) if len(flat) > 1 else 0.0,
        "min_ms": round(min(flat), 5), "max_ms": round(max(flat), 5), "samples": len(flat),
    }
    api_all = [api_samples] + [c["api_samples_ms"] for c in child_samples]
    api_flat = [x for ss in api_all for x in ss]
    if api_flat:
        timing["sync_api_median_ms"] = round(statistics.median(api_flat), 5)
        timing["sync_api_process_medians_ms"] = [round(statistics.median(ss), 5) for ss in api_all if ss]
        timing["sync_api_note"] = ("synchronous wall time of the Python entry point per call: output and "
                                   "workspace allocation, argument checks, launch, completion")

    cpu = None
    if not a.no_cpu:
        from oracle import o1, siso
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        log("oracle CPU baseline " + ("on two sampled heads" if bwd2_op else f"on the whole workload ({threads} OpenMP threads)"))
        t = time.perf_counter()
        sample = f"the whole {a.config} workload once (OpenMP over the {case.B * case.H} (batch, head) pairs)"
        scale = 1.0
        if siso_op:
            siso.run(*[inp[n] for n in SISO_ORDER], chunk_size=case.C)
        elif bwd2_op:
            from oracle import bwd2
            heads = (0, case.H // 2)
            for h in heads:
                sl = o1.slice_heads(inp, 0, h)
                bwd2.run_inputs(sl, caches[0][:, h:h + 1].cpu(), caches[1][:, h:h + 1].cpu())
            scale = case.B * case.H / len(heads)
            sample = (f"{len(heads)} of the {case.B * case.H} (batch, head) pairs of {a.config} (float64 autograd, "
                      f"one thread per op), scaled by {scale:g} to the whole workload")
        elif op == "fwd":
            o1.run_fwd_inputs(inp)
        else:
            o1.run_inputs(inp, fp32=op == "bwd_fwd_fp32")
        cpu_ms = (time.perf_counter() - t) * 1e3 * scale
        cores = torch.get_num_threads() if bwd2_op else min(threads, case.B * case.H)
        cpu = {"value": round(cpu_ms, 3), "unit": "ms/call", "cores": cores, "kind": "oracle", "sample": sample,
               "cpu_model": cpu_model(), "host_threads": os.cpu_count()}
        log(f"oracle: {cpu_ms:.1f} ms")
        if op in ("bwd_fwd", "fwd", "bwd_fwd_fp32"):
            # one (batch, head) pair runs on one thread; scaled to the workload
            sl = o1.slice_heads(inp, 0, 0)
            t = time.perf_counter()
            if op == "fwd":
                o1.run_fwd_inputs(sl)
            else:
                o1.run_inputs(sl, fp32=op == "bwd_fwd_fp32")
            one = (time.perf_counter() - t) * 1e3
            cpu["single_thread"] = {"value": round(one * case.B * case.H, 3), "unit": "ms/call",
                                    "sample": f"(batch 0, head 0) on one thread, scaled by {case.B * case.H}"}
            log(f"oracle, one thread: {one:.1f} ms per head")

    gbps = alg_bytes / (ms * 1e-3) / 1e9
    metric = {"bwd_fwd": METRIC, "fwd": FWD_METRIC, "bwd_fwd_fp32": FP32_METRIC, "siso": SISO_METRIC,
              "bwd_bwd": BWD2_METRIC}[op]
    if not siso_op and (case.B, case.S, case.H, case.G, case.N, case.P, case.R, case.C) != (1, 8192, 16, 1, 64, 64, 4, 16):
        # another workload: the same metric, named with that workload's shape
        metric = metric.split(" at ")[0] + (f" at B{case.B} S{case.S} H{case.H} G{case.G} N{case.N} P{case.P} "
                                            f"R{case.R} C{case.C}")
    if siso_op:
        config = {"workload": a.config, "op": op, "B": case.B, "S": case.S, "Hq": case.Hq, "H": case.H,
                  "K": case.K, "V": case.V, "A": case.width, "chunk_size": case.C, "dtype": case.dtype,
                  "has_z": case.has_z, "has_d": case.has_d, "buffer_sets": nsets,
                  "algorithmic_bytes": alg_bytes, "algorithmic_flops": alg_flops}
        dtype = case.dtype + " in/out, f32 compute"
    else:
        config = {"workload": a.config, "op": op, "B": B, "S": S, "H": H, "G": G, "N": N, "P": P, "R": R,
                  "chunk_size": C, "rotary_dim_divisor": case.rd, "reduce_o": case.reduce_o,
                  "has_z": case.has_z, "has_d": case.has_d, "buffer_sets": nsets,
                  "algorithmic_bytes": alg_bytes, "algorithmic_flops": alg_flops}
        dtype = "f32" if op in ("bwd_fwd_fp32", "bwd_bwd") else "bf16"
    line = {
        "metric": metric,
        "value": round(ms, 5),
        "unit": "ms/call",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round(ms / PAGES_MS, 6) if a.config == "perf_s8192" and op == "bwd_fwd" else None,
        "dtype": dtype,
        "data": "synthetic",
        "hbm_gbps": round(gbps, 2),
        "hbm_frac": round(gbps / HBM_PEAK_GBS, 4),
        "per_kernel_ms": {k: round(v, 5) for k, v in per.items()},
        "timing": timing,
        "config": config,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
