"""Benchmark of the Mamba-3 MIMO backward first stage (mamba_mimo_bwd_fwd) on
one MI355X.

One step = one call of the whole operation (all kernels) on one batch of
synthetic inputs already resident in device memory. Default workload: the
pages' performance shape B=1, S=8192, H=16, G=1, N=P=64, R=4, C=16 with
reduced dout and the D and Z branches on (seeded synthetic inputs).

Several input/output buffer sets are used in turn so that the data of one
call is not still sitting in the 256 MB Infinity Cache from the previous
call: the figures are device-memory (HBM) figures.

``--op fwd`` times the layer output ``mamba_mimo_fwd`` (the forward whose
gradients the backward stage computes) on the same workload instead.

Prints progress on stderr and ONE JSON line on stdout.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "mimo_bwd_fwd ms/call + HBM GB/s at B1 S8192 H16 G1 N=P=64 R4 C16"
FWD_METRIC = "mimo_fwd (layer output) ms/call + HBM GB/s at B1 S8192 H16 G1 N=P=64 R4 C16"
PAGES_MS = 53.849475          # the pages' Ascend910_9382 median at this exact workload (context)
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0
# fp32 vector peak 157.3 TFLOP/s counts an FMA as two flops: 78.6 T fp32
# element operations per second (256 CUs x 4 SIMDs x 32 lane-ops x 2.4 GHz,
# i.e. with packed-fp32 dual issue). Without packed fp32 the issue ceiling is
# half of that, 39.3 T/s.
ALU_PEAK_TOPS = 256 * 4 * 32 * 2.4e9 / 1e12
ALU_NONPACKED_TOPS = ALU_PEAK_TOPS / 2

KERNEL_SOURCES = [ROOT / "mamba_mimo_chunked_amd" / "csrc" / n for n in ("mimo_kernels.hpp", "mimo_bwd_fwd.hip")]
TRAFFIC_FILES = {"bwd_fwd": ROOT / "profiles" / "k_main_perf_s8192_traffic.json",
                 "fwd": ROOT / "profiles" / "k_main_fwd_perf_s8192_traffic.json"}


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


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="perf_s8192", help="workload name from synth.inputs.CONFIGS")
    ap.add_argument("--sets", type=int, default=0, help="rotating buffer sets (0: enough for > 512 MB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--mode", choices=("op", "copy"), default="op",
                    help="copy: a plain device copy of known size, for counter calibration")
    ap.add_argument("--op", choices=("bwd_fwd", "fwd"), default="bwd_fwd",
                    help="fwd: time the layer output mamba_mimo_fwd instead of the backward stage")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    from mamba_mimo_chunked_amd import _lib, mamba_mimo_bwd_fwd
    from mamba_mimo_chunked_amd.api import _make_args, _make_fwd_args
    from synth.inputs import API_ORDER, CONFIGS, make_inputs

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

    case = CONFIGS[a.config]
    log(f"workload {a.config}: {case}")
    t = time.perf_counter()
    inp = make_inputs(case)
    log(f"inputs generated in {time.perf_counter() - t:.1f}s")
    fwd = a.op == "fwd"
    alg_bytes = algorithmic_bytes(case, fwd)
    alg_flops = algorithmic_flops(case, fwd)
    nsets = a.sets or max(2, math.ceil(512e6 / alg_bytes))
    B, S, H, G, R, N, P, C = case.B, case.S, case.H, case.G, case.R, case.N, case.P, case.C
    nc = case.nchunks
    sets = []
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
    from mamba_mimo_chunked_amd import fwd_workspace_size, workspace_size
    wsf = fwd_workspace_size if fwd else workspace_size
    ws_bytes = wsf(B, S, H, G, R, N, P, C, case.rd, reduce_o=case.reduce_o, has_z=case.has_z)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    L = _lib.lib()
    mk = _make_fwd_args if fwd else _make_args
    cargs = [mk(B, S, H, G, R, N, P, C, case.rd, d, out, ws, ws_bytes) for d, out in sets]
    run_call = L.mimo_fwd if fwd else L.mimo_bwd_fwd
    run_timed = L.mimo_fwd_timed if fwd else L.mimo_bwd_fwd_timed
    stream = torch.cuda.current_stream(dev).cuda_stream

    def call(i):
        st = run_call(ctypes.byref(cargs[i % nsets]), ctypes.c_void_p(stream))
        if st != 0:
            raise RuntimeError(_lib.last_error())

    log(f"{nsets} buffer sets, workspace {ws_bytes} B; warmup {a.warmup}")
    for i in range(a.warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        call(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / a.steps
    log(f"timed {a.steps} steps: {ms:.4f} ms/call")

    # per-kernel durations, HIP events recorded by the library on its stream
    hip = HipEvents()
    evs = [hip.create(_lib.TIMED_EVENTS) for _ in range(a.steps)]
    for i in range(a.steps):
        arr = (ctypes.c_void_p * _lib.TIMED_EVENTS)(*[e.value for e in evs[i]])
        st = run_timed(ctypes.byref(cargs[i % nsets]), ctypes.c_void_p(stream), arr)
        if st != 0:
            raise RuntimeError(_lib.last_error())
    torch.cuda.synchronize()
    names = ("k_agg", "k_scan", "k_main", "k_finish")
    per = {n: 0.0 for n in names}
    for e in evs:
        for j, n in enumerate(names):
            per[n] += hip.elapsed_ms(e[j], e[j + 1]) / a.steps
        hip.destroy(e)
    log("per-kernel ms: " + ", ".join(f"{n}={v:.4f}" for n, v in per.items()))

    main_ms = per["k_main"]
    alu_ops = algorithmic_alu_ops(case, fwd)
    hbm_gbps_main = alg_bytes / (main_ms * 1e-3) / 1e9
    alu_tops = alu_ops / (main_ms * 1e-3) / 1e12
    traffic = None
    tfile = TRAFFIC_FILES[a.op]
    if tfile.exists():
        rec = json.loads(tfile.read_text())
        if rec.get("source_sha256") == source_hash() and rec.get("workload") == a.config:
            traffic = rec.get("bytes_per_launch")
    # The binding roof is the one whose ideal time is longest: elementwise ALU
    # work at the fp32 vector peak versus algorithmic bytes at the HBM peak.
    t_alu = alu_ops / (ALU_PEAK_TOPS * 1e12)
    t_hbm = alg_bytes / (HBM_PEAK_GBS * 1e9)
    if t_alu >= t_hbm:
        roofline = {"bound": "alu", "achieved": round(alu_tops, 3), "peak": round(ALU_PEAK_TOPS, 2),
                    "unit": "Top/s", "frac": round(alu_tops / ALU_PEAK_TOPS, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(hbm_gbps_main, 2), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(hbm_gbps_main / HBM_PEAK_GBS, 4)}
    roofline.update({
        "traffic": traffic, "kernel": "k_main", "kernel_ms": round(main_ms, 5),
        "algorithmic_alu_ops_per_launch": alu_ops, "algorithmic_bytes_per_launch": alg_bytes,
        "hbm_frac": round(hbm_gbps_main / HBM_PEAK_GBS, 4),
        "alu_frac_nonpacked": round(alu_tops / ALU_NONPACKED_TOPS, 4),
        "mfma_frac": round(alg_flops / (main_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5)})

    cpu = None
    if not a.no_cpu:
        from oracle import o1
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        log(f"oracle CPU baseline on the whole workload ({threads} OpenMP threads)")
        t = time.perf_counter()
        (o1.run_fwd_inputs if fwd else o1.run_inputs)(inp)
        cpu_ms = (time.perf_counter() - t) * 1e3
        cpu = {"value": round(cpu_ms, 3), "unit": "ms/call", "cores": min(threads, B * H), "kind": "oracle",
               "sample": f"the whole {a.config} workload once (OpenMP over the {B * H} (batch, head) pairs)"}
        log(f"oracle: {cpu_ms:.1f} ms")

    gbps = alg_bytes / (ms * 1e-3) / 1e9
    line = {
        "metric": FWD_METRIC if fwd else METRIC,
        "value": round(ms, 5),
        "unit": "ms/call",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round(ms / PAGES_MS, 6) if a.config == "perf_s8192" and not fwd else None,
        "dtype": "bf16",
        "data": "synthetic",
        "hbm_gbps": round(gbps, 2),
        "hbm_frac": round(gbps / HBM_PEAK_GBS, 4),
        "per_kernel_ms": {k: round(v, 5) for k, v in per.items()},
        "config": {"workload": a.config, "op": a.op, "B": B, "S": S, "H": H, "G": G, "N": N, "P": P, "R": R,
                   "chunk_size": C, "rotary_dim_divisor": case.rd, "reduce_o": case.reduce_o,
                   "has_z": case.has_z, "has_d": case.has_d, "buffer_sets": nsets,
                   "algorithmic_bytes": alg_bytes, "algorithmic_flops": alg_flops},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
