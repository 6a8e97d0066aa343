"""O4 -- a second, independently written contract oracle, in chunk-matrix form.

TEST INFRASTRUCTURE ONLY: the tests may import it; the product path never does.
It shares no code with O1 (``o1_contract.c``) or with the HIP library.

Source of the method: the Triton-Ascend mamba_mimo_bwd_fwd pull request page,
"BF16-boundary PyTorch reference" section, read as a list of formulas:

1. q0 = bf(q + bf(q_bias)), k0 likewise; qk_dot[t,r,r'] = bf(q0[t,r] . k0[t,r']).
2. Partial rotate-half by the angles: columns [0, W) pair with [N/2, N/2 + W);
   each rotated value is bf(cos*a - sin*e) or bf(sin*a + cos*e), with every
   product its own fp32 operation.
3. Psi = bf(v * bf(mimo_v)); gamma_t = bf(dt_t) * sigmoid(trap_t) (fp32);
   beta_t = bf(bf(dt_{t+1}) * sigmoid(-trap_{t+1})), zero at the last token;
   factor = bf(gamma + beta); Kt = bf(k_rot * factor); kappa = bf(Kt * exp(da_cs_rev)).
4. Per chunk c from the fp32 entry state S_c: states[c] = bf(S_c);
   inter = (Q_c bf(S_c)) * exp(da_cs); A = bf((Q_c Kt_c^T) * exp(segsum)) on
   strictly earlier tokens, zero elsewhere; intra = A Psi_c; the diagonal is the
   rank-ordered chain acc <- bf(acc + bf(qk_dot * Psi)), then bf(acc * gamma);
   y = bf(((inter + intra) + diag) + d * Psi);
   S_{c+1} = S_c * exp(da_cs[last real token]) + kappa_c^T Psi_c.
5. Gating with pz = z * mimo_z (mimo_z unrounded): reduced dout gives
   dmimo_o = sum_t y * silu(pz) * dout (or y * dout without z) and
   G = bf(bf(dout * bf(mimo_o)) * y); per-rank dout gives G = bf(dout * y);
   gz = G * sigmoid(pz) * (1 + pz * sigmoid(-pz)); dz is the rank-ordered chain
   a <- bf(a + gz * mimo_z); dmimo_z = sum_t gz * z.

How this differs from O1 on purpose, so that the two are independent checks of
the same reading:

* whole-sequence numpy arrays per (batch, head) instead of token-by-token
  loops; the chunk's rows are rank-major (row r*cl + t) instead of token-major;
* the bf16 rounding is torch's float32 -> bfloat16 conversion (a library
  routine) instead of O1's bit-level rounding;
* fp32 operations are numpy float32 operations; exponentials, logistic
  functions, sines and cosines are taken in float64 and rounded to float32;
  every contraction (dot products, matrix products, sums over tokens)
  accumulates in float64 and is rounded to float32 once, which fixes no
  summation order beyond what the page fixes (it fixes none).

``fp32=True`` gives the same page's FP32 reference instead: no intermediate
bf16 rounding (states, qk_dot and dz are still bf16 outputs), and the
look-ahead weight written as dt[t+1] * (1 - sigmoid(trap[t+1])).
"""

from __future__ import annotations

import numpy as np
import torch

F32 = np.float32


def _bf(x) -> np.ndarray:
    """bf16 round-to-nearest-even of float32 values, returned as float32."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=F32)))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _f(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(F32)


def _np(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _exp(x):
    return _f(np.exp(np.asarray(x, np.float64)))


def _sig(x):
    return _f(1.0 / (1.0 + np.exp(-np.asarray(x, np.float64))))


def _mm(a, b):
    """fp32 result of a float64-accumulated matrix product."""
    return _f(np.asarray(a, np.float64) @ np.asarray(b, np.float64))


class _Head:
    """Everything the chunk walk of one (batch, head) needs, over the whole sequence."""

    def __init__(self, inp, b, h, C, W, bfi, fp32):
        q, k, v = inp["q"], inp["k"], inp["v"]
        _, S, R, G, N = q.shape
        H, P = v.shape[2], v.shape[3]
        g = h // (H // G)
        M = N // 2
        # step 1: bias, bf16, same-token rank-by-rank dots
        q0 = bfi(_f(q[b, :, :, g, :]) + bfi(_f(inp["q_bias"][h]))[None])    # [S,R,N]
        k0 = bfi(_f(k[b, :, :, g, :]) + bfi(_f(inp["k_bias"][h]))[None])
        dots = _f(np.einsum("trn,tsn->trs", q0.astype(np.float64), k0.astype(np.float64)))
        self.qk_out = _bf(dots)          # the output is bf16 in every mode
        self.qk = bfi(dots)              # the value the diagonal uses
        # step 2: rotation of the W column pairs
        ang = np.asarray(inp["angles"][b, :, h, :], np.float64)              # [S,W]
        cs, sn = _f(np.cos(ang))[:, None, :], _f(np.sin(ang))[:, None, :]

        def rot(x):
            y = x.copy()
            a, e = x[..., :W], x[..., M:M + W]
            y[..., :W] = bfi((cs * a) - (sn * e))
            y[..., M:M + W] = bfi((sn * a) + (cs * e))
            return y

        self.qr = rot(q0)
        kr = rot(k0)
        # step 3: Psi, discretisation, Kt, kappa
        self.psi = bfi(_f(v[b, :, h, :])[:, None, :] * bfi(_f(inp["mimo_v"][h]))[None])   # [S,R,P]
        dt = _f(inp["dt"][b, h])
        trap = _f(inp["trap"][b, h])
        self.gamma = bfi(dt) * _sig(trap)
        beta = np.zeros(S, F32)
        if S > 1:
            # the FP32 reference writes the look-ahead weight as 1 - sigmoid(trap)
            w = (F32(1.0) - _sig(trap[1:])) if fp32 else _sig(-trap[1:].astype(np.float64))
            beta[:-1] = bfi(bfi(dt[1:]) * w)
        factor = bfi(self.gamma + beta)
        self.kt = bfi(kr * factor[:, None, None])
        self.kap = bfi(self.kt * _exp(inp["da_cs_rev"][b, h])[:, None, None])
        self.da_cs = inp["da_cs"][b, h]
        self.ecs = _exp(self.da_cs)
        self.seg = inp["segsum"][b, h]                                       # [nc,C,C] float64
        self.d = None if inp["d"] is None else F32(inp["d"][h])
        self.S, self.R, self.N, self.P, self.C = S, R, N, P, C


def _ident(x):
    return np.asarray(x, dtype=F32)


def _chunk_walk(hd: _Head, bfi):
    """Step 4 over every chunk: the bf16 entry states and y [S,R,P]."""
    S, R, N, P, C = hd.S, hd.R, hd.N, hd.P, hd.C
    nc = (S + C - 1) // C
    state = np.zeros((N, P), F32)
    states = np.zeros((nc, N, P), F32)
    y = np.zeros((S, R, P), F32)
    for c in range(nc):
        t0, t1 = c * C, min(S, (c + 1) * C)
        cl = t1 - t0
        states[c] = _bf(state)
        # rank-major rows: row = r * cl + t
        def rows(x):
            return np.ascontiguousarray(np.swapaxes(x[t0:t1], 0, 1)).reshape(R * cl, -1)
        Q, Kt, Kap, Psi = rows(hd.qr), rows(hd.kt), rows(hd.kap), rows(hd.psi)
        tok = np.tile(np.arange(cl), R)                                   # token of each row
        inter = _mm(Q, bfi(state)) * hd.ecs[t0:t1][tok][:, None]
        es = _exp(hd.seg[c][:cl, :cl])                                    # [cl,cl]
        strict = tok[:, None] > tok[None, :]
        # the strict mask is a selection: entries on or above the diagonal are never used
        A = bfi(np.where(strict, _mm(Q, Kt.T) * es[tok[:, None], tok[None, :]], F32(0)))
        intra = _mm(A, Psi)
        # rank-ordered diagonal chain, all tokens of the chunk at once: [cl, R(out), P]
        qk, psi = hd.qk[t0:t1], hd.psi[t0:t1]
        acc = np.zeros((cl, R, P), F32)
        for r2 in range(R):
            prod = bfi(qk[:, :, r2][:, :, None] * psi[:, r2, :][:, None, :])
            acc = bfi(acc + prod)
        diag = bfi(acc * hd.gamma[t0:t1][:, None, None])
        diag_rows = np.swapaxes(diag, 0, 1).reshape(R * cl, P)
        out = (inter + intra) + diag_rows
        if hd.d is not None:
            out = out + hd.d * Psi
        y[t0:t1] = np.swapaxes(bfi(out).reshape(R, cl, P), 0, 1)
        dl = _exp(hd.da_cs[t1 - 1])                                       # last real token
        state = (state * dl) + _mm(Kap.T, Psi)
    return states, y


def run_inputs(inp: dict, *, fp32: bool = False):
    """O4 on a ``synth.inputs.make_inputs`` dict. Returns float64 arrays
    (dmimo_o, states, dz, dmimo_z, qk_dot); inactive outputs are None."""
    a = {n: _np(inp[n]) for n in ("dout", "q", "k", "v", "q_bias", "k_bias", "mimo_v", "mimo_o",
                                   "z", "mimo_z", "angles", "da_cs", "da_cs_rev", "dt", "trap",
                                   "d", "segsum")}
    C = int(inp["chunk_size"])
    B, S, R, G, N = a["q"].shape
    H, P = a["v"].shape[2], a["v"].shape[3]
    W = a["angles"].shape[-1]
    nc = (S + C - 1) // C
    bfi = _ident if fp32 else _bf
    reduce_o, has_z = a["mimo_o"] is not None, a["z"] is not None
    dmimo_o = np.zeros((B, H, R, P)) if reduce_o else None
    dmimo_z = np.zeros((B, H, R, P)) if has_z else None
    dz = np.zeros((B, S, H, P)) if has_z else None
    states = np.zeros((B, H, nc, N, P))
    qk_dot = np.zeros((B, H, S, R, R))
    for b in range(B):
        for h in range(H):
            hd = _Head(a, b, h, C, W, bfi, fp32)
            st, y = _chunk_walk(hd, bfi)
            states[b, h] = st
            qk_dot[b, h] = hd.qk_out
            _gate(a, b, h, y, bfi, dmimo_o, dz, dmimo_z)
    return dmimo_o, states, dz, dmimo_z, qk_dot


def _gate(a, b, h, y, bfi, dmimo_o, dz, dmimo_z):
    """Step 5 for one (batch, head); y is [S,R,P]."""
    S, R, P = y.shape
    reduce_o, has_z = a["mimo_o"] is not None, a["z"] is not None
    if has_z:
        zf = _f(a["z"][b, :, h, :])[:, None, :]                          # [S,1,P]
        pz = zf * _f(a["mimo_z"][h])[None]                               # [S,R,P]
        sg = _sig(pz)
    if reduce_o:
        dv = _f(a["dout"][b, :, h, :])[:, None, :]
        term = ((y * (pz * sg)) * dv) if has_z else (y * dv)
        dmimo_o[b, h] = _f(term.astype(np.float64).sum(axis=0))
        if has_z:
            G = bfi(bfi(dv * bfi(_f(a["mimo_o"][h]))[None]) * y)
    elif has_z:
        G = bfi(_f(a["dout"][b, :, :, h, :]) * y)                       # per-rank dout [S,R,P]
    if has_z:
        gz = (G * sg) * (F32(1.0) + pz * _sig(-pz.astype(np.float64)))
        acc = np.zeros((S, P), F32)
        for r in range(R):
            acc = bfi(acc + gz[:, r, :] * _f(a["mimo_z"][h, r])[None])
        dz[b, :, h, :] = _bf(acc)
        dmimo_z[b, h] = _f((gz * zf).astype(np.float64).sum(axis=0))


def run_fwd_inputs(inp: dict, *, fp32: bool = False):
    """Layer output o of the same chunk walk: reduced (mimo_o given)
    o[b,t,h,p] = bf(sum_r in rank order (y * bf(mimo_o)) * silu(pz)), otherwise
    o[b,t,r,h,p] = bf(y * silu(pz)); silu(pz) = pz * sigmoid(pz), left out without z."""
    a = {n: _np(inp[n]) for n in ("q", "k", "v", "q_bias", "k_bias", "mimo_v", "mimo_o", "z",
                                   "mimo_z", "angles", "da_cs", "da_cs_rev", "dt", "trap", "d",
                                   "segsum")}
    C = int(inp["chunk_size"])
    B, S, R, G, N = a["q"].shape
    H, P = a["v"].shape[2], a["v"].shape[3]
    W = a["angles"].shape[-1]
    bfi = _ident if fp32 else _bf
    reduce_o, has_z = a["mimo_o"] is not None, a["z"] is not None
    o = np.zeros((B, S, H, P)) if reduce_o else np.zeros((B, S, R, H, P))
    for b in range(B):
        for h in range(H):
            hd = _Head(a, b, h, C, W, bfi, fp32)
            _, y = _chunk_walk(hd, bfi)
            val = y
            if reduce_o:
                val = val * bfi(_f(a["mimo_o"][h]))[None]
            if has_z:
                pz = _f(a["z"][b, :, h, :])[:, None, :] * _f(a["mimo_z"][h])[None]
                val = val * (pz * _sig(pz))
            if reduce_o:
                acc = np.zeros((S, P), F32)
                for r in range(R):
                    acc = acc + val[:, r, :]
                o[b, :, h, :] = _bf(acc)
            else:
                o[b, :, :, h, :] = _bf(val)
    return o
