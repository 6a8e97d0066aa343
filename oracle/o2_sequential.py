"""O2 -- exact, unchunked, token-by-token recurrence (float64, no rounding).

TEST INFRASTRUCTURE ONLY (tests, smoke check and benchmark CPU leg).

This is the MIMO state-space recurrence that the chunked method of the
Triton-Ascend mamba_mimo_bwd_fwd page ("BF16-boundary PyTorch reference")
evaluates chunk by chunk, written one token at a time, with the stage-2
page's statement of the state semantics ("states[c] is the forward state
before chunk c"; "state_out = state_in * exp(da_cs_sum) + K_state^T PsiV").

Per (batch b, head h), with g = h // (H/G) and the per-token log decay da:

  q0[t,r] = q[b,t,r,g] + q_bias[h,r]         k0 likewise
  qk[t,r,r'] = q0[t,r] . k0[t,r']            (same-token rank-by-rank dot)
  qh, kh = partial rotate-half of q0, k0 by angles[b,t,h]
  psi[t,r] = v[b,t,h] * mimo_v[h,r]
  gamma_t = dt_t * sigmoid(trap_t);  beta_t = dt_{t+1} * sigmoid(-trap_{t+1}) (0 at t = S-1)
  kt[t,r] = kh[t,r] * (gamma_t + beta_t)
  h_{-1} = 0;  states[c] = h_{cC-1}  (the state before token cC)
  u_t = exp(da_t) h_{t-1}
  y[t,r] = qh[t,r] . u_t + gamma_t sum_r' qk[t,r,r'] psi[t,r'] + d_h psi[t,r]
  h_t = u_t + sum_r kt[t,r]^T psi[t,r]

Gating, with pz = z * mimo_z, silu(x) = x sigmoid(x):
  reduced dout:  dmimo_o = sum_t y silu(pz) dout   (y dout without z)
                 G = dout mimo_o y
  non-reduced:   G = dout[b,t,r,h] y
  gz = G sigmoid(pz) (1 + pz sigmoid(-pz));  dz = sum_r gz mimo_z;  dmimo_z = sum_t gz z
"""

from __future__ import annotations

import numpy as np
import torch


def _np(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def _rot(x, th):
    """Partial rotate-half of the last axis: columns [0,W) pair with [N/2, N/2+W),
    W = the angles' last axis."""
    N = x.shape[-1]
    W, M = th.shape[-1], N // 2
    c, s = np.cos(th), np.sin(th)       # [..., W]
    out = x.copy()
    a, e = x[..., :W], x[..., M:M + W]
    out[..., :W] = c * a - s * e
    out[..., M:M + W] = s * a + c * e
    return out


def run(dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da, dt, trap, d,
        chunk_size, rotary_dim_divisor=4):
    """Return float64 (dmimo_o, states, dz, dmimo_z, qk_dot, y) from the recurrence."""
    q, k, v = _np(q), _np(k), _np(v)
    B, S, R, G, N = q.shape
    H, P = v.shape[2:]
    C = int(chunk_size)
    nc = (S + C - 1) // C
    rep = H // G
    qb, kb, mv = _np(q_bias), _np(k_bias), _np(mimo_v)
    ang, da, dt, trap = _np(angles), _np(da), _np(dt), _np(trap)
    dout = _np(dout)
    reduce_o, has_z = mimo_o is not None, z is not None
    mo, zz, mz, dd = _np(mimo_o), _np(z), _np(mimo_z), _np(d)

    heads_g = np.arange(H) // rep
    hstate = np.zeros((B, H, N, P))
    states = np.zeros((B, H, nc, N, P))
    qk_dot = np.zeros((B, H, S, R, R))
    y = np.zeros((B, H, S, R, P))
    for t in range(S):
        q0 = q[:, t][:, :, heads_g].transpose(0, 2, 1, 3) + qb[None]      # [B,H,R,N]
        k0 = k[:, t][:, :, heads_g].transpose(0, 2, 1, 3) + kb[None]
        qk = np.einsum("bhrn,bhsn->bhrs", q0, k0)
        qk_dot[:, :, t] = qk
        th = ang[:, t][:, :, None, :]                                       # [B,H,1,W]
        qh = _rot(q0, th)
        kh = _rot(k0, th)
        psi = v[:, t][:, :, None, :] * mv[None]                            # [B,H,R,P]
        gamma = dt[:, :, t] * _sig(trap[:, :, t])                           # [B,H]
        beta = dt[:, :, t + 1] * _sig(-trap[:, :, t + 1]) if t + 1 < S else np.zeros_like(gamma)
        kt = kh * (gamma + beta)[:, :, None, None]
        if t % C == 0:
            states[:, :, t // C] = hstate
        u = np.exp(da[:, :, t])[:, :, None, None] * hstate
        yt = np.einsum("bhrn,bhnp->bhrp", qh, u)
        yt = yt + gamma[:, :, None, None] * np.einsum("bhrs,bhsp->bhrp", qk, psi)
        if dd is not None:
            yt = yt + dd[None, :, None, None] * psi
        y[:, :, t] = yt
        hstate = u + np.einsum("bhrn,bhrp->bhnp", kt, psi)

    dmimo_o = dz = dmimo_z = None
    doh = None
    if reduce_o:
        doh = dout.transpose(0, 2, 1, 3)[:, :, :, None, :]                 # [B,H,S,1,P]
    if has_z:
        zh = zz.transpose(0, 2, 1, 3)[:, :, :, None, :]
        pz = zh * mz[None, :, None]                                         # [B,H,S,R,P]
        sg = _sig(pz)
        if reduce_o:
            dmimo_o = (y * pz * sg * doh).sum(axis=2)
            Gp = doh * mo[None, :, None] * y
        else:
            Gp = dout.transpose(0, 3, 1, 2, 4) * y
        gz = Gp * sg * (1.0 + pz * _sig(-pz))
        dz = (gz * mz[None, :, None]).sum(axis=3).transpose(0, 2, 1, 3)    # [B,S,H,P]
        dmimo_z = (gz * zh).sum(axis=2)
    elif reduce_o:
        dmimo_o = (y * doh).sum(axis=2)
    return dmimo_o, states, dz, dmimo_z, qk_dot, y


def forward(y, mimo_o, z, mimo_z):
    """Layer output from O2's y [B,H,S,R,P]: sum over ranks of mimo_o * y * silu(z * mimo_z)
    as [B,S,H,P] when mimo_o is given, else the per-rank y * silu(...) as [B,S,R,H,P];
    the silu factor is 1 without z."""
    y = _np(y)
    g = np.ones_like(y)
    if z is not None:
        pz = _np(z).transpose(0, 2, 1, 3)[:, :, :, None, :] * _np(mimo_z)[None, :, None]
        g = pz * _sig(pz)
    if mimo_o is not None:
        return (y * g * _np(mimo_o)[None, :, None]).sum(axis=3).transpose(0, 2, 1, 3)
    return (y * g).transpose(0, 2, 3, 1, 4)


def run_inputs(inp: dict):
    """Run O2 on a ``synth.inputs.make_inputs`` dict ("configs" recipe: needs da)."""
    return run(inp["dout"], inp["q"], inp["k"], inp["v"], inp["q_bias"], inp["k_bias"],
               inp["mimo_v"], inp["mimo_o"], inp["z"], inp["mimo_z"], inp["angles"], inp["da"],
               inp["dt"], inp["trap"], inp["d"], inp["chunk_size"], inp["rotary_dim_divisor"])
