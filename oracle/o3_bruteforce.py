"""O3 -- quadratic-form brute force for tiny inputs (float64, no rounding).

TEST INFRASTRUCTURE ONLY.

Unrolls the recurrence of the Triton-Ascend mamba_mimo_bwd_fwd page's
chunked scan into its closed form over all token pairs, with the global
inclusive cumulative log decay L_t = sum_{l<=t} da_l:

  y[t,r]    = sum_{j<t} sum_r' exp(L_t - L_j) (qh[t,r] . kt[j,r']) psi[j,r']
              + gamma_t sum_r' (q0[t,r] . k0[t,r']) psi[t,r'] + d_h psi[t,r]
  states[c] = sum_{j<cC} exp(L_{cC-1} - L_j) sum_r kt[j,r]^T psi[j,r]

Each preparation step (bias, rotation, PsiV, trapezoidal factor) and the
gating are written here a second time, in matrix form, so that nothing is
shared with O1 or O2. O(S^2) memory: tiny inputs only.
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


def run(dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da, dt, trap, d,
        chunk_size, rotary_dim_divisor=4):
    q, k, v = _np(q), _np(k), _np(v)
    B, S, R, G, N = q.shape
    H, P = v.shape[2:]
    assert S <= 512, "brute force is for tiny inputs"
    C = int(chunk_size)
    nc = (S + C - 1) // C
    W, M = _np(angles).shape[-1], N // 2
    grp = np.arange(H) // (H // G)
    ang, da, dt, trap = _np(angles), _np(da), _np(dt), _np(trap)

    # [B,H,S,R,N] biased q/k for every head
    Q0 = q[:, :, :, grp, :].transpose(0, 3, 1, 2, 4) + _np(q_bias)[None, :, None]
    K0 = k[:, :, :, grp, :].transpose(0, 3, 1, 2, 4) + _np(k_bias)[None, :, None]
    # rotation as an explicit orthogonal matrix per (b,h,t): x_rot = x @ Rm^T
    th = ang.transpose(0, 2, 1, 3)                                # [B,H,S,W]
    Rm = np.broadcast_to(np.eye(N), (B, H, S, N, N)).copy()
    idx = np.arange(W)
    Rm[..., idx, idx] = np.cos(th)
    Rm[..., idx, M + idx] = -np.sin(th)
    Rm[..., M + idx, idx] = np.sin(th)
    Rm[..., M + idx, M + idx] = np.cos(th)
    Qh = np.einsum("bhtmn,bhtrn->bhtrm", Rm, Q0)
    Kh = np.einsum("bhtmn,bhtrn->bhtrm", Rm, K0)
    Psi = v.transpose(0, 2, 1, 3)[:, :, :, None, :] * _np(mimo_v)[None, :, None]   # [B,H,S,R,P]
    sig = lambda x: 1.0 / (1.0 + np.exp(-x))
    gamma = dt * sig(trap)                                          # [B,H,S]
    beta = np.zeros_like(gamma)
    beta[..., :-1] = dt[..., 1:] * sig(-trap[..., 1:])
    Kt = Kh * (gamma + beta)[..., None, None]

    L = np.cumsum(da, axis=-1)                                      # [B,H,S]
    lower = np.tril(np.ones((S, S), dtype=bool), -1)               # j < t
    Dm = np.where(lower, np.exp(np.where(lower, L[..., :, None] - L[..., None, :], 0.0)), 0.0)
    scores = np.einsum("bhtrn,bhjsn->bhtrjs", Qh, Kt) * Dm[:, :, :, None, :, None]
    y = np.einsum("bhtrjs,bhjsp->bhtrp", scores, Psi)
    QK0 = np.einsum("bhtrn,bhtsn->bhtrs", Q0, K0)
    y = y + gamma[..., None, None] * np.einsum("bhtrs,bhtsp->bhtrp", QK0, Psi)
    if d is not None:
        y = y + _np(d)[None, :, None, None, None] * Psi

    states = np.zeros((B, H, nc, N, P))
    outer = np.einsum("bhjrn,bhjrp->bhjnp", Kt, Psi)                # per-token K^T Psi
    for c in range(1, nc):
        e = c * C - 1
        w = np.exp(L[..., e:e + 1] - L[..., : c * C])               # [B,H,cC]
        states[:, :, c] = np.einsum("bhj,bhjnp->bhnp", w, outer[:, :, : c * C])

    dmimo_o = dz = dmimo_z = None
    if mimo_o is not None:
        Dh = _np(dout).transpose(0, 2, 1, 3)[:, :, :, None, :]
    if z is not None:
        Zh = _np(z).transpose(0, 2, 1, 3)[:, :, :, None, :]
        PZ = Zh * _np(mimo_z)[None, :, None]
        if mimo_o is not None:
            dmimo_o = np.sum(y * (PZ * sig(PZ)) * Dh, axis=2)
            Gp = Dh * _np(mimo_o)[None, :, None] * y
        else:
            Gp = np.einsum("bsrhp->bhsrp", _np(dout)) * y
        GZ = Gp * sig(PZ) * (1.0 + PZ * sig(-PZ))
        dz = np.einsum("bhsrp,hrp->bshp", GZ, _np(mimo_z))
        dmimo_z = np.sum(GZ * Zh, axis=2)
    elif mimo_o is not None:
        dmimo_o = np.sum(y * Dh, axis=2)
    return dmimo_o, states, dz, dmimo_z, QK0, y


def run_inputs(inp: dict):
    return run(inp["dout"], inp["q"], inp["k"], inp["v"], inp["q_bias"], inp["k_bias"],
               inp["mimo_v"], inp["mimo_o"], inp["z"], inp["mimo_z"], inp["angles"], inp["da"],
               inp["dt"], inp["trap"], inp["d"], inp["chunk_size"], inp["rotary_dim_divisor"])
