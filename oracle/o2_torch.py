"""Unchunked token-by-token MIMO recurrence in float64 torch, for autograd.

TEST INFRASTRUCTURE ONLY. The same recurrence as ``o2_sequential`` (numpy),
written with torch operations so that its gradients can be taken; it shares no
code with the chunked oracles. Per token t (Triton-Ascend mamba_mimo_bwd_fwd
page, BF16-boundary reference read in exact arithmetic):
    q^, k^ = rot(q + q_bias), rot(k + k_bias);   Psi = v * mimo_v
    gamma = dt_t sigmoid(trap_t),  beta = dt_{t+1} (1 - sigmoid(trap_{t+1}))
    u = exp(da_t) h_{t-1};   y_t = q^ u + gamma (q0 k0^T) Psi + d Psi
    h_t = u + (k^ (gamma + beta))^T Psi
"""

from __future__ import annotations

import numpy as np
import torch


def _t(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().to(torch.float64)
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def _rot(x, th):
    N, W = x.shape[-1], th.shape[-1]
    M = N // 2
    c, s = torch.cos(th), torch.sin(th)
    a, e = x[..., :W], x[..., M:M + W]
    return torch.cat([c * a - s * e, x[..., W:M], s * a + c * e, x[..., M + W:]], dim=-1)


def grads(dout, q, k, v, q_bias, k_bias, mimo_v, angles, da, dt, trap, mimo_o=None, d=None):
    """Gradients of L = sum(dPhiO * y) with respect to q, k [B,S,R,G,N], v, mimo_v,
    angles, da, dt, trap and d (float64 numpy dict; d's is None without d)."""
    Q = _t(q).clone().requires_grad_()
    K = _t(k).clone().requires_grad_()
    V = _t(v).clone().requires_grad_()
    MV = _t(mimo_v).clone().requires_grad_()
    ANG = _t(angles).clone().requires_grad_()
    DA = _t(da).clone().requires_grad_()
    DT = _t(dt).clone().requires_grad_()
    TR = _t(trap).clone().requires_grad_()
    Dd = None if d is None else _t(d).clone().requires_grad_()
    B, S, R, G, N = Q.shape
    H, P = V.shape[2], V.shape[3]
    grp = torch.arange(H) // (H // G)
    dout = _t(dout)
    if mimo_o is not None:
        dphio = dout[:, :, :, None, :] * _t(mimo_o)[None, None]                      # [B,S,H,R,P]
    else:
        dphio = dout.permute(0, 1, 3, 2, 4)                                          # [B,S,H,R,P]
    qb, kb = _t(q_bias), _t(k_bias)
    sig = torch.sigmoid(TR)
    h = torch.zeros((B, H, N, P), dtype=torch.float64)
    L = torch.zeros((), dtype=torch.float64)
    for t in range(S):
        q0 = Q[:, t][:, :, grp].permute(0, 2, 1, 3) + qb[None]                        # [B,H,R,N]
        k0 = K[:, t][:, :, grp].permute(0, 2, 1, 3) + kb[None]
        th = ANG[:, t][:, :, None, :]
        qh, kh = _rot(q0, th), _rot(k0, th)
        psi = V[:, t][:, :, None, :] * MV[None]                                       # [B,H,R,P]
        gamma = DT[:, :, t] * sig[:, :, t]
        beta = DT[:, :, t + 1] * (1.0 - sig[:, :, t + 1]) if t + 1 < S else torch.zeros_like(gamma)
        u = torch.exp(DA[:, :, t])[..., None, None] * h
        y = torch.einsum("bhrn,bhnp->bhrp", qh, u)
        y = y + gamma[..., None, None] * torch.einsum("bhrn,bhsn,bhsp->bhrp", q0, k0, psi)
        if Dd is not None:
            y = y + Dd[None, :, None, None] * psi
        L = L + (dphio[:, t] * y).sum()
        h = u + torch.einsum("bhrn,bhrp->bhnp", kh * (gamma + beta)[..., None, None], psi)
    L.backward()
    out = {"q": Q.grad, "k": K.grad, "v": V.grad, "mimo_v": MV.grad, "angles": ANG.grad, "da": DA.grad,
           "dt": DT.grad, "trap": TR.grad, "d": None if Dd is None else Dd.grad}
    return {kk: (None if vv is None else vv.numpy()) for kk, vv in out.items()}
