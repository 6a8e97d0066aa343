"""Stage-2 backward oracle (mamba3_mimo_bwd_bwd) -- float64 autograd of the chunked
forward.

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may use it.

Source: the Triton-Ascend mamba3_mimo_bwd_bwd pull request page ("practice"
document: cache semantics, upstream-gradient mapping, gradient groups; the
migration note: signature, input and output table, supported range). The page
gives the dstates recurrence and the output list but not every gradient
formula, so every output is defined here as a partial derivative of

    L = sum over (b, t, r, h, p) of dPhiO * y

with y the pre-gate per-rank output of the chunked forward, dPhiO = dout *
mimo_o (reduced dout) or dout (per rank), all in exact arithmetic, and with
respect to one use of one quantity of that forward:

    DQ, DK      the biased q, k of each head (q + q_bias), laid out [B, S*R, H, N]
                with row t*R + r (the caller sums heads of a q/k group);
    DV          v;      DMIMO_V  mimo_v, per batch;     DD  d, per batch and head;
    DANGLES     the rotation angles;
    DFACTOR     the K scale factor_t = gamma_t + beta_t (causal block and state);
    DGAMMA      gamma_t in the same-token (diagonal) term only;
    DDA_CS      da_cs[t] in the inter-term scale exp(da_cs[t]);
    DDA         da_cs at each chunk's last real token in the state decay
                exp(da_cs[last]) (zero at every other token);
    DDA_CS_REV  da_cs_rev[t] in kappa = K~ * exp(da_cs_rev[t]);
    DSSDA       segsum[c][t][s] (s < t) in the causal block (zero elsewhere).
The cached states (entry states of each chunk) and qk_dot of the first stage
give the values of S_c and of the same-token dots; derivatives flow as through
the recurrence S_{c+1} = exp(da_cs[last]) S_c + kappa^T Psi and through
q0 . k0. gamma_t = dt_t sigmoid(trap_t), beta_t = dt_{t+1} (1 - sigmoid(trap_{t+1}))
(zero at the last token), as in the first stage's FP32 reference.
"""

from __future__ import annotations

import numpy as np
import torch

NAMES = ("DQ", "DK", "DV", "DMIMO_V", "DANGLES", "DFACTOR", "DGAMMA", "DDA", "DSSDA", "DDA_CS_REV",
         "DDA_CS", "DD")


def _t(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().to(torch.float64)
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def _rot(x, th):
    """Partial rotate-half of the last axis by angles th [..., W]: pairs (n, N/2 + n), n < W."""
    N, W = x.shape[-1], th.shape[-1]
    M = N // 2
    c, s = torch.cos(th), torch.sin(th)
    a, e = x[..., :W], x[..., M:M + W]
    return torch.cat([c * a - s * e, x[..., W:M], s * a + c * e, x[..., M + W:]], dim=-1)


def run(dout, q, k, v, q_bias, k_bias, mimo_v, states, qk_dot, da_cs, da_cs_rev, dt, trap, segsum, angles,
        mimo_o=None, d=None, chunk_size=16):
    """float64 numpy dict of the 12 gradients (DD is None without d)."""
    q, k, v = _t(q), _t(k), _t(v)
    B, S, R, G, N = q.shape
    H, P = v.shape[2], v.shape[3]
    C = int(chunk_size)
    nc = (S + C - 1) // C
    grp = torch.arange(H) // (H // G)
    W = angles.shape[-1]
    dt, trap = _t(dt), _t(trap)
    sig = torch.sigmoid(trap)
    gam0 = dt * sig
    beta = torch.zeros_like(gam0)
    beta[..., :-1] = dt[..., 1:] * (1.0 - sig[..., 1:])

    # leaves, per batch and head where the page's outputs are per batch and head
    Q0 = (q[:, :, :, grp].permute(0, 3, 1, 2, 4) + _t(q_bias)[None, :, None]).requires_grad_()   # [B,H,S,R,N]
    K0 = (k[:, :, :, grp].permute(0, 3, 1, 2, 4) + _t(k_bias)[None, :, None]).requires_grad_()
    V = v.clone().requires_grad_()                                                              # [B,S,H,P]
    MV = _t(mimo_v)[None].expand(B, H, R, P).clone().requires_grad_()                           # [B,H,R,P]
    ANG = _t(angles).clone().requires_grad_()                                                   # [B,S,H,W]
    FAC = (gam0 + beta).clone().requires_grad_()                                                # [B,H,S]
    GAM = gam0.clone().requires_grad_()
    CSI = _t(da_cs).clone().requires_grad_()
    CSS = _t(da_cs).clone().requires_grad_()
    REV = _t(da_cs_rev).clone().requires_grad_()
    SEG = _t(segsum).clone().requires_grad_()                                                   # [B,H,nc,C,C]
    D = None if d is None else _t(d)[None].expand(B, H).clone().requires_grad_()                # [B,H]

    dout = _t(dout)
    if mimo_o is not None:
        dphio = dout.permute(0, 2, 1, 3)[:, :, :, None, :] * _t(mimo_o)[None, :, None]          # [B,H,S,R,P]
    else:
        dphio = dout.permute(0, 3, 1, 2, 4)
    SC = _t(states)                                                                             # [B,H,nc,N,P]
    QKC = _t(qk_dot)                                                                            # [B,H,S,R,R]

    th = ANG.permute(0, 2, 1, 3)[:, :, :, None, :]                                              # [B,H,S,1,W]
    Qh = _rot(Q0, th)
    Kh = _rot(K0, th)
    Kt = Kh * FAC[..., None, None]
    Psi = V.permute(0, 2, 1, 3)[:, :, :, None, :] * MV[:, :, None]                              # [B,H,S,R,P]
    qk_exact = torch.einsum("bhtrn,bhtsn->bhtrs", Q0, K0)
    qk = qk_exact + (QKC - qk_exact).detach()

    # the per-token tensors cut into chunks once: an indexed slice per chunk would make
    # autograd build a whole-sequence gradient for every chunk (quadratic in S); the
    # values and the derivatives are the same either way
    def chunks(x):
        return x.split(C, dim=2)

    Qh_c, Kt_c, Psi_c, qk_c, dpo_c = chunks(Qh), chunks(Kt), chunks(Psi), chunks(qk), chunks(dphio)
    CSI_c, CSS_c, REV_c, GAM_c = chunks(CSI), chunks(CSS), chunks(REV), chunks(GAM)
    SEG_c = SEG.unbind(2)
    L = torch.zeros((), dtype=torch.float64)
    Srec = torch.zeros((B, H, N, P), dtype=torch.float64)
    for c in range(nc):
        cl = Qh_c[c].shape[2]
        Sused = Srec + (SC[:, :, c] - Srec).detach()
        inter = torch.einsum("bhtrn,bhnp->bhtrp", Qh_c[c], Sused) * torch.exp(CSI_c[c])[..., None, None]
        scores = torch.einsum("bhtrn,bhsqn->bhtrsq", Qh_c[c], Kt_c[c])
        mask = torch.tril(torch.ones(cl, cl, dtype=torch.bool), diagonal=-1)
        decay = torch.where(mask, torch.exp(torch.where(mask, SEG_c[c][:, :, :cl, :cl], 0.0)), 0.0)
        intra = torch.einsum("bhtrsq,bhts,bhsqp->bhtrp", scores, decay, Psi_c[c])
        diag = GAM_c[c][..., None, None] * torch.einsum("bhtrs,bhtsp->bhtrp", qk_c[c], Psi_c[c])
        y = inter + intra + diag
        if D is not None:
            y = y + D[:, :, None, None, None] * Psi_c[c]
        L = L + (dpo_c[c] * y).sum()
        kap = Kt_c[c] * torch.exp(REV_c[c])[..., None, None]
        Srec = torch.exp(CSS_c[c][:, :, cl - 1])[..., None, None] * Sused + torch.einsum(
            "bhtrn,bhtrp->bhnp", kap, Psi_c[c])
    L.backward()

    def grad(x):
        # a quantity the loss does not reach (e.g. the state decay of a one-chunk
        # sequence) has a zero derivative
        return torch.zeros_like(x) if x.grad is None else x.grad

    out = {
        "DQ": grad(Q0).permute(0, 2, 3, 1, 4).reshape(B, S * R, H, N),
        "DK": grad(K0).permute(0, 2, 3, 1, 4).reshape(B, S * R, H, N),
        "DV": grad(V),
        "DMIMO_V": grad(MV),
        "DANGLES": grad(ANG),
        "DFACTOR": grad(FAC),
        "DGAMMA": grad(GAM),
        "DDA": grad(CSS),
        "DSSDA": grad(SEG),
        "DDA_CS_REV": grad(REV),
        "DDA_CS": grad(CSI),
        "DD": None if D is None else grad(D),
    }
    return {kk: (None if vv is None else vv.detach().numpy()) for kk, vv in out.items()}


def run_inputs(inp: dict, states, qk_dot, **kw):
    """``run`` on a ``synth.inputs.make_inputs`` dict with the given caches."""
    return run(inp["dout"], inp["q"], inp["k"], inp["v"], inp["q_bias"], inp["k_bias"], inp["mimo_v"], states,
               qk_dot, inp["da_cs"], inp["da_cs_rev"], inp["dt"], inp["trap"], inp["segsum"], inp["angles"],
               inp["mimo_o"], inp["d"], inp["chunk_size"], **kw)
