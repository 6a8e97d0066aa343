"""Public Python entry points: ``mamba_mimo_bwd_fwd``, the layer output ``mamba_mimo_fwd``,
their fp32-intermediate variants, the stage-2 backward ``mamba3_mimo_bwd_bwd`` and the SISO
forward ``mamba3_siso_fwd``.

Signature, defaults, output order, validation order and error types follow
the Triton-Ascend mamba_mimo_bwd_fwd page (public API module: the
``MambaMimoBwdFwdOutputs`` named tuple, ``_check_tensor`` and
``_validate_inputs``). PyTorch supplies device memory (outputs and the
workspace) and the current stream; every step of the computation runs in the
HIP library behind ``include/mimo_bwd_fwd.h``.
"""

from __future__ import annotations

import ctypes
from functools import lru_cache
from typing import NamedTuple, Optional

import torch

from . import _lib

__all__ = ["MambaMimoBwdFwdOutputs", "mamba_mimo_bwd_fwd", "mamba_mimo_fwd", "mamba_mimo_bwd_fwd_fp32",
           "mamba_mimo_fwd_fp32", "mamba3_mimo_bwd_bwd", "mamba3_siso_fwd", "workspace_size",
           "fwd_workspace_size"]

Tensor = torch.Tensor


class MambaMimoBwdFwdOutputs(NamedTuple):
    """Outputs of the first Mamba-3 MIMO backward stage, in the pages' order."""

    dmimo_o: Optional[Tensor]
    states: Tensor
    dz: Optional[Tensor]
    dmimo_z: Optional[Tensor]
    qk_dot: Tensor


@lru_cache
def _is_gfx950(index: int) -> bool:
    name = getattr(torch.cuda.get_device_properties(index), "gcnArchName", "")
    return name.startswith("gfx950")


def _check_tensor(name, tensor, shape, dtype, device):
    if tuple(tensor.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(tensor.shape)}")
    if tensor.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {tensor.dtype}")
    if tensor.device != device:
        raise ValueError(f"{name} must be on {device}, got {tensor.device}")


def _validate_inputs(dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs,
                     da_cs_rev, dt, trap, d, segsum, chunk_size, rotary_dim_divisor, *, fwd=False):
    if q.dim() != 5:
        raise ValueError("q must have shape [B, S, R, G, N]")
    batch, seqlen, rank, groups, state_dim = q.shape
    if batch < 1 or seqlen < 1 or rank < 1 or groups < 1:
        raise ValueError("B, S, R and G must be positive")
    if q.dtype != torch.bfloat16:
        raise TypeError("q, k, v, dout and trap must use torch.bfloat16")
    if q.device.type != "cuda":
        raise ValueError("mamba_mimo_bwd_fwd requires GPU (HIP) tensors")
    if not _is_gfx950(q.device.index if q.device.index is not None else torch.cuda.current_device()):
        raise NotImplementedError("mamba_mimo_bwd_fwd supports gfx950 (MI355X) devices only")
    if chunk_size < 1 or chunk_size * rank > 128:
        raise ValueError("chunk_size * R must be in [1, 128]")
    if rotary_dim_divisor not in (2, 4):
        raise ValueError("rotary_dim_divisor must be 2 or 4")
    if state_dim % rotary_dim_divisor or state_dim % 2:
        raise ValueError("N must be even and divisible by rotary_dim_divisor")
    if state_dim > 128:
        raise ValueError("N greater than 128 is not supported")
    if k.shape != q.shape:
        raise ValueError("k must have the same shape as q")
    if v.dim() != 4 or tuple(v.shape[:2]) != (batch, seqlen):
        raise ValueError("v must have shape [B, S, H, P]")
    heads, value_dim = v.shape[2:]
    if heads % groups:
        raise ValueError("H must be divisible by G")
    if value_dim > 128:
        raise ValueError("P greater than 128 is not supported")

    device = q.device
    _check_tensor("k", k, tuple(q.shape), torch.bfloat16, device)
    _check_tensor("v", v, (batch, seqlen, heads, value_dim), torch.bfloat16, device)
    _check_tensor("q_bias", q_bias, (heads, rank, state_dim), torch.float32, device)
    _check_tensor("k_bias", k_bias, (heads, rank, state_dim), torch.float32, device)
    _check_tensor("mimo_v", mimo_v, (heads, rank, value_dim), torch.float32, device)
    _check_tensor("angles", angles, (batch, seqlen, heads, state_dim // rotary_dim_divisor),
                  torch.float32, device)
    for name, tensor in (("da_cs", da_cs), ("da_cs_rev", da_cs_rev), ("dt", dt)):
        _check_tensor(name, tensor, (batch, heads, seqlen), torch.float32, device)
    _check_tensor("trap", trap, (batch, heads, seqlen), torch.bfloat16, device)
    nchunks = (seqlen + chunk_size - 1) // chunk_size
    _check_tensor("segsum", segsum, (batch, heads, nchunks, chunk_size, chunk_size), torch.float32, device)
    if d is not None:
        _check_tensor("d", d, (heads,), torch.float32, device)
    if mimo_o is not None:
        _check_tensor("mimo_o", mimo_o, (heads, rank, value_dim), torch.float32, device)
    if not fwd:
        if mimo_o is not None:
            _check_tensor("dout", dout, (batch, seqlen, heads, value_dim), torch.bfloat16, device)
        else:
            _check_tensor("dout", dout, (batch, seqlen, rank, heads, value_dim), torch.bfloat16, device)
    if z is None:
        if mimo_z is not None:
            raise ValueError("mimo_z must be None when z is None")
    else:
        _check_tensor("z", z, (batch, seqlen, heads, value_dim), torch.bfloat16, device)
        if mimo_z is None:
            raise ValueError("mimo_z is required when z is present")
        _check_tensor("mimo_z", mimo_z, (heads, rank, value_dim), torch.float32, device)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _raise(status: int):
    msg = _lib.last_error()
    if status == _lib.MIMO_ERR_VALUE:
        raise ValueError(msg)
    if status == _lib.MIMO_ERR_TYPE:
        raise TypeError(msg)
    if status == _lib.MIMO_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise RuntimeError(f"mimo_bwd_fwd failed: {msg}")


def _make_args(B, S, H, G, R, N, P, C, rd, t: dict, outs: dict, workspace=None, ws_bytes=0):
    a = _lib.MimoBwdFwdArgs()
    a.B, a.S, a.H, a.G, a.R, a.N, a.P = B, S, H, G, R, N, P
    a.chunk_size, a.rotary_dim_divisor = C, rd
    for name in ("dout", "q", "k", "v", "q_bias", "k_bias", "mimo_v", "mimo_o", "z", "mimo_z",
                 "angles", "da_cs", "da_cs_rev", "dt", "trap", "d", "segsum"):
        x = t.get(name)
        setattr(a, name, None if x is None else x.data_ptr())
    for name in ("dmimo_o", "states", "dz", "dmimo_z", "qk_dot"):
        x = outs.get(name)
        setattr(a, name, None if x is None else x.data_ptr())
    a.workspace = None if workspace is None else workspace.data_ptr()
    a.workspace_bytes = ws_bytes
    return a


def workspace_size(B, S, H, G, R, N, P, chunk_size, rotary_dim_divisor=4, *, reduce_o=True,
                   has_z=True) -> int:
    """Workspace bytes the library needs for these sizes and branches."""
    a = _lib.MimoBwdFwdArgs()
    a.B, a.S, a.H, a.G, a.R, a.N, a.P = B, S, H, G, R, N, P
    a.chunk_size, a.rotary_dim_divisor = chunk_size, rotary_dim_divisor
    # only NULL-ness of the optional pointers matters here
    a.mimo_o = 1 if reduce_o else None
    a.z = a.mimo_z = 1 if has_z else None
    n = ctypes.c_size_t(0)
    st = _lib.lib().mimo_bwd_fwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
    if st != _lib.MIMO_OK:
        _raise(st)
    return int(n.value)


def mamba_mimo_bwd_fwd(dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs,
                       da_cs_rev, dt, trap, d, segsum, chunk_size: int = 16,
                       rotary_dim_divisor: int = 4, *, out: Optional[dict] = None,
                       workspace: Optional[Tensor] = None) -> MambaMimoBwdFwdOutputs:
    """Run the Mamba-3 MIMO backward first stage on the current HIP stream.

    Passing ``mimo_o`` selects reduced dout; passing ``z`` enables ``dz`` and
    ``dmimo_z``; passing ``d`` enables the skip term. Optional ``out`` holds
    preallocated output tensors (keys dmimo_o, states, dz, dmimo_z, qk_dot) and
    ``workspace`` a preallocated uint8 scratch tensor (see ``workspace_size``).
    The call is asynchronous with respect to the host.
    """
    return _bwd_fwd("mimo_bwd_fwd", dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles,
                    da_cs, da_cs_rev, dt, trap, d, segsum, chunk_size, rotary_dim_divisor, out, workspace)


def mamba_mimo_bwd_fwd_fp32(dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs,
                            da_cs_rev, dt, trap, d, segsum, chunk_size: int = 16,
                            rotary_dim_divisor: int = 4, *, out: Optional[dict] = None,
                            workspace: Optional[Tensor] = None) -> MambaMimoBwdFwdOutputs:
    """``mamba_mimo_bwd_fwd`` with fp32 intermediates (no intermediate bf16 rounding;
    outputs in their dtypes): the pages' FP32 reference semantics."""
    return _bwd_fwd("mimo_bwd_fwd_f32", dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z,
                    angles, da_cs, da_cs_rev, dt, trap, d, segsum, chunk_size, rotary_dim_divisor, out,
                    workspace)


def _bwd_fwd(fn, dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs, da_cs_rev,
             dt, trap, d, segsum, chunk_size, rotary_dim_divisor, out, workspace):
    _validate_inputs(dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs,
                     da_cs_rev, dt, trap, d, segsum, chunk_size, rotary_dim_divisor)
    L = _lib.lib()
    B, S, R, G, N = q.shape
    H, P = v.shape[2:]
    C = int(chunk_size)
    nc = (S + C - 1) // C
    dev = q.device
    t = {name: (None if x is None else x.contiguous()) for name, x in (
        ("dout", dout), ("q", q), ("k", k), ("v", v), ("q_bias", q_bias), ("k_bias", k_bias),
        ("mimo_v", mimo_v), ("mimo_o", mimo_o), ("z", z), ("mimo_z", mimo_z), ("angles", angles),
        ("da_cs", da_cs), ("da_cs_rev", da_cs_rev), ("dt", dt), ("trap", trap), ("d", d),
        ("segsum", segsum))}
    reduce_o, has_z = mimo_o is not None, z is not None
    if out is None:
        out = {
            "dmimo_o": torch.empty((B, H, R, P), dtype=torch.float32, device=dev) if reduce_o else None,
            "states": torch.empty((B, H, nc, N, P), dtype=torch.bfloat16, device=dev),
            "dz": torch.empty((B, S, H, P), dtype=torch.bfloat16, device=dev) if has_z else None,
            "dmimo_z": torch.empty((B, H, R, P), dtype=torch.float32, device=dev) if has_z else None,
            "qk_dot": torch.empty((B, H, S, R, R), dtype=torch.bfloat16, device=dev),
        }
    args = _make_args(B, S, H, G, R, N, P, C, int(rotary_dim_divisor), t, out)
    need = ctypes.c_size_t(0)
    st = getattr(L, fn + "_workspace_size")(ctypes.byref(args), ctypes.byref(need))
    if st != _lib.MIMO_OK:
        _raise(st)
    if need.value > 0:
        if workspace is None or workspace.numel() < need.value:
            workspace = torch.empty(int(need.value), dtype=torch.uint8, device=dev)
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = getattr(L, fn)(ctypes.byref(args), ctypes.c_void_p(stream))
    if st != _lib.MIMO_OK:
        _raise(st)
    return MambaMimoBwdFwdOutputs(out["dmimo_o"], out["states"], out["dz"], out["dmimo_z"], out["qk_dot"])


_FWD_INPUTS = ("q", "k", "v", "q_bias", "k_bias", "mimo_v", "mimo_o", "z", "mimo_z", "angles", "da_cs",
               "da_cs_rev", "dt", "trap", "d", "segsum")


def _make_fwd_args(B, S, H, G, R, N, P, C, rd, t: dict, o, workspace=None, ws_bytes=0):
    a = _lib.MimoFwdArgs()
    a.B, a.S, a.H, a.G, a.R, a.N, a.P = B, S, H, G, R, N, P
    a.chunk_size, a.rotary_dim_divisor = C, rd
    for name in _FWD_INPUTS:
        x = t.get(name)
        setattr(a, name, None if x is None else x.data_ptr())
    a.o = None if o is None else o.data_ptr()
    a.workspace = None if workspace is None else workspace.data_ptr()
    a.workspace_bytes = ws_bytes
    return a


def fwd_workspace_size(B, S, H, G, R, N, P, chunk_size, rotary_dim_divisor=4, *, reduce_o=True,
                       has_z=True) -> int:
    """Workspace bytes ``mamba_mimo_fwd`` needs for these sizes and branches."""
    a = _lib.MimoFwdArgs()
    a.B, a.S, a.H, a.G, a.R, a.N, a.P = B, S, H, G, R, N, P
    a.chunk_size, a.rotary_dim_divisor = chunk_size, rotary_dim_divisor
    a.mimo_o = 1 if reduce_o else None
    a.z = a.mimo_z = 1 if has_z else None
    n = ctypes.c_size_t(0)
    st = _lib.lib().mimo_fwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
    if st != _lib.MIMO_OK:
        _raise(st)
    return int(n.value)


def mamba_mimo_fwd(q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs, da_cs_rev, dt,
                   trap, d, segsum, chunk_size: int = 16, rotary_dim_divisor: int = 4, *,
                   out: Optional[Tensor] = None, workspace: Optional[Tensor] = None) -> Tensor:
    """Layer output of the chunked MIMO scan whose gradients ``mamba_mimo_bwd_fwd``
    computes: ``o`` [B,S,H,P] bf16 = sum over ranks of (y * bf16(mimo_o)) * silu(z * mimo_z)
    when ``mimo_o`` is given, else the per-rank ``y * silu(z * mimo_z)`` as [B,S,R,H,P]
    (the gate is left out without ``z``). Same inputs as the backward stage minus dout;
    asynchronous on the current HIP stream.
    """
    return _fwd("mimo_fwd", q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs,
                da_cs_rev, dt, trap, d, segsum, chunk_size, rotary_dim_divisor, out, workspace)


def mamba_mimo_fwd_fp32(q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs, da_cs_rev,
                        dt, trap, d, segsum, chunk_size: int = 16, rotary_dim_divisor: int = 4, *,
                        out: Optional[Tensor] = None, workspace: Optional[Tensor] = None) -> Tensor:
    """``mamba_mimo_fwd`` with fp32 intermediates (only o is rounded to bf16)."""
    return _fwd("mimo_fwd_f32", q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs,
                da_cs_rev, dt, trap, d, segsum, chunk_size, rotary_dim_divisor, out, workspace)


def _fwd(fn, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs, da_cs_rev, dt, trap, d,
         segsum, chunk_size, rotary_dim_divisor, out, workspace):
    _validate_inputs(None, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs,
                     da_cs_rev, dt, trap, d, segsum, chunk_size, rotary_dim_divisor, fwd=True)
    L = _lib.lib()
    B, S, R, G, N = q.shape
    H, P = v.shape[2:]
    C = int(chunk_size)
    dev = q.device
    vals = (q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs, da_cs_rev, dt, trap, d,
            segsum)
    t = {name: (None if x is None else x.contiguous()) for name, x in zip(_FWD_INPUTS, vals)}
    shape = (B, S, H, P) if mimo_o is not None else (B, S, R, H, P)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    else:
        _check_tensor("out", out, shape, torch.bfloat16, dev)
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
    args = _make_fwd_args(B, S, H, G, R, N, P, C, int(rotary_dim_divisor), t, out)
    need = ctypes.c_size_t(0)
    st = getattr(L, fn + "_workspace_size")(ctypes.byref(args), ctypes.byref(need))
    if st != _lib.MIMO_OK:
        _raise(st)
    if need.value > 0:
        if workspace is None or workspace.numel() < need.value:
            workspace = torch.empty(int(need.value), dtype=torch.uint8, device=dev)
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = getattr(L, fn)(ctypes.byref(args), ctypes.c_void_p(stream))
    if st != _lib.MIMO_OK:
        _raise(st)
    return out


# ---------------------------------------------------------------- SISO forward
_SISO_INPUTS = ("q", "k", "v", "adt", "dt", "trap", "q_bias", "k_bias", "angles", "d", "z")


def _validate_siso(q, k, v, adt, dt, trap, q_bias, k_bias, angles, d, z, chunk_size):
    if isinstance(chunk_size, bool) or not isinstance(chunk_size, int) or chunk_size not in (32, 64):
        raise ValueError("chunk_size must be 32 or 64")
    if q.dim() != 4 or k.shape != q.shape:
        raise ValueError("q and k must have shape [B, S, Hq, K]")
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("q, k, v and z must be torch.float16 or torch.bfloat16")
    if q.device.type != "cuda":
        raise ValueError("mamba3_siso_fwd requires GPU (HIP) tensors")
    if not _is_gfx950(q.device.index if q.device.index is not None else torch.cuda.current_device()):
        raise NotImplementedError("mamba3_siso_fwd supports gfx950 (MI355X) devices only")
    B, S, Hq, K = q.shape
    if v.dim() != 4 or tuple(v.shape[:2]) != (B, S):
        raise ValueError("v must have shape [B, S, H, V]")
    H, V = v.shape[2:]
    if H % Hq:
        raise ValueError("H must be divisible by Hq")
    if angles.dim() != 4 or tuple(angles.shape[:3]) != (B, S, H):
        raise ValueError("angles must have shape [B, S, H, A]")
    A = angles.shape[3]
    if A % 2 or 2 * A > K:
        raise ValueError("the angle width A must be even and at most K / 2")
    dev = q.device
    _check_tensor("k", k, (B, S, Hq, K), q.dtype, dev)
    _check_tensor("v", v, (B, S, H, V), q.dtype, dev)
    for name, x in (("adt", adt), ("dt", dt), ("trap", trap)):
        _check_tensor(name, x, (B, H, S), torch.float32, dev)
    _check_tensor("q_bias", q_bias, (H, K), torch.float32, dev)
    _check_tensor("k_bias", k_bias, (H, K), torch.float32, dev)
    _check_tensor("angles", angles, (B, S, H, A), torch.float32, dev)
    if d is not None:
        _check_tensor("d", d, (H,), torch.float32, dev)
    if z is not None:
        _check_tensor("z", z, (B, S, H, V), q.dtype, dev)
    return B, S, Hq, H, K, V, A


def _make_siso_args(dims, dtype, t: dict, out, workspace=None, ws_bytes=0):
    B, S, Hq, H, K, V, A, C = dims
    a = _lib.MimoSisoFwdArgs()
    a.B, a.S, a.Hq, a.H, a.K, a.V = B, S, Hq, H, K, V
    a.chunk_size, a.A = C, A
    a.dtype = _lib.DTYPE_FP16 if dtype == torch.float16 else _lib.DTYPE_BF16
    for name in _SISO_INPUTS:
        x = t.get(name)
        setattr(a, name, None if x is None else x.data_ptr())
    a.out = None if out is None else out.data_ptr()
    a.workspace = None if workspace is None else workspace.data_ptr()
    a.workspace_bytes = ws_bytes
    return a


def mamba3_siso_fwd(q, k, v, adt, dt, trap, q_bias, k_bias, angles, d=None, z=None,
                    chunk_size: int = 64, *, out: Optional[Tensor] = None,
                    workspace: Optional[Tensor] = None) -> Tensor:
    """Dense SISO forward output [B,S,H,V] in q's dtype: bias and rotary on q/k, the
    trapezoid weights from dt and sigmoid(trap), the adt decay inside and across chunks,
    the same-token skip term, the optional D skip and SiLU(z) gate. q, k [B,S,Hq,K] and
    v, z [B,S,H,V] in float16 or bfloat16; adt, dt, trap [B,H,S], q_bias, k_bias [H,K],
    angles [B,S,H,A] (A even, <= K/2) and d [H] in float32; chunk_size 32 or 64.
    Intermediates are fp32. Asynchronous on the current HIP stream."""
    dims = _validate_siso(q, k, v, adt, dt, trap, q_bias, k_bias, angles, d, z, chunk_size)
    B, S, Hq, H, K, V, A = dims
    L = _lib.lib()
    dev = q.device
    vals = (q, k, v, adt, dt, trap, q_bias, k_bias, angles, d, z)
    t = {n: (None if x is None else x.contiguous()) for n, x in zip(_SISO_INPUTS, vals)}
    if out is None:
        out = torch.empty((B, S, H, V), dtype=q.dtype, device=dev)
    else:
        _check_tensor("out", out, (B, S, H, V), q.dtype, dev)
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
    args = _make_siso_args(dims + (int(chunk_size),), q.dtype, t, out)
    need = ctypes.c_size_t(0)
    st = L.mimo_siso_fwd_workspace_size(ctypes.byref(args), ctypes.byref(need))
    if st != _lib.MIMO_OK:
        _raise(st)
    if need.value > 0:
        if workspace is None or workspace.numel() < need.value:
            workspace = torch.empty(int(need.value), dtype=torch.uint8, device=dev)
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = L.mimo_siso_fwd(ctypes.byref(args), ctypes.c_void_p(stream))
    if st != _lib.MIMO_OK:
        _raise(st)
    return out


# ---------------------------------------------------------------- stage-2 backward
BWD2_KEYS = ("DQ", "DK", "DV", "DMIMO_V", "DANGLES", "DFACTOR", "DGAMMA", "DDA", "DSSDA", "DDA_CS_REV",
             "DDA_CS", "DD")
_BWD2_INPUTS = ("dout", "q", "k", "v", "q_bias", "k_bias", "mimo_v", "states", "qk_dot", "da_cs", "da_cs_rev",
                "dt", "trap", "segsum", "angles", "mimo_o", "d")
_BWD2_OUT_FIELDS = {"DQ": "dq", "DK": "dk", "DV": "dv", "DMIMO_V": "dmimo_v", "DANGLES": "dangles",
                    "DFACTOR": "dfactor", "DGAMMA": "dgamma", "DDA": "dda", "DSSDA": "dssda",
                    "DDA_CS_REV": "dda_cs_rev", "DDA_CS": "dda_cs", "DD": "dd"}


def _aligned(x: Tensor) -> Tensor:
    """Contiguous and 16-byte aligned (a copy when a view starts inside a row)."""
    x = x.contiguous()
    return x if x.data_ptr() % 16 == 0 else x.clone()


def _make_bwd2_args(dims, C, rd, out_f32, t: dict, outs: dict, workspace=None, ws_bytes=0):
    B, S, H, G, R, N, P = dims
    a = _lib.MimoBwdBwdArgs()
    a.B, a.S, a.H, a.G, a.R, a.N, a.P = B, S, H, G, R, N, P
    a.chunk_size, a.rotary_dim_divisor, a.out_f32 = C, rd, int(out_f32)
    for name in _BWD2_INPUTS:
        x = t.get(name)
        setattr(a, name, None if x is None else x.data_ptr())
    for key, field in _BWD2_OUT_FIELDS.items():
        x = outs.get(key)
        setattr(a, field, None if x is None else x.data_ptr())
    a.workspace = None if workspace is None else workspace.data_ptr()
    a.workspace_bytes = ws_bytes
    return a


def mamba3_mimo_bwd_bwd(dout, q, k, v, q_bias, k_bias, mimo_v, states, qk_dot, da_cs, da_cs_rev, dt, trap,
                        segsum, angles, mimo_o=None, d=None, chunk_size: int = 16, rotary_dim_divisor: int = 4,
                        output_dtype=None, *, workspace: Optional[Tensor] = None) -> dict:
    """Stage-2 backward of the MIMO scan: the twelve gradients (dict keys DQ, DK, DV,
    DMIMO_V, DANGLES, DFACTOR, DGAMMA, DDA, DSSDA, DDA_CS_REV, DDA_CS, DD) of
    sum(dPhiO * y) given the first stage's ``states`` and ``qk_dot``. DQ, DK
    [B, S*R, H, N] and DV take q's dtype (bf16) unless ``output_dtype=torch.float32``;
    the others are float32; DD is None without ``d``. Asynchronous on the current
    HIP stream."""
    _validate_inputs(dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, None, None, angles, da_cs, da_cs_rev,
                     dt, trap, d, segsum, chunk_size, rotary_dim_divisor)
    B, S, R, G, N = q.shape
    H, P = v.shape[2:]
    C = int(chunk_size)
    nc = (S + C - 1) // C
    dev = q.device
    _check_tensor("states", states, (B, H, nc, N, P), torch.bfloat16, dev)
    _check_tensor("qk_dot", qk_dot, (B, H, S, R, R), torch.bfloat16, dev)
    if output_dtype not in (None, torch.bfloat16, torch.float32):
        raise TypeError("output_dtype must be None, torch.bfloat16 or torch.float32")
    out_f32 = output_dtype == torch.float32
    odt = torch.float32 if out_f32 else torch.bfloat16
    L = _lib.lib()
    vals = (dout, q, k, v, q_bias, k_bias, mimo_v, states, qk_dot, da_cs, da_cs_rev, dt, trap, segsum, angles,
            mimo_o, d)
    t = {n: (None if x is None else _aligned(x)) for n, x in zip(_BWD2_INPUTS, vals)}
    f32 = torch.float32
    W = N // rotary_dim_divisor
    outs = {
        "DQ": torch.empty((B, S * R, H, N), dtype=odt, device=dev),
        "DK": torch.empty((B, S * R, H, N), dtype=odt, device=dev),
        "DV": torch.empty((B, S, H, P), dtype=odt, device=dev),
        "DMIMO_V": torch.empty((B, H, R, P), dtype=f32, device=dev),
        "DANGLES": torch.empty((B, S, H, W), dtype=f32, device=dev),
        "DFACTOR": torch.empty((B, H, S), dtype=f32, device=dev),
        "DGAMMA": torch.empty((B, H, S), dtype=f32, device=dev),
        "DDA": torch.empty((B, H, S), dtype=f32, device=dev),
        "DSSDA": torch.empty((B, H, nc, C, C), dtype=f32, device=dev),
        "DDA_CS_REV": torch.empty((B, H, S), dtype=f32, device=dev),
        "DDA_CS": torch.empty((B, H, S), dtype=f32, device=dev),
        "DD": torch.empty((B, H), dtype=f32, device=dev) if d is not None else None,
    }
    args = _make_bwd2_args((B, S, H, G, R, N, P), C, int(rotary_dim_divisor), out_f32, t, outs)
    need = ctypes.c_size_t(0)
    st = L.mimo_bwd_bwd_workspace_size(ctypes.byref(args), ctypes.byref(need))
    if st != _lib.MIMO_OK:
        _raise(st)
    if need.value > 0:
        if workspace is None or workspace.numel() < need.value:
            workspace = torch.empty(int(need.value), dtype=torch.uint8, device=dev)
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = L.mimo_bwd_bwd(ctypes.byref(args), ctypes.c_void_p(stream))
    if st != _lib.MIMO_OK:
        _raise(st)
    return outs
