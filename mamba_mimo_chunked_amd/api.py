"""Public Python entry points: ``mamba_mimo_bwd_fwd``, the layer output ``mamba_mimo_fwd``,
their fp32-intermediate variants, the stage-2 backward ``mamba3_mimo_bwd_bwd`` and the SISO
forward ``mamba3_siso_fwd``.

Signature, defaults, output order and error types follow the Triton-Ascend
mamba_mimo_bwd_fwd page (public API module: the output named tuple and the
classes of its input errors; operator document: the input and output tables).
The argument checks here are table-driven: one (name, shape, dtype, branch)
entry per tensor. PyTorch supplies device memory (outputs and the
workspace) and the current stream; every step of the computation runs in the
HIP library behind ``include/mimo_bwd_fwd.h``.
"""

from __future__ import annotations

import ctypes
from functools import lru_cache
from typing import NamedTuple, Optional

import torch

from . import _lib

__all__ = ["MambaMimoBwdFwdOutputs", "mamba_mimo_bwd_fwd", "mamba_mimo_bwd_fwd_noalloc", "mamba_mimo_fwd", "mamba_mimo_bwd_fwd_fp32",
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
    """One argument against its expected shape (ValueError), dtype (TypeError) and device."""
    if tuple(tensor.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(tensor.shape)}")
    if tensor.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {tensor.dtype}")
    if tensor.device != device:
        raise ValueError(f"{name} must be on {device}, got {tensor.device}")


_BF16, _F32 = torch.bfloat16, torch.float32

# When a tensor argument must be present: always, or only on a branch.
_ALWAYS, _IF_REDUCED, _IF_Z, _IF_D = "always", "reduced", "z", "d"


def _sizes(q, v, chunk_size, rotary_dim_divisor, what="mamba_mimo_bwd_fwd", data_dtypes=(_BF16,)):
    """The problem sizes, read from q [B,S,R,G,N] and v [B,S,H,P], after the checks
    that need no other tensor. The order of the checks (rank of q, positive sizes,
    q's dtype, device, architecture, then the size constraints of the operator
    document) is the order the operator's invalid-input tests rely on."""
    if q.dim() != 5:
        raise ValueError("q must have shape [B, S, R, G, N]")
    B, S, R, G, N = (int(x) for x in q.shape)
    if min(B, S, R, G) < 1:
        raise ValueError("B, S, R and G must be positive")
    if q.dtype not in data_dtypes:
        names = " or ".join(str(d) for d in data_dtypes)
        raise TypeError(f"q, k, v, dout and trap must use {names}")
    if q.device.type != "cuda":
        raise ValueError(f"{what} requires GPU (HIP) tensors")
    if not _is_gfx950(q.device.index if q.device.index is not None else torch.cuda.current_device()):
        raise NotImplementedError(f"{what} supports gfx950 (MI355X) devices only")
    C, rd = int(chunk_size), int(rotary_dim_divisor)
    limits = (
        (1 <= C and C * R <= 128, "chunk_size * R must be in [1, 128]"),
        (rd in (2, 4), "rotary_dim_divisor must be 2 or 4"),
        (N % 2 == 0 and N % max(rd, 1) == 0, "N must be even and divisible by rotary_dim_divisor"),
        (N <= 128, "N greater than 128 is not supported"),
        (v.dim() == 4 and tuple(v.shape[:2]) == (B, S), "v must have shape [B, S, H, P]"),
    )
    for ok, msg in limits:
        if not ok:
            raise ValueError(msg)
    H, P = (int(x) for x in v.shape[2:])
    if H % G:
        raise ValueError("H must be divisible by G")
    if P > 128:
        raise ValueError("P greater than 128 is not supported")
    return B, S, H, G, R, N, P, C, rd


def _input_table(B, S, H, G, R, N, P, C, rd, *, reduce_o, with_dout, data=_BF16):
    """(name, expected shape, dtype, when present) of every tensor input but q;
    ``data`` is the dtype of the data tensors (k, v, trap, z, dout)."""
    nc = (S + C - 1) // C
    dout_shape = (B, S, H, P) if reduce_o else (B, S, R, H, P)
    table = [
        ("k", (B, S, R, G, N), data, _ALWAYS),
        ("v", (B, S, H, P), data, _ALWAYS),
        ("q_bias", (H, R, N), _F32, _ALWAYS),
        ("k_bias", (H, R, N), _F32, _ALWAYS),
        ("mimo_v", (H, R, P), _F32, _ALWAYS),
        ("angles", (B, S, H, N // rd), _F32, _ALWAYS),
        ("da_cs", (B, H, S), _F32, _ALWAYS),
        ("da_cs_rev", (B, H, S), _F32, _ALWAYS),
        ("dt", (B, H, S), _F32, _ALWAYS),
        ("trap", (B, H, S), data, _ALWAYS),
        ("segsum", (B, H, nc, C, C), _F32, _ALWAYS),
        ("d", (H,), _F32, _IF_D),
        ("mimo_o", (H, R, P), _F32, _IF_REDUCED),
        ("z", (B, S, H, P), data, _IF_Z),
        ("mimo_z", (H, R, P), _F32, _IF_Z),
    ]
    if with_dout:
        table.append(("dout", dout_shape, data, _ALWAYS))
    return table


def _check_table(table, values: dict, device):
    for name, shape, dtype, when in table:
        x = values.get(name)
        if x is None:
            if when == _ALWAYS:
                raise ValueError(f"{name} is required")
            continue
        _check_tensor(name, x, shape, dtype, device)


def _validate_inputs(dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs,
                     da_cs_rev, dt, trap, d, segsum, chunk_size, rotary_dim_divisor, *, fwd=False,
                     what="mamba_mimo_bwd_fwd", data_dtypes=(_BF16,)):
    """Check every argument of the backward first stage (or, with ``fwd``, of the
    layer output, which takes no dout); returns the problem sizes. The data tensors
    take q's dtype, one of ``data_dtypes``."""
    dims = _sizes(q, v, chunk_size, rotary_dim_divisor, what, data_dtypes)
    if (z is None) != (mimo_z is None):
        raise ValueError("z and mimo_z must either both be present or both be None")
    values = dict(dout=dout, k=k, v=v, q_bias=q_bias, k_bias=k_bias, mimo_v=mimo_v, mimo_o=mimo_o,
                  z=z, mimo_z=mimo_z, angles=angles, da_cs=da_cs, da_cs_rev=da_cs_rev, dt=dt,
                  trap=trap, d=d, segsum=segsum)
    _check_table(_input_table(*dims, reduce_o=mimo_o is not None, with_dout=not fwd, data=q.dtype), values,
                 q.device)
    return dims


def _output_table(B, S, H, G, R, N, P, C, rd, *, reduce_o, has_z):
    """(name, shape, dtype, present) of the backward first stage's outputs."""
    nc = (S + C - 1) // C
    return (
        ("dmimo_o", (B, H, R, P), _F32, reduce_o),
        ("states", (B, H, nc, N, P), _BF16, True),
        ("dz", (B, S, H, P), _BF16, has_z),
        ("dmimo_z", (B, H, R, P), _F32, has_z),
        ("qk_dot", (B, H, S, R, R), _BF16, True),
    )


def _check_output(name, x, shape, dtype, device):
    """A caller-supplied output: the library writes it in place, rows of eight bf16
    at a time, so it must be dense and 16-byte aligned."""
    _check_tensor(name, x, shape, dtype, device)
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if x.data_ptr() % 16:
        raise ValueError(f"{name} must be 16-byte aligned")


def _outputs(table, out: Optional[dict], device) -> dict:
    """The output tensors: allocated here, or the caller's, checked against the table."""
    if out is None:
        return {name: (torch.empty(shape, dtype=dtype, device=device) if present else None)
                for name, shape, dtype, present in table}
    unknown = set(out) - {name for name, *_ in table}
    if unknown:
        raise ValueError(f"out has unknown keys {sorted(unknown)}")
    res = {}
    for name, shape, dtype, present in table:
        x = out.get(name)
        if not present:
            if x is not None:
                raise ValueError(f"out[{name!r}] must be None on this branch")
            res[name] = None
            continue
        if x is None:
            raise ValueError(f"out[{name!r}] is required")
        _check_output(f"out[{name!r}]", x, shape, dtype, device)
        res[name] = x
    return res


def _workspace(workspace: Optional[Tensor], need: int, device) -> Optional[Tensor]:
    """A caller's workspace (uint8, dense, on the device, at least ``need`` bytes) or a new one."""
    if need == 0:
        return workspace
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8:
        raise TypeError(f"workspace must have dtype torch.uint8, got {workspace.dtype}")
    if workspace.device != device:
        raise ValueError(f"workspace must be on {device}, got {workspace.device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if workspace.numel() < need:
        raise ValueError(f"workspace too small: need {need} bytes, got {workspace.numel()}")
    return workspace


def _aligned(x: Optional[Tensor]) -> Optional[Tensor]:
    """Contiguous and 16-byte aligned (a copy when a view starts inside a row)."""
    if x is None:
        return None
    x = x.contiguous()
    return x if x.data_ptr() % 16 == 0 else x.clone()


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


def mamba_mimo_bwd_fwd_noalloc(dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs,
                               da_cs_rev, dt, trap, d, segsum, chunk_size: int = 16,
                               rotary_dim_divisor: int = 4, *, out: Optional[dict] = None) -> MambaMimoBwdFwdOutputs:
    """``mamba_mimo_bwd_fwd`` through the library's entry point that allocates nothing
    (``mimo_bwd_fwd_noalloc``): its scratch is a fixed device array inside the library,
    shared by every call on the device, so calls on one device must not overlap.
    Pass ``out`` to allocate nothing on this side either."""
    return _bwd_fwd("mimo_bwd_fwd_noalloc", dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles,
                    da_cs, da_cs_rev, dt, trap, d, segsum, chunk_size, rotary_dim_divisor, out, None)


def _bwd_fwd(fn, dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs, da_cs_rev,
             dt, trap, d, segsum, chunk_size, rotary_dim_divisor, out, workspace):
    dims = _validate_inputs(dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs,
                            da_cs_rev, dt, trap, d, segsum, chunk_size, rotary_dim_divisor)
    B, S, H, G, R, N, P, C, rd = dims
    L = _lib.lib()
    dev = q.device
    t = {name: _aligned(x) for name, x in (
        ("dout", dout), ("q", q), ("k", k), ("v", v), ("q_bias", q_bias), ("k_bias", k_bias),
        ("mimo_v", mimo_v), ("mimo_o", mimo_o), ("z", z), ("mimo_z", mimo_z), ("angles", angles),
        ("da_cs", da_cs), ("da_cs_rev", da_cs_rev), ("dt", dt), ("trap", trap), ("d", d),
        ("segsum", segsum))}
    out = _outputs(_output_table(*dims, reduce_o=mimo_o is not None, has_z=z is not None), out, dev)
    args = _make_args(B, S, H, G, R, N, P, C, rd, t, out)
    if not fn.endswith("_noalloc"):
        need = ctypes.c_size_t(0)
        st = getattr(L, fn + "_workspace_size")(ctypes.byref(args), ctypes.byref(need))
        if st != _lib.MIMO_OK:
            _raise(st)
        workspace = _workspace(workspace, int(need.value), dev)
        if need.value > 0:
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
    dims = _validate_inputs(None, q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs,
                            da_cs_rev, dt, trap, d, segsum, chunk_size, rotary_dim_divisor, fwd=True)
    B, S, H, G, R, N, P, C, rd = dims
    L = _lib.lib()
    dev = q.device
    vals = (q, k, v, q_bias, k_bias, mimo_v, mimo_o, z, mimo_z, angles, da_cs, da_cs_rev, dt, trap, d,
            segsum)
    t = {name: _aligned(x) for name, x in zip(_FWD_INPUTS, vals)}
    shape = (B, S, H, P) if mimo_o is not None else (B, S, R, H, P)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    else:
        _check_output("out", out, shape, torch.bfloat16, dev)
    args = _make_fwd_args(B, S, H, G, R, N, P, C, rd, t, out)
    need = ctypes.c_size_t(0)
    st = getattr(L, fn + "_workspace_size")(ctypes.byref(args), ctypes.byref(need))
    if st != _lib.MIMO_OK:
        _raise(st)
    workspace = _workspace(workspace, int(need.value), dev)
    if need.value > 0:
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
    t = {n: _aligned(x) for n, x in zip(_SISO_INPUTS, vals)}
    if out is None:
        out = torch.empty((B, S, H, V), dtype=q.dtype, device=dev)
    else:
        _check_output("out", out, (B, S, H, V), q.dtype, dev)
    args = _make_siso_args(dims + (int(chunk_size),), q.dtype, t, out)
    need = ctypes.c_size_t(0)
    st = L.mimo_siso_fwd_workspace_size(ctypes.byref(args), ctypes.byref(need))
    if st != _lib.MIMO_OK:
        _raise(st)
    workspace = _workspace(workspace, int(need.value), dev)
    if need.value > 0:
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


def _make_bwd2_args(dims, C, rd, in_dtype: int, out_dtype: int, t: dict, outs: dict, workspace=None, ws_bytes=0):
    """The C argument struct; ``in_dtype`` / ``out_dtype`` are _lib.DTYPE_* codes."""
    B, S, H, G, R, N, P = dims
    a = _lib.MimoBwdBwdArgs()
    a.B, a.S, a.H, a.G, a.R, a.N, a.P = B, S, H, G, R, N, P
    a.chunk_size, a.rotary_dim_divisor = C, rd
    a.in_dtype, a.out_dtype = int(in_dtype), int(out_dtype)
    for name in _BWD2_INPUTS:
        x = t.get(name)
        setattr(a, name, None if x is None else x.data_ptr())
    for key, field in _BWD2_OUT_FIELDS.items():
        x = outs.get(key)
        setattr(a, field, None if x is None else x.data_ptr())
    a.workspace = None if workspace is None else workspace.data_ptr()
    a.workspace_bytes = ws_bytes
    return a


_BWD2_DTYPES = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}   # _lib.DTYPE_* codes


def mamba3_mimo_bwd_bwd(dout, q, k, v, q_bias, k_bias, mimo_v, states, qk_dot, da_cs, da_cs_rev, dt, trap,
                        segsum, angles, mimo_o=None, d=None, chunk_size: int = 16, rotary_dim_divisor: int = 4,
                        output_dtype=None, *, workspace: Optional[Tensor] = None) -> dict:
    """Stage-2 backward of the MIMO scan: the twelve gradients (dict keys DQ, DK, DV,
    DMIMO_V, DANGLES, DFACTOR, DGAMMA, DDA, DSSDA, DDA_CS_REV, DDA_CS, DD) of
    sum(dPhiO * y) given the first stage's ``states`` and ``qk_dot`` (the
    Triton-Ascend mamba3_mimo_bwd_bwd pull request page, migration note). The data
    tensors dout, q, k, v, states, qk_dot and trap share one dtype: bfloat16,
    float16 or float32. DQ, DK [B, S*R, H, N] and DV take that dtype unless
    ``output_dtype`` names another of the three; the others are float32; DD is None
    without ``d``. Asynchronous on the current HIP stream."""
    B, S, H, G, R, N, P, C, rd = _validate_inputs(dout, q, k, v, q_bias, k_bias, mimo_v, mimo_o, None, None,
                                                  angles, da_cs, da_cs_rev, dt, trap, d, segsum, chunk_size,
                                                  rotary_dim_divisor, what="mamba3_mimo_bwd_bwd",
                                                  data_dtypes=tuple(_BWD2_DTYPES))
    nc = (S + C - 1) // C
    dev = q.device
    _check_tensor("states", states, (B, H, nc, N, P), q.dtype, dev)
    _check_tensor("qk_dot", qk_dot, (B, H, S, R, R), q.dtype, dev)
    if output_dtype is not None and output_dtype not in _BWD2_DTYPES:
        raise TypeError("output_dtype must be None, torch.bfloat16, torch.float16 or torch.float32")
    odt = q.dtype if output_dtype is None else output_dtype
    L = _lib.lib()
    vals = (dout, q, k, v, q_bias, k_bias, mimo_v, states, qk_dot, da_cs, da_cs_rev, dt, trap, segsum, angles,
            mimo_o, d)
    t = {n: _aligned(x) for n, x in zip(_BWD2_INPUTS, vals)}
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
    args = _make_bwd2_args((B, S, H, G, R, N, P), C, int(rotary_dim_divisor), _BWD2_DTYPES[q.dtype],
                           _BWD2_DTYPES[odt], t, outs)
    need = ctypes.c_size_t(0)
    st = L.mimo_bwd_bwd_workspace_size(ctypes.byref(args), ctypes.byref(need))
    if st != _lib.MIMO_OK:
        _raise(st)
    workspace = _workspace(workspace, int(need.value), dev)
    if need.value > 0:
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = L.mimo_bwd_bwd(ctypes.byref(args), ctypes.c_void_p(stream))
    if st != _lib.MIMO_OK:
        _raise(st)
    return outs
