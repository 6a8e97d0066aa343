"""ctypes view of the C ABI in include/mimo_bwd_fwd.h.

Only argument marshalling lives here. The shared library is the in-tree
build (``mamba_mimo_chunked_amd/_build/libmimo_bwd_fwd.so``); when it is
missing the import of this module's ``lib()`` raises, there is no fallback.
"""

from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "_build" / "libmimo_bwd_fwd.so"

MIMO_OK, MIMO_ERR_VALUE, MIMO_ERR_TYPE, MIMO_ERR_UNSUPPORTED, MIMO_ERR_HIP = range(5)
ABI_VERSION = 2

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)


class MimoBwdFwdArgs(ctypes.Structure):
    """Mirror of ``mimo_bwd_fwd_args`` (field order and types must match)."""

    _fields_ = [
        ("B", ctypes.c_int64), ("S", ctypes.c_int64), ("H", ctypes.c_int64), ("G", ctypes.c_int64),
        ("R", ctypes.c_int64), ("N", ctypes.c_int64), ("P", ctypes.c_int64),
        ("chunk_size", ctypes.c_int32), ("rotary_dim_divisor", ctypes.c_int32),
        ("dout", ctypes.c_void_p), ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("q_bias", ctypes.c_void_p), ("k_bias", ctypes.c_void_p), ("mimo_v", ctypes.c_void_p),
        ("mimo_o", ctypes.c_void_p),
        ("z", ctypes.c_void_p),
        ("mimo_z", ctypes.c_void_p),
        ("angles", ctypes.c_void_p), ("da_cs", ctypes.c_void_p), ("da_cs_rev", ctypes.c_void_p),
        ("dt", ctypes.c_void_p),
        ("trap", ctypes.c_void_p),
        ("d", ctypes.c_void_p),
        ("segsum", ctypes.c_void_p),
        ("dmimo_o", ctypes.c_void_p),
        ("states", ctypes.c_void_p),
        ("dz", ctypes.c_void_p),
        ("dmimo_z", ctypes.c_void_p),
        ("qk_dot", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class MimoFwdArgs(ctypes.Structure):
    """Mirror of ``mimo_fwd_args`` (field order and types must match)."""

    _fields_ = [
        ("B", ctypes.c_int64), ("S", ctypes.c_int64), ("H", ctypes.c_int64), ("G", ctypes.c_int64),
        ("R", ctypes.c_int64), ("N", ctypes.c_int64), ("P", ctypes.c_int64),
        ("chunk_size", ctypes.c_int32), ("rotary_dim_divisor", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("q_bias", ctypes.c_void_p), ("k_bias", ctypes.c_void_p), ("mimo_v", ctypes.c_void_p),
        ("mimo_o", ctypes.c_void_p),
        ("z", ctypes.c_void_p),
        ("mimo_z", ctypes.c_void_p),
        ("angles", ctypes.c_void_p), ("da_cs", ctypes.c_void_p), ("da_cs_rev", ctypes.c_void_p),
        ("dt", ctypes.c_void_p),
        ("trap", ctypes.c_void_p),
        ("d", ctypes.c_void_p),
        ("segsum", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class MimoSisoFwdArgs(ctypes.Structure):
    """Mirror of ``mimo_siso_fwd_args`` (field order and types must match)."""

    _fields_ = [
        ("B", ctypes.c_int64), ("S", ctypes.c_int64), ("Hq", ctypes.c_int64), ("H", ctypes.c_int64),
        ("K", ctypes.c_int64), ("V", ctypes.c_int64),
        ("chunk_size", ctypes.c_int32), ("A", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("adt", ctypes.c_void_p), ("dt", ctypes.c_void_p), ("trap", ctypes.c_void_p),
        ("q_bias", ctypes.c_void_p), ("k_bias", ctypes.c_void_p), ("angles", ctypes.c_void_p),
        ("d", ctypes.c_void_p),
        ("z", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class MimoBwdBwdArgs(ctypes.Structure):
    """Mirror of ``mimo_bwd_bwd_args`` (field order and types must match)."""

    _fields_ = [
        ("B", ctypes.c_int64), ("S", ctypes.c_int64), ("H", ctypes.c_int64), ("G", ctypes.c_int64),
        ("R", ctypes.c_int64), ("N", ctypes.c_int64), ("P", ctypes.c_int64),
        ("chunk_size", ctypes.c_int32), ("rotary_dim_divisor", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("dout", ctypes.c_void_p), ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("q_bias", ctypes.c_void_p), ("k_bias", ctypes.c_void_p), ("mimo_v", ctypes.c_void_p),
        ("states", ctypes.c_void_p), ("qk_dot", ctypes.c_void_p),
        ("da_cs", ctypes.c_void_p), ("da_cs_rev", ctypes.c_void_p), ("dt", ctypes.c_void_p),
        ("trap", ctypes.c_void_p),
        ("segsum", ctypes.c_void_p), ("angles", ctypes.c_void_p),
        ("mimo_o", ctypes.c_void_p),
        ("d", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("dmimo_v", ctypes.c_void_p), ("dangles", ctypes.c_void_p), ("dfactor", ctypes.c_void_p),
        ("dgamma", ctypes.c_void_p), ("dda", ctypes.c_void_p), ("dssda", ctypes.c_void_p),
        ("dda_cs_rev", ctypes.c_void_p), ("dda_cs", ctypes.c_void_p),
        ("dd", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


DTYPE_BF16, DTYPE_FP16, DTYPE_FP32 = 0, 1, 2

EXPORTED = ("mimo_bwd_fwd", "mimo_bwd_fwd_timed", "mimo_bwd_fwd_workspace_size", "mimo_fwd",
            "mimo_fwd_timed", "mimo_fwd_workspace_size", "mimo_bwd_fwd_f32", "mimo_bwd_fwd_f32_timed",
            "mimo_bwd_fwd_f32_workspace_size", "mimo_fwd_f32", "mimo_fwd_f32_workspace_size",
            "mimo_siso_fwd", "mimo_siso_fwd_timed", "mimo_siso_fwd_workspace_size", "mimo_bwd_bwd",
            "mimo_bwd_bwd_timed", "mimo_bwd_bwd_workspace_size", "mimo_last_error", "mimo_abi_version",
            "mimo_bwd_fwd_noalloc")
NOALLOC_SCRATCH_BYTES = 64 << 20
TIMED_EVENTS = 5

_lib = None


def lib():
    """Load the HIP library (once). Raises ImportError if it has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m mamba_mimo_chunked_amd.build` "
                "(or __graft_entry__.build()); there is no fallback implementation")
        L = ctypes.CDLL(str(LIB_PATH))
        argp = ctypes.POINTER(MimoBwdFwdArgs)
        L.mimo_bwd_fwd.argtypes = [argp, ctypes.c_void_p]
        L.mimo_bwd_fwd.restype = ctypes.c_int
        L.mimo_bwd_fwd_timed.argtypes = [argp, ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
        L.mimo_bwd_fwd_timed.restype = ctypes.c_int
        L.mimo_bwd_fwd_workspace_size.argtypes = [argp, ctypes.POINTER(ctypes.c_size_t)]
        L.mimo_bwd_fwd_workspace_size.restype = ctypes.c_int
        L.mimo_bwd_fwd_noalloc.argtypes = [argp, ctypes.c_void_p]
        L.mimo_bwd_fwd_noalloc.restype = ctypes.c_int
        fargp = ctypes.POINTER(MimoFwdArgs)
        L.mimo_fwd.argtypes = [fargp, ctypes.c_void_p]
        L.mimo_fwd.restype = ctypes.c_int
        L.mimo_fwd_timed.argtypes = [fargp, ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
        L.mimo_fwd_timed.restype = ctypes.c_int
        L.mimo_fwd_workspace_size.argtypes = [fargp, ctypes.POINTER(ctypes.c_size_t)]
        L.mimo_fwd_workspace_size.restype = ctypes.c_int
        evp = ctypes.POINTER(ctypes.c_void_p)
        szp = ctypes.POINTER(ctypes.c_size_t)
        for name, ap in (("mimo_bwd_fwd_f32", argp), ("mimo_fwd_f32", fargp)):
            getattr(L, name).argtypes = [ap, ctypes.c_void_p]
            getattr(L, name).restype = ctypes.c_int
            getattr(L, name + "_workspace_size").argtypes = [ap, szp]
            getattr(L, name + "_workspace_size").restype = ctypes.c_int
        L.mimo_bwd_fwd_f32_timed.argtypes = [argp, ctypes.c_void_p, evp]
        L.mimo_bwd_fwd_f32_timed.restype = ctypes.c_int
        sargp = ctypes.POINTER(MimoSisoFwdArgs)
        L.mimo_siso_fwd.argtypes = [sargp, ctypes.c_void_p]
        L.mimo_siso_fwd.restype = ctypes.c_int
        L.mimo_siso_fwd_timed.argtypes = [sargp, ctypes.c_void_p, evp]
        L.mimo_siso_fwd_timed.restype = ctypes.c_int
        L.mimo_siso_fwd_workspace_size.argtypes = [sargp, szp]
        L.mimo_siso_fwd_workspace_size.restype = ctypes.c_int
        bargp = ctypes.POINTER(MimoBwdBwdArgs)
        L.mimo_bwd_bwd.argtypes = [bargp, ctypes.c_void_p]
        L.mimo_bwd_bwd.restype = ctypes.c_int
        L.mimo_bwd_bwd_timed.argtypes = [bargp, ctypes.c_void_p, evp]
        L.mimo_bwd_bwd_timed.restype = ctypes.c_int
        L.mimo_bwd_bwd_workspace_size.argtypes = [bargp, szp]
        L.mimo_bwd_bwd_workspace_size.restype = ctypes.c_int
        L.mimo_last_error.argtypes = []
        L.mimo_last_error.restype = ctypes.c_char_p
        L.mimo_abi_version.argtypes = []
        L.mimo_abi_version.restype = ctypes.c_int
        if L.mimo_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH}: ABI version {L.mimo_abi_version()} != {ABI_VERSION}")
        _lib = L
    return _lib


def last_error() -> str:
    return lib().mimo_last_error().decode(errors="replace")
