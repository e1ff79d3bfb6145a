"""ctypes view of the C ABI in include/attn_varlen.h.

Loads the in-tree ``libragged_gqa_attn.so``; raises if it has not been built.
There is no fallback implementation: every step runs in the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import threading

from .build import LIB_PATH

ATTN_OK = 0
ATTN_INVALID_ARG = -1
ATTN_UNSUPPORTED = -2
ATTN_MISALIGNED = -3
ATTN_WORKSPACE_TOO_SMALL = -4
ATTN_HIP_ERROR = -5
ATTN_BAD_SEQLENS = -6

ATTN_F16 = 0
ATTN_BF16 = 1

ATTN_FLAG_ALL_KEYS = 1   # evaluate every key, also where P is exactly 0

NOALLOC_SCRATCH_BYTES = 256 << 20   # ATTN_NOALLOC_SCRATCH_BYTES

ENTRY_FWD = 0
ENTRY_BWD = 1
ENTRY_FULL_VJP = 2

# phases of the full-VJP call, in launch order
PHASES = ("plan", "fwd", "dkdv", "dq")

EXPORTED = (
    "attn_varlen_workspace_size",
    "attn_varlen_workspace_size_ds",
    "attn_varlen_fwd",
    "attn_varlen_bwd",
    "attn_varlen_full_vjp",
    "attn_varlen_full_vjp_timed",
    "attn_varlen_full_vjp_noalloc",
    "attn_varlen_check_plan",
    "attn_varlen_key_steps",
    "attn_status_string",
    "attn_last_error",
)


class AttnTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p),
                ("tok_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64)]


class AttnProblem(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32),
                ("batch", ctypes.c_int32),
                ("hq", ctypes.c_int32),
                ("hkv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32),
                ("total_q", ctypes.c_int64),
                ("total_k", ctypes.c_int64),
                ("cu_q", ctypes.c_void_p),
                ("cu_k", ctypes.c_void_p),
                ("alibi_slopes", ctypes.c_void_p),
                ("slopes_stride", ctypes.c_int64),
                ("causal", ctypes.c_int32),
                ("window_left", ctypes.c_int32),
                ("window_right", ctypes.c_int32),
                ("softcap", ctypes.c_float),
                ("scale_multiplier", ctypes.c_float),
                ("flags", ctypes.c_int32),
                ("dropout_p", ctypes.c_float),
                ("dropout_seed", ctypes.c_uint64),
                ("dropout_rates", ctypes.c_void_p)]


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lock = threading.Lock()
_lib = None


def lib_path() -> str:
    return os.environ.get("RAGGED_GQA_ATTN_LIB", LIB_PATH)


def load() -> ctypes.CDLL:
    """The loaded library, with argument types declared.  Raises if it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"HIP library {path} is not built; run __graft_entry__.build() or "
                "python -m ragged_gqa_attention_amd.build")
        lib = ctypes.CDLL(path)
        P = ctypes.POINTER
        T = P(AttnTensor)
        vp, sz, fp = ctypes.c_void_p, ctypes.c_size_t, P(ctypes.c_float)
        lib.attn_varlen_workspace_size.argtypes = [P(AttnProblem), ctypes.c_int, P(sz)]
        i32p = P(ctypes.c_int32)
        lib.attn_varlen_workspace_size_ds.argtypes = [P(AttnProblem), ctypes.c_int, i32p, i32p,
                                                      P(sz)]
        lib.attn_varlen_fwd.argtypes = [P(AttnProblem), T, T, T, T, fp, vp, sz, vp]
        lib.attn_varlen_bwd.argtypes = [P(AttnProblem), T, T, T, T, fp, T, T, T, T, vp, sz, vp]
        lib.attn_varlen_full_vjp.argtypes = [P(AttnProblem), T, T, T, T, T, T, T, T, fp,
                                             vp, sz, vp]
        lib.attn_varlen_full_vjp_timed.argtypes = lib.attn_varlen_full_vjp.argtypes + [
            P(ctypes.c_void_p)]
        lib.attn_varlen_full_vjp_noalloc.argtypes = [P(AttnProblem), T, T, T, T, T, T, T, T, fp,
                                                     vp]
        lib.attn_varlen_check_plan.argtypes = [vp, vp]
        lib.attn_varlen_key_steps.argtypes = [P(AttnProblem), ctypes.c_int, vp, i32p,
                                              ctypes.c_int64, vp]
        lib.attn_status_string.argtypes = [ctypes.c_int]
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_last_error.argtypes = []
        lib.attn_last_error.restype = ctypes.c_char_p
        for name in ("attn_varlen_workspace_size", "attn_varlen_workspace_size_ds",
                     "attn_varlen_fwd", "attn_varlen_bwd",
                     "attn_varlen_full_vjp", "attn_varlen_full_vjp_timed",
                     "attn_varlen_full_vjp_noalloc",
                     "attn_varlen_check_plan", "attn_varlen_key_steps"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
        return lib


def raise_for(status: int, what: str) -> None:
    if status == ATTN_OK:
        return
    lib = load()
    text = lib.attn_status_string(status).decode()
    detail = lib.attn_last_error().decode()
    msg = f"{what}: {text}" + (f" ({detail})" if detail else "")
    if status in (ATTN_INVALID_ARG, ATTN_MISALIGNED, ATTN_WORKSPACE_TOO_SMALL, ATTN_BAD_SEQLENS):
        err = ValueError(msg)
    elif status == ATTN_UNSUPPORTED:
        err = NotImplementedError(msg)
    else:
        err = AttnError(status, msg)
    err.status = status
    raise err
