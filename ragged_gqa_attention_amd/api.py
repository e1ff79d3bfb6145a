"""Python entry points over the C ABI (argument marshalling only).

``attention_varlen_feature_full_vjp`` keeps the signature of page "Noncausal
Global Extreme-GQA Ragged Attention Full VJP", section "Hard Constraints":
(q, k, v, cu_q, cu_k, alibi_slopes, dout, causal, window_left, window_right,
softcap, scale_multiplier) -> (out, dq, dk, dv).  Tensors are device tensors;
torch only provides memory and the current stream.  Every step of the
computation runs in the HIP library.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

HEAD_DIMS = (64, 128, 160)
_DTYPES = {torch.float16: _lib.ATTN_F16, torch.bfloat16: _lib.ATTN_BF16}


def _view(t: torch.Tensor, name: str, dtype, heads=None, dim=None) -> _lib.AttnTensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.dim() != 3 or (dim is not None and t.shape[2] != dim):
        raise ValueError(f"{name} must be [tokens, heads, {dim}], got {tuple(t.shape)}")
    if heads is not None and t.shape[1] != heads:
        raise ValueError(f"{name} has {t.shape[1]} heads, expected {heads}")
    if t.shape[0] > 0 and t.stride(2) != 1:
        raise ValueError(f"{name} must have a contiguous feature axis")
    return _lib.AttnTensor(t.data_ptr(), t.stride(0), t.stride(1))


def make_problem(q, k, cu_q, cu_k, alibi_slopes, causal, window_left, window_right,
                 softcap, scale_multiplier, all_keys=False, dropout_p=0.0, dropout_seed=0,
                 dropout_rates=None) -> _lib.AttnProblem:
    """``all_keys``: evaluate every key, also the far ones whose P is exactly
    zero (the library skips those by default; results are bitwise the same).
    Dropout: a rate ``dropout_p`` in [0, 1) or per-row rates ``dropout_rates``
    (float32 GPU tensor [Tq, Hq], contiguous) with ``dropout_seed`` (see the
    header's "Dropout")."""
    if q.dtype not in _DTYPES:
        raise NotImplementedError(f"dtype {q.dtype} is not supported (FP16 / BF16 only)")
    if q.dim() != 3 or k.dim() != 3 or k.shape[2] != q.shape[2]:
        raise ValueError("q [Tq, Hq, D] and k [Tk, Hkv, D] must share D")
    for name, cu in (("cu_q", cu_q), ("cu_k", cu_k)):
        if cu.dtype != torch.int32 or cu.dim() != 1 or cu.device.type != "cuda":
            raise ValueError(f"{name} must be an int32 GPU vector")
        if not cu.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if cu_q.numel() != cu_k.numel() or cu_q.numel() < 1:
        raise ValueError("cu_q and cu_k must both hold batch + 1 offsets")
    batch = cu_q.numel() - 1
    hq = q.shape[1]
    for name, w in (("window_left", window_left), ("window_right", window_right)):
        if not -1 <= int(w) <= 2**31 - 1:
            raise ValueError(f"{name} must lie in [-1, 2**31 - 1] (got {w})")
    if (alibi_slopes.dtype != torch.float32 or alibi_slopes.device.type != "cuda"
            or alibi_slopes.dim() != 2 or tuple(alibi_slopes.shape) != (batch, hq)
            or (batch > 0 and alibi_slopes.stride(1) != 1)):
        raise ValueError(f"alibi_slopes must be a float32 GPU tensor [{batch}, {hq}] "
                         "with contiguous rows")
    if dropout_rates is not None:
        if (dropout_rates.dtype != torch.float32 or dropout_rates.device.type != "cuda"
                or tuple(dropout_rates.shape) != (q.shape[0], hq)
                or not dropout_rates.is_contiguous()):
            raise ValueError(f"dropout_rates must be a contiguous float32 GPU tensor "
                             f"[{q.shape[0]}, {hq}]")
    if not 0.0 <= float(dropout_p) < 1.0:
        raise ValueError("dropout_p must lie in [0, 1)")
    return _lib.AttnProblem(
        dropout_p=float(dropout_p), dropout_seed=int(dropout_seed) & (2**64 - 1),
        dropout_rates=dropout_rates.data_ptr() if dropout_rates is not None else None,
        dtype=_DTYPES[q.dtype], batch=batch, hq=hq, hkv=k.shape[1], head_dim=q.shape[2],
        total_q=q.shape[0], total_k=k.shape[0],
        cu_q=cu_q.data_ptr(), cu_k=cu_k.data_ptr(),
        alibi_slopes=alibi_slopes.data_ptr(),
        slopes_stride=alibi_slopes.stride(0) if batch > 0 else hq,
        causal=int(bool(causal)), window_left=int(window_left), window_right=int(window_right),
        softcap=float(softcap), scale_multiplier=float(scale_multiplier),
        flags=_lib.ATTN_FLAG_ALL_KEYS if all_keys else 0)


def workspace_size(problem: _lib.AttnProblem, entry: int, cu_q=None, cu_k=None) -> int:
    """Minimum workspace bytes; with cu_q / cu_k (copied to the host, which
    synchronises) the size at which the backward stores dS for every sequence."""
    n = ctypes.c_size_t(0)
    lib = _lib.load()
    if cu_q is None:
        st = lib.attn_varlen_workspace_size(ctypes.byref(problem), entry, ctypes.byref(n))
        _lib.raise_for(st, "attn_varlen_workspace_size")
        return n.value
    hq = cu_q.detach().to("cpu", torch.int32).contiguous()
    hk = cu_k.detach().to("cpu", torch.int32).contiguous()
    i32p = ctypes.POINTER(ctypes.c_int32)
    st = lib.attn_varlen_workspace_size_ds(ctypes.byref(problem), entry,
                                           ctypes.cast(hq.data_ptr(), i32p),
                                           ctypes.cast(hk.data_ptr(), i32p), ctypes.byref(n))
    _lib.raise_for(st, "attn_varlen_workspace_size_ds")
    return n.value


# Default cap on the workspace bytes spent on stored dS (see
# attn_varlen_workspace_size_ds); sequences beyond it recompute dS in dQ.
DS_DEFAULT_BUDGET = 8 << 30


def _bwd_workspace_size(problem, entry, cu_q, cu_k, store_ds) -> int:
    """store_ds: False (the default everywhere: the minimum workspace, linear
    in tokens, sized from host-known shapes only), True (room for every
    sequence's dS up to DS_DEFAULT_BUDGET bytes; reads cu_q / cu_k back to the
    host, which synchronises) or a number of extra bytes beyond the minimum."""
    base = workspace_size(problem, entry)
    if store_ds is True:
        return min(workspace_size(problem, entry, cu_q, cu_k), base + DS_DEFAULT_BUDGET)
    return base + (0 if store_ds is False or store_ds is None else int(store_ds))


def _workspace(nbytes: int, device, ws=None) -> torch.Tensor:
    if ws is not None:
        if ws.device != device or ws.dtype != torch.uint8 or ws.numel() < nbytes:
            raise ValueError("workspace tensor is too small or on the wrong device")
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _fptr(t):
    return ctypes.cast(t.data_ptr(), ctypes.POINTER(ctypes.c_float)) if t is not None else None


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_plan(ws, device):
    _lib.raise_for(_lib.load().attn_varlen_check_plan(ctypes.c_void_p(ws.data_ptr()),
                                                      _stream(device)),
                   "cu_q / cu_k check")


def attn_varlen_fwd(q, k, v, cu_q, cu_k, alibi_slopes, softcap=3.0, scale_multiplier=0.75,
                    causal=False, window_left=-1, window_right=-1, *, out=None, lse=None,
                    workspace=None, check=False, all_keys=False, dropout_p=0.0, dropout_seed=0,
                    dropout_rates=None):
    """Forward only: returns (out [Tq,Hq,D] like q, lse float32 [Tq,Hq])."""
    prob = make_problem(q, k, cu_q, cu_k, alibi_slopes, causal, window_left, window_right,
                        softcap, scale_multiplier, all_keys, dropout_p, dropout_seed,
                        dropout_rates)
    d = q.shape[2]
    tq, tk = _view(q, "q", q.dtype, dim=d), _view(k, "k", q.dtype, dim=d)
    tv = _view(v, "v", q.dtype, heads=k.shape[1], dim=d)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(q.shape[:2]) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [Tq, Hq] tensor")
    to = _view(out, "out", q.dtype, heads=q.shape[1], dim=d)
    ws = _workspace(workspace_size(prob, _lib.ENTRY_FWD), q.device, workspace)
    st = _lib.load().attn_varlen_fwd(ctypes.byref(prob), ctypes.byref(tq), ctypes.byref(tk),
                                     ctypes.byref(tv), ctypes.byref(to), _fptr(lse),
                                     ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                     _stream(q.device))
    _lib.raise_for(st, "attn_varlen_fwd")
    if check:
        _check_plan(ws, q.device)
    return out, lse


def attn_varlen_bwd(q, k, v, out, lse, dout, cu_q, cu_k, alibi_slopes, softcap=3.0,
                    scale_multiplier=0.75, causal=False, window_left=-1, window_right=-1, *,
                    dq=None, dk=None, dv=None, workspace=None, check=False, store_ds=False,
                    all_keys=False, dropout_p=0.0, dropout_seed=0, dropout_rates=None):
    """Backward from a saved forward: returns (dq, dk, dv).  ``store_ds``: see
    _bwd_workspace_size (ignored when ``workspace`` is given: its size decides).
    The dropout arguments must be those of the forward."""
    prob = make_problem(q, k, cu_q, cu_k, alibi_slopes, causal, window_left, window_right,
                        softcap, scale_multiplier, all_keys, dropout_p, dropout_seed,
                        dropout_rates)
    dt, d = q.dtype, q.shape[2]
    tq, tk = _view(q, "q", dt, dim=d), _view(k, "k", dt, dim=d)
    tv = _view(v, "v", dt, heads=k.shape[1], dim=d)
    to = _view(out, "out", dt, heads=q.shape[1], dim=d)
    tdo = _view(dout, "dout", dt, heads=q.shape[1], dim=d)
    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(q.shape[:2]) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [Tq, Hq] tensor")
    dq = torch.empty(q.shape, dtype=dt, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=dt, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=dt, device=q.device) if dv is None else dv
    tdq = _view(dq, "dq", dt, heads=q.shape[1], dim=d)
    tdk = _view(dk, "dk", dt, heads=k.shape[1], dim=d)
    tdv = _view(dv, "dv", dt, heads=k.shape[1], dim=d)
    if workspace is None:
        ws = _workspace(_bwd_workspace_size(prob, _lib.ENTRY_BWD, cu_q, cu_k, store_ds), q.device)
    else:
        ws = _workspace(workspace_size(prob, _lib.ENTRY_BWD), q.device, workspace)
    st = _lib.load().attn_varlen_bwd(ctypes.byref(prob), ctypes.byref(tq), ctypes.byref(tk),
                                     ctypes.byref(tv), ctypes.byref(to), _fptr(lse),
                                     ctypes.byref(tdo), ctypes.byref(tdq), ctypes.byref(tdk),
                                     ctypes.byref(tdv), ctypes.c_void_p(ws.data_ptr()),
                                     ws.numel(), _stream(q.device))
    _lib.raise_for(st, "attn_varlen_bwd")
    if check:
        _check_plan(ws, q.device)
    return dq, dk, dv


class FullVJP:
    """Pre-bound forward + full VJP call with preallocated outputs and workspace.

    Binding once and calling many times keeps the timed region to the library
    call itself.  Outputs are dense [Tq,Hq,160] / [Tk,1,160] tensors.
    ``store_ds`` sizes the workspace (see _bwd_workspace_size); the default
    is the minimum workspace, and True reads cu_q / cu_k back to the host
    once, here, to give every sequence's dS a place.
    """

    def __init__(self, q, k, v, cu_q, cu_k, alibi_slopes, dout, causal=False, window_left=-1,
                 window_right=-1, softcap=3.0, scale_multiplier=0.75, *, want_lse=False,
                 store_ds=False, all_keys=False, dropout_p=0.0, dropout_seed=0,
                 dropout_rates=None):
        self.prob = make_problem(q, k, cu_q, cu_k, alibi_slopes, causal, window_left,
                                 window_right, softcap, scale_multiplier, all_keys, dropout_p,
                                 dropout_seed, dropout_rates)
        dt, dev = q.dtype, q.device
        self.inputs = (q, k, v, dout, cu_q, cu_k, alibi_slopes, dropout_rates)   # keep alive
        self.out = torch.empty(q.shape, dtype=dt, device=dev)
        self.dq = torch.empty(q.shape, dtype=dt, device=dev)
        self.dk = torch.empty(k.shape, dtype=dt, device=dev)
        self.dv = torch.empty(v.shape, dtype=dt, device=dev)
        self.lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev) if want_lse else None
        d = q.shape[2]
        self.views = [_view(q, "q", dt, dim=d), _view(k, "k", dt, dim=d),
                      _view(v, "v", dt, heads=k.shape[1], dim=d),
                      _view(dout, "dout", dt, heads=q.shape[1], dim=d),
                      _view(self.out, "out", dt, dim=d), _view(self.dq, "dq", dt, dim=d),
                      _view(self.dk, "dk", dt, dim=d), _view(self.dv, "dv", dt, dim=d)]
        self.ws = _workspace(_bwd_workspace_size(self.prob, _lib.ENTRY_FULL_VJP, cu_q, cu_k,
                                                 store_ds), dev)
        self.device = dev
        self._fn = _lib.load().attn_varlen_full_vjp
        self._fn_timed = _lib.load().attn_varlen_full_vjp_timed

    def __call__(self, stream=None, events=None):
        """Enqueue one call.  ``events``: optional list of len(PHASES) + 1 recorded
        torch.cuda.Event(enable_timing=True); event i brackets the start of phase i."""
        s = ctypes.c_void_p(stream if stream is not None
                            else torch.cuda.current_stream(self.device).cuda_stream)
        args = [ctypes.byref(self.prob)] + [ctypes.byref(t) for t in self.views] + [
            _fptr(self.lse), ctypes.c_void_p(self.ws.data_ptr()), self.ws.numel(), s]
        if events is None:
            st = self._fn(*args)
        else:
            if len(events) != len(_lib.PHASES) + 1:
                raise ValueError("need one event per phase plus a final one")
            handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
            st = self._fn_timed(*args, handles)
        _lib.raise_for(st, "attn_varlen_full_vjp")
        return self.out, self.dq, self.dk, self.dv

    def check_plan(self):
        _check_plan(self.ws, self.device)

    def key_steps(self):
        """Key-step ranges the last call visited (see key_steps)."""
        return key_steps(self.prob, _lib.ENTRY_FULL_VJP, self.ws, self.inputs[4])


def attn_varlen_full_vjp(q, k, v, cu_q, cu_k, alibi_slopes, dout, softcap=3.0,
                         scale_multiplier=0.75, causal=False, window_left=-1, window_right=-1,
                         *, want_lse=False, check=False, store_ds=False, all_keys=False,
                         dropout_p=0.0, dropout_seed=0, dropout_rates=None):
    """Forward + full VJP: returns (out, dq, dk, dv[, lse]).  With the default
    store_ds=False nothing synchronises the host: the workspace size depends
    only on the tensors' shapes and dQ recomputes dS."""
    call = FullVJP(q, k, v, cu_q, cu_k, alibi_slopes, dout, causal, window_left, window_right,
                   softcap, scale_multiplier, want_lse=want_lse, store_ds=store_ds,
                   all_keys=all_keys, dropout_p=dropout_p, dropout_seed=dropout_seed,
                   dropout_rates=dropout_rates)
    res = call()
    if check:
        call.check_plan()
    return res + ((call.lse,) if want_lse else ())


def key_steps(problem: _lib.AttnProblem, entry: int, ws: torch.Tensor, cu_q) -> "np.ndarray":
    """int32 [n_tiles, 2]: per 256-row tile of folded rows (row h * Lq + i of a
    sequence's group of hq / hkv heads sharing a K/V head; tiles in batch order,
    the K/V heads of a sequence in turn) the first and one past the last 64-key
    step the last call of ``entry`` on workspace ``ws`` visited.  Synchronises."""
    import numpy as np
    cq = cu_q.detach().to("cpu", torch.int64)
    lq = (cq[1:] - cq[:-1]).numpy()
    group = problem.hq // problem.hkv
    n = int(((lq * group + 255) // 256).sum()) * problem.hkv if lq.size else 0
    out = np.zeros((n, 2), dtype=np.int32)
    st = _lib.load().attn_varlen_key_steps(
        ctypes.byref(problem), entry, ctypes.c_void_p(ws.data_ptr()),
        out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n, _stream(ws.device))
    _lib.raise_for(st, "attn_varlen_key_steps")
    return out


def attention_varlen_feature_full_vjp(q, k, v, cu_q, cu_k, alibi_slopes, dout, causal,
                                      window_left, window_right, softcap, scale_multiplier):
    """The page's entry point: returns (out, dq, dk, dv), dense, in the inputs'
    dtype.  It never synchronises the host (minimum workspace, see
    attn_varlen_full_vjp); callers that want dQ from stored dS bind a FullVJP
    with store_ds=True."""
    return attn_varlen_full_vjp(q, k, v, cu_q, cu_k, alibi_slopes, dout, softcap=softcap,
                                scale_multiplier=scale_multiplier, causal=causal,
                                window_left=window_left, window_right=window_right)
