"""attn_varlen_full_vjp_noalloc, the entry point that allocates nothing, called
through the C ABI: its outputs equal those of attn_varlen_full_vjp given a
workspace of ATTN_NOALLOC_SCRATCH_BYTES bytes, bit for bit, on two calls in a
row (the second on a smaller problem, so it reuses the scratch the first left
behind), and it rejects problems whose minimum workspace exceeds the array."""
import ctypes

import pytest
import torch

import ragged_gqa_attention_amd as rga
from ragged_gqa_attention_amd import _lib
import workloads as W
from tests.gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu


def _views(g, outs):
    dt = g.q.dtype
    api = rga.api
    return ([api._view(g.q, "q", dt), api._view(g.k, "k", dt), api._view(g.v, "v", dt),
             api._view(g.dout, "dout", dt)] + [api._view(t, n, dt) for n, t in
                                               zip(("out", "dq", "dk", "dv"), outs)])


def _outputs(g):
    dev = g.q.device
    return [torch.full(g.q.shape, float("nan"), dtype=g.q.dtype, device=dev),
            torch.full(g.q.shape, float("nan"), dtype=g.q.dtype, device=dev),
            torch.full(g.k.shape, float("nan"), dtype=g.q.dtype, device=dev),
            torch.full(g.v.shape, float("nan"), dtype=g.q.dtype, device=dev),
            torch.full(g.q.shape[:2], float("nan"), dtype=torch.float32, device=dev)]


def _noalloc(g):
    lib = _lib.load()
    prob = rga.api.make_problem(g.q, g.k, g.cu_q, g.cu_k, g.slopes, False, -1, -1, g.softcap,
                                g.scale_multiplier)
    outs = _outputs(g)
    views = _views(g, outs[:4])
    st = lib.attn_varlen_full_vjp_noalloc(ctypes.byref(prob), *[ctypes.byref(t) for t in views],
                                          rga.api._fptr(outs[4]), rga.api._stream(g.q.device))
    _lib.raise_for(st, "attn_varlen_full_vjp_noalloc")
    return outs


def _with_workspace(g):
    lib = _lib.load()
    prob = rga.api.make_problem(g.q, g.k, g.cu_q, g.cu_k, g.slopes, False, -1, -1, g.softcap,
                                g.scale_multiplier)
    outs = _outputs(g)
    views = _views(g, outs[:4])
    ws = torch.empty(_lib.NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device=g.q.device)
    st = lib.attn_varlen_full_vjp(ctypes.byref(prob), *[ctypes.byref(t) for t in views],
                                  rga.api._fptr(outs[4]), ctypes.c_void_p(ws.data_ptr()),
                                  ws.numel(), rga.api._stream(g.q.device))
    _lib.raise_for(st, "attn_varlen_full_vjp")
    return outs


def test_noalloc_matches_workspace_entry():
    need_gpu()
    names = ("out", "dq", "dk", "dv", "lse")
    for label, wl in (("q_short_k_long", W.make_workload(1)), ("tiny_ragged_gqa", W.make_workload(0))):
        say(f"[noalloc] {label} Tq={wl.total_q} Tk={wl.total_k} hq={wl.hq}")
        g = wl.to("cuda")
        got = _noalloc(g)
        torch.cuda.synchronize()
        want = _with_workspace(g)
        torch.cuda.synchronize()
        for n, a, b in zip(names, want, got):
            assert torch.equal(a, b), (label, n)


def test_noalloc_rejects_problems_beyond_the_scratch():
    need_gpu()
    wl = W.custom_workload(lq=[1], lk=[1], hq=48)
    g = wl.to("cuda")
    lib = _lib.load()
    # a problem whose minimum workspace exceeds the array (2e6 query tokens x
    # 64 heads of row records); no tensor is touched before the size check
    prob = rga.api.make_problem(g.q, g.k, g.cu_q, g.cu_k, g.slopes, False, -1, -1, g.softcap,
                                g.scale_multiplier)
    prob.total_q = 2_000_000
    prob.hq = 64
    prob.slopes_stride = 64
    t = _lib.AttnTensor(0, 0, 0)
    st = lib.attn_varlen_full_vjp_noalloc(ctypes.byref(prob), *[ctypes.byref(t)] * 8, None,
                                          None)
    assert st == _lib.ATTN_WORKSPACE_TOO_SMALL
    assert "static scratch" in lib.attn_last_error().decode()
