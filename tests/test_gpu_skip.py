"""Exact skipping of far keys.

With a soft cap every capped logit lies in [-c, c], so the ALiBi term alone
decides that keys far from a row's centre get probabilities below FP32's
smallest subnormal (page "Noncausal Global Extreme-GQA Ragged Attention Full
VJP", section "Hard Constraints": the cap sits between the scaled dot product
and ALiBi; section "What You Have": the bias grows with |i + Lk - Lq - j|).
The library skips the 64-key steps that hold only such keys for a whole
256-row tile.  These tests check that

* out, lse and dq are bitwise those of evaluating every key
  (ATTN_FLAG_ALL_KEYS), for the full-VJP call in both dS modes and for the
  separate entries; dk and dv agree to within one unit in the last place plus
  FP32 summation-order noise (the planner splits a key tile's visiting rows
  into units by the visits, so the FP32 partial sums group differently);
* the recorded key-step ranges follow the rule exactly (index work: equal);
* every skipped (row, key) pair has a float64 probability below 2^-149, i.e.
  the rule only drops what the definition makes negligible.
"""
import numpy as np
import pytest
import torch

import ragged_gqa_attention_amd as rga
from ragged_gqa_attention_amd import _lib
from ragged_gqa_attention_amd.api import key_steps
import workloads as W
from tests.gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634
SKIP_UNDERFLOW = 160.0   # log2 units below the row's largest logit (see the header)


def _long_key_workload():
    """Short query runs against long key runs, where far keys are plentiful."""
    return W.custom_workload(lq=[37, 5, 300, 0, 64], lk=[3000, 900, 4100, 50, 1], hq=64,
                             dtype="bf16", width=160, step=2, seed=9)


WORKLOADS = {
    "tiny_ragged_gqa": lambda: W.make_workload(0),
    "q_short_k_long": lambda: W.make_workload(1),
    "mixed_extreme": lambda: W.make_workload(3),
    "long_keys": _long_key_workload,
}


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _same(name, a, b, label):
    if name in ("dk", "dv"):
        # one unit in the last place, plus FP32 summation-order noise where
        # the partial sums cancel (2^-16 of the tensor's largest value)
        x, y = a.float(), b.float()
        bound = torch.finfo(a.dtype).eps * torch.maximum(x.abs(), y.abs())
        bound = bound + 2.0 ** -16 * x.abs().max()
        bad = (x - y).abs() > bound
        assert not bad.any(), f"{label}: {name} differs beyond summation order"
    else:
        assert torch.equal(_bits(a), _bits(b)), f"{label}: {name} differs"


def _call(g, all_keys, store_ds):
    c = rga.FullVJP(g.q, g.k, g.v, g.cu_q, g.cu_k, g.slopes, g.dout, softcap=g.softcap,
                    scale_multiplier=g.scale_multiplier, want_lse=True, store_ds=store_ds,
                    all_keys=all_keys)
    c()
    torch.cuda.synchronize()
    return c


def _host_ranges(wl, thr):
    """The rule of row_key_steps in FP32, min / max over each 256-row tile."""
    lq = np.asarray(wl.lq, np.int64)
    lk = np.asarray(wl.lk, np.int64)
    slopes = wl.slopes.cpu().numpy().astype(np.float32)
    out = []
    for b in range(len(lq)):
        Lq, Lk, hq = int(lq[b]), int(lk[b]), wl.hq
        rows = Lq * hq
        if rows == 0:
            continue
        R = np.arange(rows)
        h, i = R // Lq, R % Lq
        centre = np.maximum(i + Lk - Lq, 0)
        nks = (Lk + 63) // 64
        lo = np.zeros(rows, np.int64)
        hi = np.full(rows, nks, np.int64)
        slope2 = slopes[b, h] * np.float32(LOG2E)
        if thr > 0:
            with np.errstate(divide="ignore", over="ignore"):
                span = np.float32(thr) / slope2
            cut = (slope2 > 0) & (span < np.float32(Lk))
            ds = np.where(cut, span, 0).astype(np.int64)
            lo = np.where(cut, np.maximum(0, centre - ds) // 64, lo)
            hi = np.where(cut, np.minimum(Lk - 1, centre + ds) // 64 + 1, hi)
        for t0 in range(0, rows, 256):
            out.append((lo[t0:t0 + 256].min(), hi[t0:t0 + 256].max()))
    return np.array(out, np.int64).reshape(-1, 2)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_skip_is_bitwise_exact(name):
    need_gpu()
    wl = WORKLOADS[name]()
    g = wl.to("cuda")
    for store_ds in (True, False):
        say(f"{name} store_ds={store_ds}")
        ref = _call(g, True, store_ds)
        got = _call(g, False, store_ds)
        for n in ("out", "dq", "dk", "dv", "lse"):
            _same(n, getattr(ref, n), getattr(got, n), f"{name} store_ds={store_ds}")
        full = ref.key_steps()
        part = got.key_steps()
        nks = np.array([(int(lk) + 63) // 64 for lq_, lk in zip(wl.lq, wl.lk)
                        for _ in range((int(lq_) * wl.hq + 255) // 256)], np.int64)
        assert np.array_equal(full[:, 0], np.zeros_like(nks)) and np.array_equal(full[:, 1], nks)
        kept = float((part[:, 1] - part[:, 0]).sum()) / max(1, int(nks.sum()))
        say(f"  key steps visited: {kept:.3f} of all")
        if name in ("q_short_k_long", "long_keys"):
            assert kept < 0.95, "the workload should exercise the skipping"


@pytest.mark.parametrize("name", ["q_short_k_long", "long_keys"])
def test_key_steps_follow_the_rule(name):
    need_gpu()
    wl = WORKLOADS[name]()
    g = wl.to("cuda")
    call = _call(g, False, True)
    got = call.key_steps().astype(np.int64)
    thr = np.float32(SKIP_UNDERFLOW + 2.0 * wl.softcap * LOG2E)
    want = _host_ranges(wl, float(thr))
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def test_no_cap_means_no_skipping():
    need_gpu()
    wl = W.custom_workload(lq=[37, 5], lk=[3000, 900], hq=64, dtype="f16", width=160, step=1,
                           seed=3, softcap=0.0)
    g = wl.to("cuda")
    call = _call(g, False, True)
    got = call.key_steps()
    want = _host_ranges(wl, 0.0)
    assert np.array_equal(got, want)


def test_skipped_pairs_have_negligible_probability():
    """Every (row, key) outside its tile's recorded range has P < 2^-149 in
    float64, computed from the definition of the logits and the oracle-free
    log-sum-exp over all keys."""
    need_gpu()
    wl = _long_key_workload()
    g = wl.to("cuda")
    ks = _call(g, False, True).key_steps()
    inp = W.oracle_inputs(wl)
    sigma = wl.scale_multiplier / np.sqrt(160.0)
    c = wl.softcap
    tile = 0
    worst = -np.inf
    for b in range(len(wl.lq)):
        q0, q1 = int(inp["cu_q"][b]), int(inp["cu_q"][b + 1])
        k0, k1 = int(inp["cu_k"][b]), int(inp["cu_k"][b + 1])
        Lq, Lk = q1 - q0, k1 - k0
        if Lq == 0:
            continue
        K = inp["k"][k0:k1, 0]
        j = np.arange(Lk)
        i = np.arange(Lq)
        rows_lo = []
        rows_hi = []
        for t0 in range(0, Lq * wl.hq, 256):
            lo, hi = ks[tile]
            tile += 1
            n = min(256, Lq * wl.hq - t0)
            rows_lo += [lo] * n
            rows_hi += [hi] * n
        rows_lo = np.array(rows_lo).reshape(wl.hq, Lq)
        rows_hi = np.array(rows_hi).reshape(wl.hq, Lq)
        if Lk == 0:
            continue
        for h in range(wl.hq):
            S = sigma * (inp["q"][q0:q1, h] @ K.T)
            A = c * np.tanh(S / c) - inp["alibi_slopes"][b, h] * np.abs(
                i[:, None] + (Lk - Lq) - j[None, :])
            m = A.max(axis=1, keepdims=True)
            lse = m + np.log(np.exp(A - m).sum(axis=1, keepdims=True))
            skipped = (j[None, :] < 64 * rows_lo[h][:, None]) | (j[None, :] >= 64 * rows_hi[h][:, None])
            if skipped.any():
                worst = max(worst, float((A - lse)[skipped].max()))
    assert tile == len(ks)
    say(f"  largest log P among skipped pairs: {worst:.1f} (bound {np.log(2.0 ** -149):.1f})")
    assert worst < np.log(2.0 ** -149)
    assert np.isfinite(worst), "the workload should skip some pairs"


def test_separate_entries_bitwise_exact():
    need_gpu()
    wl = _long_key_workload()
    g = wl.to("cuda")
    res = {}
    for all_keys in (True, False):
        out, lse = rga.attn_varlen_fwd(g.q, g.k, g.v, g.cu_q, g.cu_k, g.slopes, g.softcap,
                                       g.scale_multiplier, all_keys=all_keys)
        grads = rga.attn_varlen_bwd(g.q, g.k, g.v, out, lse, g.dout, g.cu_q, g.cu_k, g.slopes,
                                    g.softcap, g.scale_multiplier, all_keys=all_keys)
        torch.cuda.synchronize()
        res[all_keys] = (out, lse) + tuple(grads)
    for n, a, b in zip(("out", "lse", "dq", "dk", "dv"), res[True], res[False]):
        _same(n, a, b, "separate entries")


def test_backward_entry_records_ranges():
    """The standalone backward derives its ranges from the caller's L: with the
    forward's own L they lie inside the forward's ranges."""
    need_gpu()
    wl = _long_key_workload()
    g = wl.to("cuda")
    prob = rga.api.make_problem(g.q, g.k, g.cu_q, g.cu_k, g.slopes, False, -1, -1, g.softcap,
                                g.scale_multiplier)
    ws_f = torch.empty(rga.workspace_size(prob, _lib.ENTRY_FWD), dtype=torch.uint8,
                       device="cuda")
    out, lse = rga.attn_varlen_fwd(g.q, g.k, g.v, g.cu_q, g.cu_k, g.slopes, g.softcap,
                                   g.scale_multiplier, workspace=ws_f)
    ws_b = torch.empty(rga.workspace_size(prob, _lib.ENTRY_BWD), dtype=torch.uint8,
                       device="cuda")
    rga.attn_varlen_bwd(g.q, g.k, g.v, out, lse, g.dout, g.cu_q, g.cu_k, g.slopes, g.softcap,
                        g.scale_multiplier, workspace=ws_b)
    fwd = key_steps(prob, _lib.ENTRY_FWD, ws_f, g.cu_q)
    bwd = key_steps(prob, _lib.ENTRY_BWD, ws_b, g.cu_q)
    assert fwd.shape == bwd.shape
    assert (bwd[:, 0] >= fwd[:, 0]).all() and (bwd[:, 1] <= fwd[:, 1]).all()
    assert (bwd[:, 1] > bwd[:, 0]).all()
