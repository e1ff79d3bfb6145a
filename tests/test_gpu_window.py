"""Causal and sliding-window masks on the HIP path against the oracle.

The arguments come from the entry point's signature on page "Noncausal
Global Extreme-GQA Ragged Attention Full VJP" (section "What You Have"),
which never defines them; the reading checked here (and pinned in the
oracle's own tests) keeps key j of query row i iff
i + Lk - Lq - window_left <= j <= i + Lk - Lq + window_right, a bound of -1
meaning none and causal meaning window_right = 0.  Rows that keep no key
(causal rows of a sequence with Lq > Lk, for instance) must come out as rows
with no keys: out = 0, L = -inf, zero gradients."""
import numpy as np
import pytest
import torch

import oracle
import ragged_gqa_attention_amd as rga
import workloads as W
from tests.gpu_util import TOL, assert_close, assert_lse, need_gpu, say, to_np

pytestmark = pytest.mark.gpu

WINDOWS = [(True, -1, -1), (True, 24, -1), (False, 0, 0), (False, 5, 9), (False, -1, 70),
           (False, 40, -1), (False, 130, 0)]


def _oracle(wl, causal, wl_, wr):
    inp = W.oracle_inputs(wl)
    return oracle.vjp(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"],
                      inp["alibi_slopes"], inp["dout"], inp["softcap"], inp["scale_multiplier"],
                      causal=causal, window_left=wl_, window_right=wr)


def _check(wl, causal, wl_, wr, label, store_ds=True):
    say(f"[{label}] causal={causal} window=({wl_},{wr}) {wl.dtype} softcap={wl.softcap} "
        f"store_ds={store_ds} lq={list(wl.lq)} lk={list(wl.lk)}")
    g = wl.to("cuda")
    out, dq, dk, dv, lse = rga.attn_varlen_full_vjp(
        g.q, g.k, g.v, g.cu_q, g.cu_k, g.slopes, g.dout, softcap=g.softcap,
        scale_multiplier=g.scale_multiplier, causal=causal, window_left=wl_, window_right=wr,
        want_lse=True, check=True, store_ds=store_ds)
    torch.cuda.synchronize()
    ref = _oracle(wl, causal, wl_, wr)
    tol = TOL[wl.dtype]
    names = ("out", "dq", "dk", "dv")
    if (wl_, wr) == (0, 0) and not causal:
        # One kept key: P = 1 and the exact dS = dP - Delta is 0, a difference
        # of two FP32 sums of 160 products (dP from the MFMA, Delta from the
        # rounded O), each within 160 * 2^-24 of sum |dO_d v_d| <= 160 max|dO|
        # max|v|.  dQ = sigma dS k and dK sums dS q over the hq rows centred on
        # a key, so both stay within that bound times sigma, max|k| or
        # hq max|q|, and 4 (the cap's factor 4 r (1 - r) <= 1 is folded in).
        inp = W.oracle_inputs(wl)
        sigma = wl.scale_multiplier / np.sqrt(160.0)
        ds_bound = 2 * 160 * 2.0 ** -24 * 160 * np.abs(inp["dout"]).max() * np.abs(inp["v"]).max()
        bounds = {"dq": 4 * sigma * ds_bound * np.abs(inp["k"]).max(),
                  "dk": 4 * sigma * ds_bound * wl.hq * np.abs(inp["q"]).max()}
        for name, t in (("dq", dq), ("dk", dk)):
            e = np.abs(to_np(t)).max()
            say(f"  {label} {name}: max|got| {e:.3e} (exact 0, rounding bound {bounds[name]:.3e})")
            assert e <= bounds[name], (label, name, e)
        names = ("out", "dv")
    got = dict(out=out, dq=dq, dk=dk, dv=dv)
    for name in names:
        assert_close(name, to_np(got[name]), ref[name], tol, label)
    assert_lse(to_np(lse), ref["lse"], label)
    return ref


@pytest.mark.parametrize("causal,wl_,wr", WINDOWS)
def test_window_parity_bf16(causal, wl_, wr):
    """Sequences with Lq < Lk, Lq > Lk (rows that keep nothing under causal)
    and Lq = Lk, several 256-row tiles and ragged key tails."""
    wl = W.custom_workload(lq=[37, 150, 64, 9, 0], lk=[300, 90, 64, 200, 17], hq=48,
                           dtype="bf16", width=192, step=1, seed=41)
    _check(wl, causal, wl_, wr, "bf16")


@pytest.mark.parametrize("causal,wl_,wr", [(True, -1, -1), (False, 5, 9), (False, 130, 0)])
def test_window_parity_f16_recompute_and_no_cap(causal, wl_, wr):
    """FP16, dQ recomputing dS (minimum workspace), and the uncapped forward
    whose running maximum starts on rows that see only masked keys."""
    wl = W.custom_workload(lq=[70, 120, 33], lk=[260, 40, 129], hq=64, dtype="f16", width=176,
                           step=2, seed=42)
    _check(wl, causal, wl_, wr, "f16 recompute", store_ds=False)
    wl0 = W.custom_workload(lq=[70, 120, 33], lk=[260, 40, 129], hq=64, dtype="f16", width=176,
                            step=2, seed=43, softcap=0.0)
    _check(wl0, causal, wl_, wr, "f16 no cap")


def test_causal_empty_rows_and_separate_entries():
    """Causal with Lq > Lk: the first Lq - Lk rows keep nothing.  The separate
    forward and backward entries agree with the oracle too."""
    wl = W.custom_workload(lq=[40, 8], lk=[10, 30], hq=48, dtype="bf16", width=160, step=1,
                           seed=44)
    ref = _check(wl, True, -1, -1, "causal empty rows")
    assert np.isneginf(ref["lse"][:30]).all() and np.isfinite(ref["lse"][30:40]).all()
    g = wl.to("cuda")
    tol = TOL[wl.dtype]
    out, lse = rga.attn_varlen_fwd(g.q, g.k, g.v, g.cu_q, g.cu_k, g.slopes, g.softcap,
                                   g.scale_multiplier, causal=True, check=True)
    torch.cuda.synchronize()
    assert_close("out", to_np(out), ref["out"], tol, "fwd entry")
    assert_lse(to_np(lse), ref["lse"], "fwd entry")
    assert np.all(to_np(out)[:30] == 0)
    for store_ds in (True, False):
        dq, dk, dv = rga.attn_varlen_bwd(g.q, g.k, g.v, out, lse, g.dout, g.cu_q, g.cu_k,
                                         g.slopes, g.softcap, g.scale_multiplier, causal=True,
                                         check=True, store_ds=store_ds)
        torch.cuda.synchronize()
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            assert_close(name, to_np(t), ref[name], tol, f"bwd entry store_ds={store_ds}")


def _window_ranges_host(wl, wl_, wr, thr):
    """The library's range rule on the host: per head of a 256-row tile, the
    ALiBi steps of its first and last token (FP32 half-width) intersected with
    the steps holding its tokens' window keys; the union over the tile's heads."""
    LOG2E = 1.4426950408889634
    slopes = wl.slopes.numpy().astype(np.float32)
    out = []
    for b in range(wl.batch):
        Lq, Lk = int(wl.lq[b]), int(wl.lk[b])
        rows = Lq * wl.hq
        for R0 in range(0, rows, 256):
            R1 = min(rows, R0 + 256)
            lo, hi = 2**31 - 1, 0
            for h in range(R0 // Lq, (R1 - 1) // Lq + 1):
                ia = R0 - h * Lq if h == R0 // Lq else 0
                ib = R1 - 1 - h * Lq if h == (R1 - 1) // Lq else Lq - 1
                slope2 = slopes[b, h] * np.float32(LOG2E)
                span = np.float32(thr) / slope2 if slope2 > 0 else np.inf
                nks = (Lk + 63) // 64
                if slope2 > 0 and span < np.float32(Lk):
                    ds = int(span)
                    l0 = max(0, max(ia + Lk - Lq, 0) - ds) // 64
                    u1 = min(Lk - 1, max(ib + Lk - Lq, 0) + ds) // 64 + 1
                else:
                    l0, u1 = 0, nks
                klo = max(0, ia + Lk - Lq - wl_) if wl_ >= 0 else 0
                khi = min(Lk - 1, ib + Lk - Lq + wr) if wr >= 0 else Lk - 1
                if klo > khi:
                    continue
                l, u = max(l0, klo // 64), min(u1, khi // 64 + 1)
                if l < u:
                    lo, hi = min(lo, l), max(hi, u)
            out.append((lo, hi) if lo < hi else (0, 0))   # rows that keep nothing
    return np.array(out, np.int64).reshape(-1, 2)


@pytest.mark.parametrize("causal,wl_,wr", [(True, -1, -1), (False, 100, 0), (False, 64, 64),
                                           (False, -1, 5)])
def test_window_key_steps(causal, wl_, wr):
    """The row tiles visit only the key steps that hold some row's window
    keys (intersected with the far-key rule): the recorded ranges equal the
    host rule (tiles whose rows keep nothing get the empty range (0, 0)),
    cover every kept key of every row, the outputs match the oracle, and a
    causal call on equal lengths visits at most 80 % of the steps (a 256-row
    tile spans 256 consecutive tokens of one head, so its causal range is a
    prefix of the keys)."""
    need_gpu()
    wl = W.custom_workload(lq=[700, 37, 300, 1000], lk=[700, 900, 40, 1000], hq=16,
                           dtype="bf16", width=160, step=1, seed=46)
    g = wl.to("cuda")
    call = rga.FullVJP(g.q, g.k, g.v, g.cu_q, g.cu_k, g.slopes, g.dout, causal=causal,
                       window_left=wl_, window_right=wr, softcap=g.softcap,
                       scale_multiplier=g.scale_multiplier, store_ds=True)
    out, dq, dk, dv = call()
    torch.cuda.synchronize()
    got = call.key_steps().astype(np.int64)
    ewr = 0 if causal else wr
    ref = _oracle(wl, causal, wl_, wr)
    for name, t in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert_close(name, to_np(t), ref[name], TOL[wl.dtype], f"window ranges {causal} {wl_} {wr}")
    want = _window_ranges_host(wl, wl_, ewr, 160.0 + 2.0 * wl.softcap * 1.4426950408889634)
    assert got.shape == want.shape
    assert np.array_equal(got, want)
    # every key a row keeps (inside its window and within the ALiBi rule's
    # half-width of its clamped centre) lies inside its tile's range
    thr = np.float32(160.0 + 2.0 * wl.softcap * 1.4426950408889634)
    slopes = wl.slopes.numpy().astype(np.float32)
    t = 0
    for b in range(wl.batch):
        Lq, Lk = int(wl.lq[b]), int(wl.lk[b])
        rows = Lq * wl.hq
        R = np.arange(rows)
        i, h = R % Lq, R // Lq
        c = i + Lk - Lq
        cc = np.maximum(c, 0)
        slope2 = slopes[b, h] * np.float32(1.4426950408889634)
        with np.errstate(divide="ignore", over="ignore"):
            span = np.where(slope2 > 0, thr / slope2, np.inf)
        ds = np.where(span < Lk, np.floor(np.minimum(span, 2.0**30)), 2**30).astype(np.int64)
        klo = np.maximum(cc - ds, 0)
        khi = np.minimum(cc + ds, Lk - 1)
        if wl_ >= 0:
            klo = np.maximum(klo, c - wl_)
        if ewr >= 0:
            khi = np.minimum(khi, c + ewr)
        for R0 in range(0, rows, 256):
            lo, hi = got[t]
            t += 1
            sel = slice(R0, min(rows, R0 + 256))
            kept = klo[sel] <= khi[sel]
            if kept.any():
                assert lo < hi
                assert np.all(klo[sel][kept] >= 64 * lo) and np.all(khi[sel][kept] < 64 * hi)
    if causal:
        full = sum(((int(lk) + 63) // 64) * ((int(lq) * wl.hq + 255) // 256)
                   for lq, lk in zip(wl.lq, wl.lk) if lq == lk)
        vis = 0
        t = 0
        for lq, lk in zip(wl.lq, wl.lk):
            n = (int(lq) * wl.hq + 255) // 256
            if lq == lk:
                vis += int(np.maximum(got[t:t + n, 1] - got[t:t + n, 0], 0).sum())
            t += n
        say(f"  causal, equal lengths: {vis} of {full} key steps visited")
        assert vis < 0.8 * full
