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
