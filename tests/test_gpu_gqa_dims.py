"""General grouped-query ratios and head dimensions against the float64 oracle.

Page "Pairwise-Gated Attention Engine", section "The task", names head sizes
64 and 128 and grouped key/value heads; the oracle takes any Hkv dividing Hq
(query head h reads K/V head h // (Hq / Hkv)) and any head dimension, and is
pinned for Hkv = 2 by the brute-force and autograd tests of
tests/test_oracle.py.  Here the HIP path runs Hkv in {1, 2, 4, 8} and
D in {64, 128, 160}: every element of out, dq, dk, dv and lse, both dS modes,
masks, no cap, the separate forward / backward entries and bitwise repeats.
"""
import numpy as np
import pytest
import torch

import oracle
import ragged_gqa_attention_amd as rga
import workloads as W
from tests.gpu_util import (TOL, assert_close, assert_lse, check_full, need_gpu, oracle_full,
                            say, to_np)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", range(16))
def test_fuzz_gqa_dims_parity(seed):
    need_gpu()
    wl = W.fuzz_gqa_workload(seed)
    say(f"hkv={wl.hkv} D={wl.head_dim}")
    check_full(wl, f"fuzz_gqa{seed}")


@pytest.mark.parametrize("hkv,head_dim,dtype", [(8, 128, "bf16"), (4, 64, "f16"), (2, 160, "bf16"),
                                                (1, 128, "f16"), (1, 64, "bf16"),
                                                (8, 160, "f16")])
def test_gqa_dims_long_keys(hkv, head_dim, dtype):
    """Several 256-row tiles, long key runs (far-key skipping active) and
    ragged tails, in each head dimension."""
    need_gpu()
    wl = W.custom_workload(lq=[37, 5, 130, 0, 64], lk=[1500, 900, 700, 50, 1], hq=64, hkv=hkv,
                           head_dim=head_dim, dtype=dtype, width=head_dim + 32, step=2,
                           seed=60 + hkv + head_dim)
    check_full(wl, f"hkv{hkv} D{head_dim} {dtype}")


@pytest.mark.parametrize("hkv,head_dim", [(4, 128), (8, 64)])
@pytest.mark.parametrize("causal,wl_,wr,softcap", [(True, -1, -1, 3.0), (False, 20, 5, 3.0),
                                                   (False, -1, -1, 0.0)])
def test_gqa_dims_masks_and_no_cap(hkv, head_dim, causal, wl_, wr, softcap):
    need_gpu()
    wl = W.custom_workload(lq=[40, 150, 9], lk=[300, 90, 200], hq=32, hkv=hkv,
                           head_dim=head_dim, dtype="bf16", width=head_dim + 16, step=3,
                           seed=70 + hkv, softcap=softcap)
    g = wl.to("cuda")
    inp = W.oracle_inputs(wl)
    ref = oracle.vjp(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"],
                     inp["alibi_slopes"], inp["dout"], inp["softcap"], inp["scale_multiplier"],
                     causal=causal, window_left=wl_, window_right=wr)
    tol = TOL[wl.dtype]
    for store_ds in (True, False):
        lab = f"hkv{hkv} D{head_dim} mask=({causal},{wl_},{wr}) cap={softcap} ds={store_ds}"
        say(f"[{lab}]")
        out, dq, dk, dv, lse = rga.attn_varlen_full_vjp(
            g.q, g.k, g.v, g.cu_q, g.cu_k, g.slopes, g.dout, softcap=g.softcap,
            scale_multiplier=g.scale_multiplier, causal=causal, window_left=wl_,
            window_right=wr, want_lse=True, check=True, store_ds=store_ds)
        torch.cuda.synchronize()
        for name, t in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
            assert_close(name, to_np(t), ref[name], tol, lab)
        assert_lse(to_np(lse), ref["lse"], lab)


@pytest.mark.parametrize("hkv,head_dim", [(2, 64), (8, 128)])
def test_gqa_dims_separate_entries(hkv, head_dim):
    need_gpu()
    wl = W.custom_workload(lq=[33, 0, 70, 3], lk=[129, 5, 64, 1], hq=16, hkv=hkv,
                           head_dim=head_dim, dtype="f16", width=head_dim, step=1, seed=80)
    g = wl.to("cuda")
    ref = oracle_full(wl)
    tol = TOL[wl.dtype]
    out, lse = rga.attn_varlen_fwd(g.q, g.k, g.v, g.cu_q, g.cu_k, g.slopes, g.softcap,
                                   g.scale_multiplier, check=True)
    torch.cuda.synchronize()
    assert_close("out", to_np(out), ref["out"], tol, "fwd entry")
    assert_lse(to_np(lse), ref["lse"], "fwd entry")
    for store_ds in (True, False):
        dq, dk, dv = rga.attn_varlen_bwd(g.q, g.k, g.v, out, lse, g.dout, g.cu_q, g.cu_k,
                                         g.slopes, g.softcap, g.scale_multiplier, check=True,
                                         store_ds=store_ds)
        torch.cuda.synchronize()
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            assert_close(name, to_np(t), ref[name], tol, f"bwd entry ds={store_ds}")


@pytest.mark.parametrize("cfg", [5, 6])
def test_gqa_variant_configs_full_parity_and_repeat(cfg):
    """The Q-short/K-long draw with 8 K/V heads at D = 128 and with 4 K/V heads
    at D = 64: every element against the oracle, and three calls agreeing bit
    for bit."""
    need_gpu()
    wl = W.make_workload(cfg)
    (stored, recomputed), _ = check_full(wl, wl.name)
    for name in ("out", "lse", "dk", "dv"):
        assert torch.equal(stored[name], recomputed[name]), name
    g = wl.to("cuda")
    call = rga.FullVJP(g.q, g.k, g.v, g.cu_q, g.cu_k, g.slopes, g.dout, softcap=g.softcap,
                       scale_multiplier=g.scale_multiplier, want_lse=True, store_ds=True)
    res = []
    for _ in range(3):
        call()
        torch.cuda.synchronize()
        res.append([t.clone() for t in (call.out, call.dq, call.dk, call.dv, call.lse)])
    for other in res[1:]:
        for a, b in zip(res[0], other):
            assert torch.equal(a, b)


def test_gqa_key_steps_follow_the_rule():
    """The recorded key-step ranges of every 256-row tile (a tile folds the rows
    of one K/V head's query heads) equal a host evaluation of the rule."""
    need_gpu()
    LOG2E = 1.4426950408889634
    wl = W.custom_workload(lq=[37, 5, 90], lk=[3000, 900, 2100], hq=64, hkv=8, head_dim=128,
                           dtype="bf16", width=128, step=1, seed=90)
    g = wl.to("cuda")
    call = rga.FullVJP(g.q, g.k, g.v, g.cu_q, g.cu_k, g.slopes, g.dout, softcap=g.softcap,
                       scale_multiplier=g.scale_multiplier, store_ds=True)
    call()
    torch.cuda.synchronize()
    got = call.key_steps().astype(np.int64)
    thr = np.float32(160.0 + 2.0 * wl.softcap * LOG2E)
    slopes = wl.slopes.numpy().astype(np.float32)
    group = wl.hq // wl.hkv
    want = []
    for b in range(wl.batch):
        Lq, Lk = int(wl.lq[b]), int(wl.lk[b])
        for kvh in range(wl.hkv):
            rows = Lq * group
            R = np.arange(rows)
            h, i = kvh * group + R // Lq, R % Lq
            centre = np.maximum(i + Lk - Lq, 0)
            slope2 = slopes[b, h] * np.float32(LOG2E)
            with np.errstate(divide="ignore", over="ignore"):
                span = thr / slope2
            cut = (slope2 > 0) & (span < np.float32(Lk))
            ds = np.where(cut, span, 0).astype(np.int64)
            lo = np.where(cut, np.maximum(0, centre - ds) // 64, 0)
            hi = np.where(cut, np.minimum(Lk - 1, centre + ds) // 64 + 1, (Lk + 63) // 64)
            for t0 in range(0, rows, 256):
                want.append((lo[t0:t0 + 256].min(), hi[t0:t0 + 256].max()))
    want = np.array(want, np.int64)
    assert got.shape == want.shape
    assert np.array_equal(got, want)
    assert (want[:, 1] - want[:, 0]).sum() < 0.95 * sum(
        ((int(lk) + 63) // 64) * ((int(lq) * group + 255) // 256) * wl.hkv
        for lq, lk in zip(wl.lq, wl.lk)), "the workload should exercise the skipping"
