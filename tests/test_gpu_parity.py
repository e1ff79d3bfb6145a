"""Parity of the HIP path with the float64 oracle, element by element.

Small cases (config 0 and 30 seeded fuzz draws with lengths on and around the
32/64/128 tile edges, empty and single-key sequences, every head count, both
dtypes, token steps 1-3 and widths 160/176/192) compare every output element.
The Hq=64 Q-short/K-long configuration that the benchmark times is compared in
full.  Small and benchmark cases run twice: with a workspace that stores dS
for dQ and with the minimum workspace (dQ recomputes dS); one case stores dS
for only some sequences.  The three larger configurations compare sampled rows of out/dq (each row
depends only on its own inputs and its sequence's K/V), full dk/dv of their
cheapest sequences, and the identity sum_j dv_j = sum_(i,h) dout_(i,h) for
every sequence (each softmax row sums to one).
"""
import numpy as np
import pytest
import torch

import oracle
import ragged_gqa_attention_amd as rga
import workloads as W
from tests.gpu_util import (TOL, assert_close, assert_lse, check_full, gpu_full, need_gpu,
                            say, to_np)

pytestmark = pytest.mark.gpu


def test_tiny_ragged_gqa_full_parity():
    need_gpu()
    check_full(W.make_workload(0), "tiny_ragged_gqa")


@pytest.mark.parametrize("seed", range(30))
def test_fuzz_parity(seed):
    need_gpu()
    check_full(W.fuzz_workload(seed), f"fuzz{seed}")


def test_q_short_k_long_full_parity():
    """The benchmarked Hq=64 Q-short/K-long configuration, every element, with
    dQ from stored dS and with dQ recomputing dS."""
    need_gpu()
    (stored, recomputed), _ = check_full(W.make_workload(1), "q_short_k_long")
    # storing dS changes nothing before dQ
    for name in ("out", "lse", "dk", "dv"):
        assert torch.equal(stored[name], recomputed[name]), name


def test_partial_ds_capacity():
    """A workspace with room for the dS of only some sequences: those use the
    stored path, the rest recompute, and the result still matches the oracle."""
    need_gpu()
    wl = W.make_workload(1)
    g = wl.to("cuda")
    prob = rga.api.make_problem(g.q, g.k, g.cu_q, g.cu_k, g.slopes, False, -1, -1, g.softcap,
                                g.scale_multiplier)
    full = rga.workspace_size(prob, 2, g.cu_q, g.cu_k)
    base = rga.workspace_size(prob, 2)
    assert full > base
    # room for about 40 % of the images, plus a few bytes that fit no image
    (part,), ref = check_full(wl, "q_short_k_long partial", modes=((full - base) * 2 // 5 + 1000,))
    stored = gpu_full(g, store_ds=True)
    for name in ("out", "lse", "dk", "dv"):
        assert torch.equal(part[name], stored[name]), name


def _seq_slices(wl, b):
    q0, q1 = int(wl.cu_q[b]), int(wl.cu_q[b + 1])
    k0, k1 = int(wl.cu_k[b]), int(wl.cu_k[b + 1])
    return q0, q1, k0, k1


def _f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_large_config_sampled_parity(cfg):
    need_gpu()
    wl = W.make_workload(cfg)
    tol = TOL[wl.dtype]
    say(f"[cfg{cfg}] B={wl.batch} Hq={wl.hq} Tq={wl.total_q} Tk={wl.total_k}")
    got = gpu_full(wl.to("cuda"))
    g = {k: v for k, v in got.items()}
    rng = np.random.default_rng([cfg, 77])
    # sampled rows of out / dq / lse, a few per sequence
    ref_rows = {n: [] for n in ("out", "dq", "lse")}
    got_rows = {n: [] for n in ("out", "dq", "lse")}
    for b in range(wl.batch):
        q0, q1, k0, k1 = _seq_slices(wl, b)
        Lq = q1 - q0
        if Lq == 0:
            continue
        n = 6
        toks = np.concatenate([[0, Lq - 1], rng.integers(0, Lq, size=n - 2)])
        heads = np.concatenate([[0, wl.hq - 1], rng.integers(0, wl.hq, size=n - 2)])
        part = oracle.rows_vjp(_f64(wl.q[q0:q1]), _f64(wl.k[k0:k1]), _f64(wl.v[k0:k1]),
                               _f64(wl.dout[q0:q1]), wl.slopes[b].double().numpy(),
                               wl.softcap, wl.scale_multiplier, toks, heads)
        for name in ("out", "dq", "lse"):
            ref_rows[name].append(part[name])
            ti = torch.as_tensor(q0 + toks, device=g[name].device)
            hi = torch.as_tensor(heads, device=g[name].device)
            sel = g[name][ti, hi]
            got_rows[name].append(to_np(sel))
    for name in ("out", "dq"):
        assert_close(name, np.concatenate(got_rows[name]), np.concatenate(ref_rows[name]), tol,
                     f"{wl.name} sampled rows")
    assert_lse(np.concatenate(got_rows["lse"]), np.concatenate(ref_rows["lse"]), f"{wl.name}")

    # full dk / dv of the cheapest sequences with more than one key and query
    cost = wl.lq * wl.lk
    cand = [b for b in np.argsort(cost) if wl.lq[b] > 1 and wl.lk[b] > 1]
    chosen = [b for b in cand if cost[b] * wl.hq <= 4e7][:2]
    if cfg != 4:
        assert chosen, "no sequence cheap enough for a full dk/dv check"
    for b in chosen:
        q0, q1, k0, k1 = _seq_slices(wl, b)
        ref = oracle.sequence_vjp(_f64(wl.q[q0:q1]), _f64(wl.k[k0:k1]), _f64(wl.v[k0:k1]),
                                  _f64(wl.dout[q0:q1]), wl.slopes[b].double().numpy(),
                                  wl.softcap, wl.scale_multiplier)
        for name in ("dk", "dv", "out", "dq"):
            sl = slice(k0, k1) if name in ("dk", "dv") else slice(q0, q1)
            assert_close(name, to_np(g[name][sl]), ref[name], tol, f"{wl.name} seq{b}")

    # sum_j dv_j = sum over the sequence's rows of dout, for every sequence
    dv = to_np(g["dv"])
    for b in range(wl.batch):
        q0, q1, k0, k1 = _seq_slices(wl, b)
        if k1 == k0:
            continue
        lhs = dv[k0:k1, 0].sum(0)
        rhs = _f64(wl.dout[q0:q1]).sum((0, 1)) if q1 > q0 else np.zeros(160)
        scale = np.abs(dv[k0:k1, 0]).sum(0).max() + np.abs(rhs).max() + 1e-30
        assert np.abs(lhs - rhs).max() <= tol * scale, f"{wl.name} seq{b}: sum dv identity"
    for name in ("out", "dq", "dk", "dv"):
        assert torch.isfinite(g[name]).all(), f"{wl.name} {name} non-finite"
