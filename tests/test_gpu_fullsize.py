"""Element-by-element parity with the float64 oracle on long sequences.

The smaller parity tests compare whole tensors at up to a few thousand keys;
these cover what only long sequences reach, against the oracle run on the
same sequence in full:

* the shortest sequence of the balanced-long workload (18 sequences of
  4096-8192 tokens, Hq = 48, FP16), every element of out, dq, dk and dv, so
  the longest dK/dV work splits and the compute-bound launch shapes are
  checked against the definition;
* a long sequence of the mixed-extreme geometry (Hq = 96, BF16, token step 3,
  width 192) with Lq, Lk >= 1000: dk and dv over ~2e8 score elements;
* short queries against 3000-4100 keys in BF16, in FP16 and without a soft cap
  (the running-maximum rescale across more than 60 key steps);
* packed views that span more than 2^31 elements (page "Noncausal Global
  Extreme-GQA Ragged Attention Full VJP", rollout table: 64-bit packed-token
  pointers for spans above 2^31 elements), checked on rows and keys that sit
  past that offset.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import (TOL, assert_close, assert_lse, f64, gpu_full, need_gpu,
                            oracle_sequence_heads, say, to_np)

pytestmark = pytest.mark.gpu


def _seq(wl, b):
    q0, q1 = int(wl.cu_q[b]), int(wl.cu_q[b + 1])
    k0, k1 = int(wl.cu_k[b]), int(wl.cu_k[b + 1])
    return q0, q1, k0, k1


def _compare_sequence(wl, got, b, label, names=("out", "dq", "dk", "dv"), workers=4):
    q0, q1, k0, k1 = _seq(wl, b)
    say(f"[{label}] sequence {b}: Lq={q1 - q0} Lk={k1 - k0} Hq={wl.hq} {wl.dtype} "
        f"softcap={wl.softcap}")
    ref = oracle_sequence_heads(f64(wl.q[q0:q1]), f64(wl.k[k0:k1]), f64(wl.v[k0:k1]),
                                f64(wl.dout[q0:q1]), wl.slopes[b].double().numpy(), wl.softcap,
                                wl.scale_multiplier, workers=workers, label=label)
    tol = TOL[wl.dtype]
    for name in names:
        sl = slice(k0, k1) if name in ("dk", "dv") else slice(q0, q1)
        assert_close(name, to_np(got[name][sl]), ref[name], tol, f"{label} seq{b}")
    if "out" in names:
        assert_lse(to_np(got["lse"][q0:q1]), ref["lse"], f"{label} seq{b}")


@pytest.mark.timeout(900)
def test_balanced_long_shortest_sequence_in_full():
    """Every element of the shortest 4096-8192-token sequence, both dS modes
    (the default 8 GiB dS budget stores the first sequences and recomputes the
    rest; the minimum workspace recomputes all)."""
    need_gpu()
    wl = W.make_workload(4)
    b = int(np.argmin(wl.lq))
    g = wl.to("cuda")
    res = {}
    for mode in (True, False):
        say(f"[balanced_long] GPU call store_ds={mode}")
        res[mode] = gpu_full(g, store_ds=mode)
    for name in ("out", "lse", "dk", "dv"):
        assert torch.equal(res[True][name], res[False][name]), name
    _compare_sequence(wl, res[True], b, "balanced_long store_ds=True", workers=6)
    q0, q1, _, _ = _seq(wl, b)
    ref_dq = res[True]["dq"][q0:q1].float()
    other = res[False]["dq"][q0:q1].float()
    # stored and recomputed dS round the same value: dq agrees to the tolerance
    err = (ref_dq - other).abs().max().item() / ref_dq.abs().max().item()
    say(f"  balanced_long dq stored vs recomputed dS: {err:.2e}")
    assert err <= TOL[wl.dtype]


@pytest.mark.timeout(600)
def test_mixed_extreme_long_sequence_dkdv():
    """Mixed-extreme draw 3 holds sequence 4 with (Lq, Lk) = (1039, 2188): full
    dk, dv, out and dq of that sequence."""
    need_gpu()
    wl = W.make_workload(3, 3)
    b = 4
    assert wl.lq[b] >= 1000 and wl.lk[b] >= 1000
    got = gpu_full(wl.to("cuda"))
    _compare_sequence(wl, got, b, "mixed_extreme trial 3", workers=6)


def _long_keys(dtype, softcap, seed):
    width = 160 if dtype == "bf16" else 176
    return W.custom_workload(lq=[37, 5, 300, 0, 64], lk=[3000, 900, 4100, 50, 1], hq=64,
                             dtype=dtype, width=width, step=2, seed=seed, softcap=softcap)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype,softcap", [("bf16", 3.0), ("f16", 3.0), ("bf16", 0.0),
                                           ("f16", 0.0)])
def test_long_keys_full(dtype, softcap):
    """Queries against up to 4100 keys, whole tensors against the whole
    oracle, with dS stored and recomputed."""
    need_gpu()
    wl = _long_keys(dtype, softcap, seed=9 if softcap else 19)
    g = wl.to("cuda")
    inp = W.oracle_inputs(wl)
    ref = oracle.vjp(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"],
                     inp["alibi_slopes"], inp["dout"], inp["softcap"], inp["scale_multiplier"])
    tol = TOL[wl.dtype]
    for mode in (True, False):
        lab = f"long keys {dtype} softcap={softcap} store_ds={mode}"
        say(f"[{lab}]")
        got = gpu_full(g, store_ds=mode)
        for name in ("out", "dq", "dk", "dv"):
            assert_close(name, to_np(got[name]), ref[name], tol, lab)
        assert_lse(to_np(got["lse"]), ref["lse"], lab)


@pytest.mark.timeout(900)
def test_views_beyond_2_31_elements():
    """q and dout views of 40,000 tokens in the mixed-extreme geometry (token
    stride 3 * 96 * 192 = 55,296 elements) end 2.21e9 elements past their
    base.  The second sequence's rows all lie beyond element 2^31: its dk and
    dv in full, and sampled rows of out / dq / lse of both sequences, whose
    results depend only on their own q / dout rows and their sequence's K/V."""
    need_gpu()
    lq, lk = [39000, 1000], [64, 600]
    wl = W.custom_workload(lq=lq, lk=lk, hq=96, dtype="bf16", width=192, step=3, seed=31)
    ts = wl.q.stride(0)
    span = (wl.total_q - 1) * ts + (wl.hq - 1) * wl.q.stride(1) + 160
    say(f"[2^31 views] token stride {ts}, view span {span} elements")
    assert span > 2**31 and 39000 * ts > 2**31
    g = wl.to("cuda")
    tol = TOL[wl.dtype]
    for mode in (True, False):
        lab = f"2^31 views store_ds={mode}"
        got = gpu_full(g, store_ds=mode)
        _compare_sequence(wl, got, 1, lab, names=("dk", "dv", "out", "dq"), workers=6)
        rng = np.random.default_rng(5)
        for b in (0, 1):
            q0, q1, k0, k1 = _seq(wl, b)
            Lq = q1 - q0
            toks = np.concatenate([[Lq - 1, Lq - 2], rng.integers(max(0, Lq - 400), Lq, 10)])
            heads = np.concatenate([[wl.hq - 1, 0], rng.integers(0, wl.hq, 10)])
            # full-length arrays (the ALiBi centre needs Lq) holding only the
            # sampled tokens; np.zeros pages stay untouched elsewhere
            qs = np.zeros((Lq, wl.hq, 160))
            ds = np.zeros((Lq, wl.hq, 160))
            sel = np.unique(toks)
            qs[sel] = f64(wl.q[q0 + torch.as_tensor(sel)])
            ds[sel] = f64(wl.dout[q0 + torch.as_tensor(sel)])
            part = oracle.rows_vjp(qs, f64(wl.k[k0:k1]), f64(wl.v[k0:k1]), ds,
                                   wl.slopes[b].double().numpy(), wl.softcap,
                                   wl.scale_multiplier, toks, heads)
            ti = torch.as_tensor(q0 + toks, device="cuda")
            hi = torch.as_tensor(heads, device="cuda")
            for name in ("out", "dq"):
                assert_close(name, to_np(got[name][ti, hi]), part[name], tol, f"{lab} rows b{b}")
            assert_lse(to_np(got["lse"][ti, hi]), part["lse"], f"{lab} rows b{b}")
        # every key of sequence 0: sum_j dv_j = sum over its rows of dout
        q0, q1, k0, k1 = _seq(wl, 0)
        lhs = to_np(got["dv"][k0:k1, 0]).sum(0)
        rhs = to_np(g.dout[q0:q1].float().sum((0, 1)))
        scale = np.abs(to_np(got["dv"][k0:k1, 0])).sum(0).max() + np.abs(rhs).max()
        assert np.abs(lhs - rhs).max() <= tol * scale
        del got
        torch.cuda.empty_cache()
