"""Pins of the oracle's counter-based dropout against things other than itself.

Page "python-20261012-ragged-flash-attention-gradient-recompute", section
"Root causes addressed": dropout from a counter-based splitmix64 hash of
(seed, b, h, row, col), the same whatever the tiling, with one rate or one
per row; section "Verification": determinism across tile sizes and correct
per-row rates.  The reading of how the hash is composed is in
oracle/dropout.py.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import dropout as dr


def test_splitmix64_reference_outputs():
    """The published reference generator (Steele, Lea and Flood 2014) started
    at state 0 returns these first four outputs."""
    assert dr.splitmix64_outputs(0, 4) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                           0x06C45D188009454F, 0xF88BB8A8724C81EC]


def test_streams_are_outputs_of_a_stepped_generator():
    """The (b, h) stream state is output b * 2^16 + h + 1 of the generator
    started at the seed, and row 0's words are that stream's outputs 1, 2, ...,
    both found by stepping a generator one output at a time."""
    seed = 0x1234_5678_9ABC_DEF0
    for b, h in ((0, 0), (0, 5), (1, 3)):
        n = (b << 16) + h + 1
        assert dr.stream_state(seed, b, h) == dr.splitmix64_outputs(seed, n)[-1]
    s = dr.stream_state(seed, 2, 7)
    w = dr.words(seed, 2, 7, [0], 50)[0]
    assert [int(x) for x in w] == dr.splitmix64_outputs(s, 50)


def test_threshold_is_exact():
    assert int(dr.threshold(np.float32(0.5))) == 2**31
    assert int(dr.threshold(np.float32(0.25))) == 2**30
    assert int(dr.threshold(np.float32(0.0))) == 0
    p = np.float32(0.1)
    assert int(dr.threshold(p)) == math.floor(float(p) * 2**32)
    with pytest.raises(ValueError):
        dr.threshold(np.float32(1.0))


@pytest.mark.parametrize("p", [0.1, 0.5, 0.875])
def test_keep_rate_and_row_independence(p):
    """The kept share of 2e5 (row, key) pairs is 1 - p within five standard
    deviations, and two different rows agree on a key as often as two
    independent draws would."""
    n, Lk = 400, 500
    ks = dr.keep_scale(99, 3, 11, np.arange(n), Lk, np.full(n, p, np.float32))
    kept = ks > 0
    N = kept.size
    sd = math.sqrt(p * (1 - p) / N)
    assert abs(kept.mean() - (1 - p)) < 5 * sd
    assert np.allclose(ks[kept], 1.0 / (1.0 - float(np.float32(p))))
    agree = (kept[:-1] == kept[1:]).mean()
    want = (1 - p) ** 2 + p ** 2
    assert abs(agree - want) < 5 * math.sqrt(want * (1 - want) / kept[:-1].size)
    # other streams (head, sequence, seed) are not the same mask
    for other in (dr.keep_scale(99, 3, 12, np.arange(n), Lk, np.full(n, p, np.float32)),
                  dr.keep_scale(99, 4, 11, np.arange(n), Lk, np.full(n, p, np.float32)),
                  dr.keep_scale(98, 3, 11, np.arange(n), Lk, np.full(n, p, np.float32))):
        assert abs(((other > 0) == kept).mean() - want) < 0.01


def _case(rng, lq, lk, hq=2, hkv=1, D=4, scale=1.5):
    lq = np.asarray(lq)
    lk = np.asarray(lk)
    return dict(q=rng.standard_normal((int(lq.sum()), hq, D)) * scale,
                k=rng.standard_normal((int(lk.sum()), hkv, D)) * scale,
                v=rng.standard_normal((int(lk.sum()), hkv, D)),
                dout=rng.standard_normal((int(lq.sum()), hq, D)),
                cu_q=np.concatenate([[0], np.cumsum(lq)]),
                cu_k=np.concatenate([[0], np.cumsum(lk)]),
                alibi_slopes=rng.uniform(0.0, 0.5, size=(len(lq), hq)),
                softcap=3.0, scale_multiplier=0.75)


def _vjp(c, **kw):
    return oracle.vjp(c["q"], c["k"], c["v"], c["cu_q"], c["cu_k"], c["alibi_slopes"],
                      c["dout"], c["softcap"], c["scale_multiplier"], **kw)


def _fwd(c, **kw):
    return oracle.forward(c["q"], c["k"], c["v"], c["cu_q"], c["cu_k"], c["alibi_slopes"],
                          c["softcap"], c["scale_multiplier"], **kw)


def test_zero_rate_is_no_dropout():
    rng = np.random.default_rng(1)
    c = _case(rng, [4, 6], [5, 3])
    base = _vjp(c)
    for p in (0.0, np.zeros((10, 2), np.float32)):
        got = _vjp(c, dropout_p=p, dropout_seed=5)
        for name in ("out", "lse", "dq", "dk", "dv"):
            assert np.array_equal(got[name], base[name]), name


def test_dropout_finite_differences():
    """The mask depends on positions only, so the VJP is the exact gradient of
    sum(out * dout) with the mask held fixed: central differences."""
    rng = np.random.default_rng(2)
    c = _case(rng, [3, 2], [4, 3], hq=2, D=3, scale=2.0)
    kw = dict(dropout_p=0.4, dropout_seed=77)
    res = _vjp(c, **kw)
    assert np.any(res["dv"] != _vjp(c)["dv"]), "the mask should drop something"

    def loss(cc):
        out, _ = _fwd(cc, **kw)
        return float((out * c["dout"]).sum())

    h = 1e-6
    for name, grad in (("q", res["dq"]), ("k", res["dk"]), ("v", res["dv"])):
        x = c[name]
        num = np.zeros_like(x)
        for idx in itertools.product(*map(range, x.shape)):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            num[idx] = (loss(dict(c, **{name: xp})) - loss(dict(c, **{name: xm}))) / (2 * h)
        assert np.abs(num - grad).max() <= 1e-7 * max(1.0, np.abs(grad).max()), name


def test_dropout_torch_autograd():
    """An independently written torch float64 expression (mask from the
    counter words, weights dropped after the softmax, autograd) gives the
    same out, dq, dk, dv, with two K/V heads and per-row rates."""
    rng = np.random.default_rng(3)
    lq, lk, hq, hkv, D = [5, 3], [6, 4], 4, 2, 5
    c = _case(rng, lq, lk, hq=hq, hkv=hkv, D=D)
    rates = rng.uniform(0.0, 0.6, size=(8, hq)).astype(np.float32)
    seed = 2024
    res = _vjp(c, dropout_p=rates, dropout_seed=seed)
    q = torch.tensor(c["q"], requires_grad=True)
    k = torch.tensor(c["k"], requires_grad=True)
    v = torch.tensor(c["v"], requires_grad=True)
    sigma = 0.75 / math.sqrt(D)
    outs = []
    for b in range(2):
        q0, q1, k0, k1 = c["cu_q"][b], c["cu_q"][b + 1], c["cu_k"][b], c["cu_k"][b + 1]
        Lq, Lk = q1 - q0, k1 - k0
        rows = []
        for h in range(hq):
            g = h // (hq // hkv)
            s = sigma * q[q0:q1, h] @ k[k0:k1, g].T
            pos = (torch.arange(Lq)[:, None] + (Lk - Lq) - torch.arange(Lk)[None, :]).abs()
            a = 3.0 * torch.tanh(s / 3.0) - float(c["alibi_slopes"][b, h]) * pos.double()
            p = torch.softmax(a, dim=-1)
            words = dr.words(seed, b, h, np.arange(Lq), Lk) >> np.uint64(32)
            thr = np.floor(rates[q0:q1, h].astype(np.float64) * 2.0**32)
            mask = torch.tensor((words.astype(np.float64) >= thr[:, None]).astype(np.float64))
            keep = mask / (1.0 - torch.tensor(rates[q0:q1, h].astype(np.float64)))[:, None]
            rows.append((p * keep) @ v[k0:k1, g])
        outs.append(torch.stack(rows, 1))
    out = torch.cat(outs, 0)
    (out * torch.tensor(c["dout"])).sum().backward()
    for name, ref in (("out", out.detach().numpy()), ("dq", q.grad.numpy()),
                      ("dk", k.grad.numpy()), ("dv", v.grad.numpy())):
        np.testing.assert_allclose(res[name], ref, rtol=1e-12, atol=1e-12, err_msg=name)
    np.testing.assert_allclose(res["delta"], (res["out"] * c["dout"]).sum(-1), rtol=1e-12,
                               atol=1e-13)


def test_dropout_expectation_over_seeds():
    """Averaged over seeds, the scaled dropped output is the undropped one
    (E[m / (1 - p)] = 1): 3000 seeds, within five standard errors."""
    rng = np.random.default_rng(4)
    c = _case(rng, [2], [3], hq=1, D=2)
    ref, _ = _fwd(c)
    outs = np.stack([_fwd(c, dropout_p=0.3, dropout_seed=s)[0] for s in range(3000)])
    mean, se = outs.mean(0), outs.std(0) / math.sqrt(len(outs))
    assert np.all(np.abs(mean - ref) <= 5 * se + 1e-12)


def test_dropout_independent_of_row_chunks_and_sampled_rows():
    """The same words whatever the row chunking, and rows_vjp reproduces the
    rows of the whole sequence (the mask depends on (seed, b, h, i, j) only)."""
    rng = np.random.default_rng(5)
    c = _case(rng, [9], [7], hq=3, D=4)
    rates = np.full((9, 3), 0.35, np.float32)
    args = (c["q"], c["k"], c["v"], c["dout"], c["alibi_slopes"][0], 3.0, 0.75)
    whole = oracle.sequence_vjp(*args, dropout=(11, 4, rates))
    for chunk in (1, 2, 4):
        part = oracle.sequence_vjp(*args, row_chunk=chunk, dropout=(11, 4, rates))
        for name in ("out", "dq", "dk", "dv"):
            np.testing.assert_allclose(part[name], whole[name], rtol=1e-15, atol=1e-15)
    toks, heads = np.array([0, 8, 3, 5]), np.array([2, 0, 1, 1])
    rows = oracle.rows_vjp(*args, toks, heads, dropout=(11, 4, rates))
    for name in ("out", "dq", "delta"):
        np.testing.assert_allclose(rows[name], whole[name][toks, heads], rtol=1e-14, atol=1e-15)


def test_per_row_rates():
    """Rows whose rate is 0 are exactly the undropped rows; a row with rate
    0.75 keeps about a quarter of its keys."""
    rng = np.random.default_rng(6)
    c = _case(rng, [6], [400], hq=2, D=4)
    rates = np.zeros((6, 2), np.float32)
    rates[1::2, :] = 0.75
    got = _vjp(c, dropout_p=rates, dropout_seed=9)
    base = _vjp(c)
    for name in ("out", "dq", "lse"):
        np.testing.assert_array_equal(got[name][0::2], base[name][0::2])
    ks = dr.keep_scale(9, 0, 1, np.array([1, 3, 5]), 400, np.full(3, 0.75, np.float32))
    frac = (ks > 0).mean()
    assert abs(frac - 0.25) < 5 * math.sqrt(0.25 * 0.75 / ks.size)
