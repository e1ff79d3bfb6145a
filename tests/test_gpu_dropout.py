"""Counter-based dropout on the HIP path against the float64 oracle.

Page "python-20261012-ragged-flash-attention-gradient-recompute", section
"Root causes addressed": a counter-based splitmix64 hash of (seed, b, h, row,
col), rebuilt identically by every pass whatever the tiling, with one rate or
per-row rates; section "Verification": determinism across tile sizes and
correct per-row rates.  The composition of the hash is the reading in
oracle/dropout.py, which the oracle's own tests pin.

* the keep decisions themselves: with q = 0, zero slopes and one-hot V rows,
  out[i, h, j] = mask * scale / Lk, so the GPU's mask must equal the oracle's
  bit for bit (an integer decision on both sides);
* out, dq, dk, dv and lse against the oracle, both dS modes, scalar and
  per-row rates, masks, no cap, K/V heads and head dimensions;
* the same mask whatever the schedule: the fused call, the separate forward
  and backward entries, every-key evaluation (other key-step ranges, so other
  dK/dV work splits) and stored vs recomputed dS agree bitwise on out and lse;
  the fused variants' dk / dv agree to FP32 summation order.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import dropout as odr
import ragged_gqa_attention_amd as rga
import workloads as W
from tests.gpu_util import TOL, assert_close, assert_lse, need_gpu, say, to_np

pytestmark = pytest.mark.gpu


def _oracle(wl, p, seed, rates=None, **mask):
    inp = W.oracle_inputs(wl)
    return oracle.vjp(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"],
                      inp["alibi_slopes"], inp["dout"], inp["softcap"], inp["scale_multiplier"],
                      dropout_p=p if rates is None else rates.cpu().numpy(),
                      dropout_seed=seed, **mask)


def _call(g, p, seed, rates=None, store_ds=True, **kw):
    res = rga.attn_varlen_full_vjp(g.q, g.k, g.v, g.cu_q, g.cu_k, g.slopes, g.dout,
                                   softcap=g.softcap, scale_multiplier=g.scale_multiplier,
                                   want_lse=True, check=True, store_ds=store_ds, dropout_p=p,
                                   dropout_seed=seed, dropout_rates=rates, **kw)
    torch.cuda.synchronize()
    return dict(zip(("out", "dq", "dk", "dv", "lse"), res))


@pytest.mark.parametrize("p,seed", [(0.3, 12345), (0.875, 2**63 + 17)])
def test_keep_pattern_is_the_oracles(p, seed):
    """q = 0 and zero slopes make every weight 1 / Lk; with v_j = e_j the
    output row is the row's kept keys times scale / Lk."""
    need_gpu()
    lq, lk, hq = [7, 40, 3], [100, 160, 1], 8
    wl = W.custom_workload(lq=lq, lk=lk, hq=hq, dtype="bf16", width=160, step=1, seed=5,
                           slopes=np.zeros((3, hq), np.float32))
    for t in wl.bufs.values():
        t.zero_()
    for b in range(3):
        k0 = int(wl.cu_k[b])
        for j in range(lk[b]):
            wl.v[k0 + j, 0, j] = 1.0
    g = wl.to("cuda")
    got = to_np(_call(g, p, seed)["out"])
    scale = 1.0 / (1.0 - float(np.float32(p)))
    for b in range(3):
        q0, k0 = int(wl.cu_q[b]), int(wl.cu_k[b])
        for h in range(hq):
            want = odr.keep_scale(seed, b, h, np.arange(lq[b]), lk[b],
                                  np.full(lq[b], p, np.float32)) > 0
            mask = got[q0:q0 + lq[b], h, :lk[b]] != 0
            assert np.array_equal(mask, want), (b, h)
            assert np.allclose(got[q0:q0 + lq[b], h, :lk[b]][want], scale / lk[b], rtol=1e-2)


CASES = {
    "bf16": dict(lq=[37, 130, 9, 0], lk=[300, 90, 200, 17], hq=48, dtype="bf16", width=192,
                 step=2),
    "f16_long_keys": dict(lq=[20, 64], lk=[1500, 700], hq=64, dtype="f16", width=176, step=3),
    "hkv4_d128": dict(lq=[33, 70, 5], lk=[129, 64, 300], hq=16, hkv=4, head_dim=128,
                      dtype="bf16", width=128, step=1),
    "hkv2_d64": dict(lq=[50, 1], lk=[80, 90], hq=8, hkv=2, head_dim=64, dtype="f16", width=96,
                     step=2),
}


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("p", [0.1, 0.5])
def test_dropout_parity(case, p):
    need_gpu()
    wl = W.custom_workload(seed=11, **CASES[case])
    g = wl.to("cuda")
    ref = _oracle(wl, p, 777)
    tol = TOL[wl.dtype]
    for store_ds in (True, False):
        lab = f"{case} p={p} ds={store_ds}"
        say(f"[{lab}]")
        got = _call(g, p, 777, store_ds=store_ds)
        for name in ("out", "dq", "dk", "dv"):
            assert_close(name, to_np(got[name]), ref[name], tol, lab)
        assert_lse(to_np(got["lse"]), ref["lse"], lab)


@pytest.mark.parametrize("causal,wl_,wr,softcap", [(True, -1, -1, 3.0), (False, 30, 4, 3.0),
                                                   (False, -1, -1, 0.0)])
def test_dropout_with_masks_and_no_cap(causal, wl_, wr, softcap):
    need_gpu()
    wl = W.custom_workload(lq=[37, 130, 9], lk=[300, 90, 200], hq=32, dtype="bf16", width=160,
                           step=1, seed=12, softcap=softcap)
    g = wl.to("cuda")
    mask = dict(causal=causal, window_left=wl_, window_right=wr)
    ref = _oracle(wl, 0.25, 99, **mask)
    for store_ds in (True, False):
        lab = f"dropout mask=({causal},{wl_},{wr}) cap={softcap} ds={store_ds}"
        got = _call(g, 0.25, 99, store_ds=store_ds, **mask)
        for name in ("out", "dq", "dk", "dv"):
            assert_close(name, to_np(got[name]), ref[name], TOL[wl.dtype], lab)
        assert_lse(to_np(got["lse"]), ref["lse"], lab)


def test_per_row_rates():
    """Per-row rates [Tq, Hq] (zero on every third row), against the oracle;
    rows with rate 0 match the undropped call to rounding: the undropped
    forward forms the ALiBi bias of key steps wholly before every centre of
    a wave as slope2 j + const, the dropout forward always as
    -slope2 |c - j| (the same value up to one rounding of slope2 c)."""
    need_gpu()
    wl = W.custom_workload(lq=[37, 130], lk=[300, 90], hq=16, dtype="f16", width=176, step=2,
                           seed=13)
    g = wl.to("cuda")
    rng = np.random.default_rng(3)
    rates = rng.uniform(0.0, 0.8, size=(wl.total_q, wl.hq)).astype(np.float32)
    rates[::3] = 0.0
    rates_g = torch.from_numpy(rates).cuda()
    ref = _oracle(wl, 0.0, 4242, rates=rates_g)
    tol = TOL[wl.dtype]
    for store_ds in (True, False):
        got = _call(g, 0.0, 4242, rates=rates_g, store_ds=store_ds)
        for name in ("out", "dq", "dk", "dv"):
            assert_close(name, to_np(got[name]), ref[name], tol, f"rates ds={store_ds}")
        assert_lse(to_np(got["lse"]), ref["lse"], "rates")
    plain = _call(g, 0.0, 0)
    x, y = got["out"][::3].float(), plain["out"][::3].float()
    ulp = torch.finfo(plain["out"].dtype).eps
    assert ((x - y).abs() <= 2 * ulp * y.abs() + 2.0 ** -24).all()
    # L is that of the undropped weights on every row
    lx, ly = got["lse"].float(), plain["lse"].float()
    fin = torch.isfinite(ly)
    assert torch.equal(torch.isfinite(lx), fin)
    assert ((lx - ly)[fin].abs() <= 1e-5 * (1.0 + ly[fin].abs())).all()


def test_same_mask_whatever_the_schedule():
    """The fused call, stored vs recomputed dS, every-key evaluation (other
    key-step ranges, hence other dK/dV splits) and the separate entries: out
    and lse bitwise equal; dk / dv of the fused variants equal to FP32
    summation order and dq equal where dS is formed the same way; three
    repeats bitwise equal; every variant within tolerance of the oracle."""
    need_gpu()
    wl = W.custom_workload(lq=[37, 5, 300, 64], lk=[3000, 900, 1100, 1], hq=64, dtype="bf16",
                           width=160, step=2, seed=14)
    g = wl.to("cuda")
    p, seed = 0.2, 31337
    base = _call(g, p, seed, store_ds=True)
    runs = {"recompute": _call(g, p, seed, store_ds=False),
            "all_keys": _call(g, p, seed, store_ds=True, all_keys=True)}
    out, lse = rga.attn_varlen_fwd(g.q, g.k, g.v, g.cu_q, g.cu_k, g.slopes, g.softcap,
                                   g.scale_multiplier, dropout_p=p, dropout_seed=seed)
    dq, dk, dv = rga.attn_varlen_bwd(g.q, g.k, g.v, out, lse, g.dout, g.cu_q, g.cu_k, g.slopes,
                                     g.softcap, g.scale_multiplier, dropout_p=p,
                                     dropout_seed=seed, store_ds=True)
    torch.cuda.synchronize()
    for name, r in runs.items():
        assert torch.equal(r["out"], base["out"]), name
        assert torch.equal(r["lse"], base["lse"]), name
        for t in ("dk", "dv"):
            x, y = r[t].float(), base[t].float()
            bound = torch.finfo(base[t].dtype).eps * torch.maximum(x.abs(), y.abs())
            bound = bound + 2.0 ** -16 * y.abs().max()
            assert not ((x - y).abs() > bound).any(), (name, t)
    assert torch.equal(runs["all_keys"]["dq"], base["dq"])
    for _ in range(2):
        again = _call(g, p, seed, store_ds=True)
        for t in ("out", "dq", "dk", "dv", "lse"):
            assert torch.equal(again[t], base[t]), t
    # the separate entries: the same mask (out bitwise equal); the backward
    # rebuilds P from the natural-log L and Delta from the stored 16-bit
    # output, so its gradients match the oracle to the tolerance, not the
    # fused bits.  A row whose only key is kept has exact dS = dP - Delta = 0;
    # from a stored output scaled by 1 / (1 - p) the two differ by that
    # output's rounding, summed over the sequence's 4096 rows into dk, so the
    # single-key sequence (the last) is compared in the fused call only.
    assert torch.equal(out, base["out"]) and torch.equal(lse, base["lse"])
    ref = _oracle(wl, p, seed)
    for t, x in (("out", base["out"]), ("dq", base["dq"]), ("dk", base["dk"]), ("dv", base["dv"])):
        assert_close(t, to_np(x), ref[t], TOL[wl.dtype], "schedule case fused")
    nq, nk = int(wl.cu_q[3]), int(wl.cu_k[3])
    for t, x, n in (("dq", dq, nq), ("dk", dk, nk), ("dv", dv, nk)):
        assert_close(t, to_np(x[:n]), ref[t][:n], TOL[wl.dtype], "schedule case separate")
