"""Pins of the float64 oracle against things other than itself.

Each test ties the oracle to a closed form, a hand-derived example, a
brute-force loop, finite differences, autograd of an independently written
expression, a textbook special case, or an invariant of the definition on
page "Noncausal Global Extreme-GQA Ragged Attention Full VJP" (sections
"What You Have" and "Hard Constraints") and page "python-20261012-ragged-
flash-attention-gradient-recompute" (section "Root causes addressed": empty
rows give L = -inf and zero output/gradients; section "Verification": float64
reference, finite differences, extreme logits).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, lq, lk, hq=2, hkv=1, D=4, scale=1.0, slope_scale=0.5):
    lq = np.asarray(lq)
    lk = np.asarray(lk)
    B = len(lq)
    Tq, Tk = int(lq.sum()), int(lk.sum())
    return dict(
        q=rng.standard_normal((Tq, hq, D)) * scale,
        k=rng.standard_normal((Tk, hkv, D)) * scale,
        v=rng.standard_normal((Tk, hkv, D)),
        dout=rng.standard_normal((Tq, hq, D)),
        cu_q=np.concatenate([[0], np.cumsum(lq)]),
        cu_k=np.concatenate([[0], np.cumsum(lk)]),
        alibi_slopes=rng.uniform(0.0, slope_scale, size=(B, hq)),
        softcap=3.0, scale_multiplier=0.75)


def _vjp(case):
    return oracle.vjp(case["q"], case["k"], case["v"], case["cu_q"], case["cu_k"],
                      case["alibi_slopes"], case["dout"], case["softcap"],
                      case["scale_multiplier"])


def _fwd(case, **over):
    c = dict(case, **over)
    return oracle.forward(c["q"], c["k"], c["v"], c["cu_q"], c["cu_k"], c["alibi_slopes"],
                          c["softcap"], c["scale_multiplier"])


# ---------------------------------------------------------------- worked example
def test_two_key_worked_example():
    """Hand-derived closed form: cap before ALiBi, bottom-right alignment, VJP."""
    with open(os.path.join(GOLDEN, "two_key_worked_example.json")) as f:
        case = json.load(f)
    inp = {k: (np.array(v, dtype=np.float64) if isinstance(v, list) else v)
           for k, v in case["inputs"].items()}
    res = _vjp(inp)
    for name in ("out", "lse", "dq", "dk", "dv"):
        np.testing.assert_allclose(res[name], np.array(case["expected"][name]),
                                   rtol=1e-14, atol=1e-15, err_msg=name)
    # the example separates the page's order from the wrong one
    assert abs(res["out"][0, 0, 0] - case["wrong_order_p"]) > 1e-2


# ---------------------------------------------------------------- closed forms
def _alibi_Z(r, c, Lk):
    """sum_j r^|c - j| for j in [0, Lk): geometric sums on both sides of c."""
    if c < 0:
        return r ** (-c) * (1 - r ** Lk) / (1 - r)
    if c > Lk - 1:
        return r ** (c - Lk + 1) * (1 - r ** Lk) / (1 - r)
    left = (1 - r ** (c + 1)) / (1 - r)          # j = c, c-1, ..., 0
    right = r * (1 - r ** (Lk - 1 - c)) / (1 - r)  # j = c+1, ..., Lk-1
    return left + right


@pytest.mark.parametrize("lq,lk", [(3, 7), (7, 3), (5, 5), (1, 8), (8, 1)])
def test_alibi_closed_form(lq, lk):
    """q = 0 makes every logit -mu |i + Lk - Lq - j|; L and P are geometric sums."""
    D = max(lk, 2)
    mu = 0.37
    case = dict(q=np.zeros((lq, 1, D)), k=np.ones((lk, 1, D)),
                v=np.eye(lk, D)[:, None, :], cu_q=[0, lq], cu_k=[0, lk],
                alibi_slopes=[[mu]], softcap=3.0, scale_multiplier=0.75)
    out, lse = _fwd(case)
    r = math.exp(-mu)
    for i in range(lq):
        c = i + lk - lq
        Z = _alibi_Z(r, c, lk)
        assert abs(lse[i, 0] - math.log(Z)) <= 1e-13 * max(1.0, abs(math.log(Z)))
        for j in range(lk):
            assert abs(out[i, 0, j] - r ** abs(c - j) / Z) <= 1e-14


def test_rows_sum_to_one():
    """A constant value vector is reproduced exactly: every row's weights sum to 1."""
    rng = np.random.default_rng(1)
    case = _rand_case(rng, [4, 9, 1], [6, 2, 11], hq=3, D=5, scale=3.0, slope_scale=2.0)
    const = np.array([0.5, -2.0, 3.0, 7.0, 1e-3])
    case["v"] = np.broadcast_to(const, case["v"].shape).copy()
    out, _ = _fwd(case)
    np.testing.assert_allclose(out, np.broadcast_to(const, out.shape), rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- brute force
def _brute_forward(case):
    q, k, v = case["q"], case["k"], case["v"]
    cu_q, cu_k, slopes = case["cu_q"], case["cu_k"], case["alibi_slopes"]
    c, sm = case["softcap"], case["scale_multiplier"]
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    sigma = sm / math.sqrt(D)
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(Tq)]
    lse = [[-math.inf] * Hq for _ in range(Tq)]
    for b in range(len(cu_q) - 1):
        q0, Lq = int(cu_q[b]), int(cu_q[b + 1] - cu_q[b])
        k0, Lk = int(cu_k[b]), int(cu_k[b + 1] - cu_k[b])
        for h in range(Hq):
            g = h * Hkv // Hq
            for i in range(Lq):
                if Lk == 0:
                    continue
                a = []
                for j in range(Lk):
                    s = sigma * math.fsum(q[q0 + i, h, d] * k[k0 + j, g, d] for d in range(D))
                    t = c * math.tanh(s / c) if c > 0 else s
                    a.append(t - slopes[b][h] * abs(i + Lk - Lq - j))
                m = max(a)
                e = [math.exp(x - m) for x in a]
                Z = math.fsum(e)
                lse[q0 + i][h] = m + math.log(Z)
                for d in range(D):
                    out[q0 + i][h][d] = math.fsum(e[j] / Z * v[k0 + j, g, d] for j in range(Lk))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_forward(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    lq = rng.integers(0, 7, size=B)
    lk = rng.integers(0, 7, size=B)
    hq = int(rng.choice([1, 2, 4]))
    hkv = 2 if hq == 4 and seed % 2 else 1
    case = _rand_case(rng, lq, lk, hq=hq, hkv=hkv, D=int(rng.integers(1, 9)), scale=2.0)
    if seed == 3:
        case["softcap"] = 0.0
    out, lse = _fwd(case)
    bout, blse = _brute_forward(case)
    np.testing.assert_allclose(out, bout, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(blse))
    fin = np.isfinite(blse)
    np.testing.assert_allclose(lse[fin], blse[fin], rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- backward
def test_finite_differences():
    """Central differences of sum(out * dout) w.r.t. every element of q, k, v."""
    rng = np.random.default_rng(7)
    case = _rand_case(rng, [3, 2, 0], [4, 1, 2], hq=2, D=4, scale=2.0)
    res = _vjp(case)

    def loss(c):
        out, _ = _fwd(c)
        return float((out * case["dout"]).sum())

    h = 1e-6
    for name, grad in (("q", res["dq"]), ("k", res["dk"]), ("v", res["dv"])):
        x = case[name]
        num = np.zeros_like(x)
        for idx in itertools.product(*map(range, x.shape)):
            xp = x.copy()
            xp[idx] += h
            xm = x.copy()
            xm[idx] -= h
            num[idx] = (loss(dict(case, **{name: xp})) - loss(dict(case, **{name: xm}))) / (2 * h)
        err = np.abs(num - grad).max()
        assert err <= 1e-7 * max(1.0, np.abs(grad).max()), (name, err)


def _torch_autograd(case):
    """Independent expression: all heads batched, torch softmax, autograd backward."""
    q = torch.tensor(case["q"], requires_grad=True)
    k = torch.tensor(case["k"], requires_grad=True)
    v = torch.tensor(case["v"], requires_grad=True)
    dout = torch.tensor(case["dout"])
    slopes = torch.tensor(np.asarray(case["alibi_slopes"], dtype=np.float64))
    c, sm = case["softcap"], case["scale_multiplier"]
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    sigma = sm / math.sqrt(D)
    outs = []
    cu_q, cu_k = case["cu_q"], case["cu_k"]
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        Lq, Lk = q1 - q0, k1 - k0
        if Lk == 0:
            outs.append(torch.zeros(Lq, Hq, D, dtype=torch.float64))
            continue
        Qb = q[q0:q1].permute(1, 0, 2)                                  # Hq, Lq, D
        Kb = k[k0:k1].permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)  # Hq, Lk, D
        Vb = v[k0:k1].permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        S = sigma * torch.matmul(Qb, Kb.transpose(1, 2).contiguous())
        T = c * torch.tanh(S / c) if c > 0 else S
        pos = (torch.arange(Lq)[:, None] + (Lk - Lq) - torch.arange(Lk)[None, :]).abs()
        A = T - slopes[b][:, None, None] * pos.to(torch.float64)[None]
        P = torch.softmax(A, dim=-1)
        outs.append(torch.matmul(P, Vb).permute(1, 0, 2))
    out = torch.cat(outs, 0)
    (out * dout).sum().backward()
    return out.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("seed", range(3))
def test_torch_autograd(seed):
    rng = np.random.default_rng(100 + seed)
    B = 3
    lq = rng.integers(0, 12, size=B)
    lk = rng.integers(1, 12, size=B)
    hq = [2, 6, 4][seed]
    hkv = [1, 1, 2][seed]
    case = _rand_case(rng, lq, lk, hq=hq, hkv=hkv, D=6, scale=2.5, slope_scale=1.0)
    if seed == 1:
        case["softcap"] = 0.0
    res = _vjp(case)
    out, dq, dk, dv = _torch_autograd(case)
    for name, ref in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_allclose(res[name], ref, rtol=1e-12, atol=1e-12, err_msg=name)


def test_textbook_sdpa_reduction():
    """Zero slopes and no cap reduce to scaled dot-product attention (torch CPU float64)."""
    rng = np.random.default_rng(5)
    lq, lk, hq, D = 7, 9, 4, 8
    case = _rand_case(rng, [lq], [lk], hq=hq, D=D, scale=1.5)
    case["alibi_slopes"] = np.zeros((1, hq))
    sigma = 0.75 / math.sqrt(D)
    q = torch.tensor(case["q"]).permute(1, 0, 2)[None].requires_grad_(True)
    k = torch.tensor(case["k"]).permute(1, 0, 2).expand(hq, lk, D)[None].contiguous().requires_grad_(True)
    v = torch.tensor(case["v"]).permute(1, 0, 2).expand(hq, lk, D)[None].contiguous().requires_grad_(True)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=sigma)
    ref.backward(torch.tensor(case["dout"]).permute(1, 0, 2)[None])
    ref_out = ref[0].permute(1, 0, 2).detach().numpy()
    ref_dq = q.grad[0].permute(1, 0, 2).numpy()
    ref_dk = k.grad[0].sum(0)[:, None, :].numpy()
    ref_dv = v.grad[0].sum(0)[:, None, :].numpy()
    for softcap in (0.0, 1e12):
        case["softcap"] = softcap
        res = _vjp(case)
        tol = 1e-12 if softcap == 0.0 else 1e-10
        np.testing.assert_allclose(res["out"], ref_out, rtol=tol, atol=tol)
        np.testing.assert_allclose(res["dq"], ref_dq, rtol=tol, atol=tol)
        np.testing.assert_allclose(res["dk"], ref_dk, rtol=tol, atol=tol)
        np.testing.assert_allclose(res["dv"], ref_dv, rtol=tol, atol=tol)


def test_delta_is_rowdot_of_out_and_dout():
    rng = np.random.default_rng(9)
    case = _rand_case(rng, [5, 3], [4, 6], hq=3, D=5, scale=2.0)
    res = _vjp(case)
    np.testing.assert_allclose(res["delta"], (res["out"] * case["dout"]).sum(-1),
                               rtol=1e-12, atol=1e-13)


def test_softcap_derivative_matches_tanh_identity():
    """d/ds [c tanh(s/c)] = 1 - tanh^2(s/c), by central differences."""
    c = 3.0
    for s in (-40.0, -3.0, -0.2, 0.0, 0.7, 5.0, 25.0):
        h = 1e-6
        num = (c * math.tanh((s + h) / c) - c * math.tanh((s - h) / c)) / (2 * h)
        assert abs(num - (1 - math.tanh(s / c) ** 2)) < 1e-8


# ---------------------------------------------------------------- special cases
def test_single_key_sequence():
    """Lk = 1: P = 1, out = v0, dq = dk = 0, dv0 = sum of dout over rows and heads."""
    rng = np.random.default_rng(11)
    case = _rand_case(rng, [5], [1], hq=3, D=4, scale=2.0)
    res = _vjp(case)
    np.testing.assert_allclose(res["out"], np.broadcast_to(case["v"][0, 0], res["out"].shape),
                               rtol=0, atol=1e-15)
    assert np.abs(res["dq"]).max() <= 1e-15
    assert np.abs(res["dk"]).max() <= 1e-14
    np.testing.assert_allclose(res["dv"][0, 0], case["dout"].sum((0, 1)), rtol=1e-14, atol=1e-14)


def test_empty_sequences():
    """Lq = 0 leaves dk = dv = 0; Lk = 0 gives out = dq = 0 and lse = -inf, no NaN."""
    rng = np.random.default_rng(12)
    case = _rand_case(rng, [0, 4, 3], [5, 0, 2], hq=2, D=4, scale=2.0)
    res = _vjp(case)
    assert np.all(res["dk"][0:5] == 0) and np.all(res["dv"][0:5] == 0)
    assert np.all(res["out"][0:4] == 0) and np.all(res["dq"][0:4] == 0)
    assert np.all(np.isneginf(res["lse"][0:4]))
    assert np.isfinite(res["lse"][4:]).all()
    for name in ("out", "dq", "dk", "dv"):
        assert np.isfinite(res[name]).all()
    assert np.abs(res["dk"][5:]).max() > 0


def test_extreme_logits_finite():
    """Logits from 1e-8 to 1e6: the cap saturates, outputs and gradients stay finite,
    and a fully saturated logit passes (numerically) no gradient to q."""
    rng = np.random.default_rng(13)
    for scale in (1e-8, 1.0, 1e3, 1e6):
        case = _rand_case(rng, [3, 4], [5, 2], hq=2, D=4, scale=scale)
        res = _vjp(case)
        for name in ("out", "dq", "dk", "dv", "lse"):
            assert np.isfinite(res[name]).all(), (scale, name)
    case = _rand_case(rng, [1], [2], hq=1, D=1, scale=1.0)
    case["q"][:] = 1e6
    case["k"][:] = np.array([[[1.0]], [[-1.0]]]) * 1e6
    res = _vjp(case)
    assert np.abs(res["dq"]).max() == 0.0


# ---------------------------------------------------------------- invariants
def test_head_sum_invariant():
    """dk/dv of Hq heads over one K/V head equal the sum of single-head runs."""
    rng = np.random.default_rng(21)
    case = _rand_case(rng, [4, 6], [5, 3], hq=3, D=4, scale=2.0)
    full = _vjp(case)
    dk = np.zeros_like(full["dk"])
    dv = np.zeros_like(full["dv"])
    for h in range(3):
        one = dict(case, q=case["q"][:, h:h + 1], dout=case["dout"][:, h:h + 1],
                   alibi_slopes=case["alibi_slopes"][:, h:h + 1])
        r = _vjp(one)
        dk += r["dk"]
        dv += r["dv"]
        np.testing.assert_allclose(r["dq"][:, 0], full["dq"][:, h], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dk, full["dk"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dv, full["dv"], rtol=1e-13, atol=1e-14)


def test_linearity():
    """out is linear in v; dq, dk, dv are linear in dout."""
    rng = np.random.default_rng(22)
    case = _rand_case(rng, [4, 2], [3, 5], hq=2, D=4, scale=2.0)
    v2 = rng.standard_normal(case["v"].shape)
    o1, _ = _fwd(case)
    o2, _ = _fwd(case, v=v2)
    o12, _ = _fwd(case, v=2.0 * case["v"] - 3.0 * v2)
    np.testing.assert_allclose(o12, 2.0 * o1 - 3.0 * o2, rtol=1e-13, atol=1e-13)
    d2 = rng.standard_normal(case["dout"].shape)
    r1 = _vjp(case)
    r2 = _vjp(dict(case, dout=d2))
    r12 = _vjp(dict(case, dout=0.5 * case["dout"] + 4.0 * d2))
    for name in ("dq", "dk", "dv"):
        np.testing.assert_allclose(r12[name], 0.5 * r1[name] + 4.0 * r2[name],
                                   rtol=1e-12, atol=1e-13)


def test_sequence_permutation():
    """Permuting sequences together with their slope rows permutes every output."""
    rng = np.random.default_rng(23)
    lq, lk = np.array([3, 0, 5, 2]), np.array([4, 2, 1, 6])
    case = _rand_case(rng, lq, lk, hq=2, D=4, scale=2.0)
    res = _vjp(case)
    perm = [2, 0, 3, 1]
    cu_q, cu_k = case["cu_q"], case["cu_k"]
    qi = np.concatenate([np.arange(cu_q[b], cu_q[b + 1]) for b in perm]).astype(int)
    ki = np.concatenate([np.arange(cu_k[b], cu_k[b + 1]) for b in perm]).astype(int)
    pcase = dict(case, q=case["q"][qi], dout=case["dout"][qi], k=case["k"][ki], v=case["v"][ki],
                 cu_q=np.concatenate([[0], np.cumsum(lq[perm])]),
                 cu_k=np.concatenate([[0], np.cumsum(lk[perm])]),
                 alibi_slopes=case["alibi_slopes"][perm])
    pres = _vjp(pcase)
    for name, idx in (("out", qi), ("dq", qi), ("lse", qi), ("dk", ki), ("dv", ki)):
        np.testing.assert_array_equal(pres[name], res[name][idx])


def test_rows_vjp_matches_sequence():
    """The sampled-row entry returns exactly the rows of the full sequence result."""
    rng = np.random.default_rng(24)
    case = _rand_case(rng, [9], [7], hq=3, D=5, scale=2.0)
    full = oracle.sequence_vjp(case["q"], case["k"], case["v"], case["dout"],
                               case["alibi_slopes"][0], 3.0, 0.75)
    toks = np.array([0, 8, 3, 3, 5])
    heads = np.array([2, 0, 1, 0, 2])
    part = oracle.rows_vjp(case["q"], case["k"], case["v"], case["dout"],
                           case["alibi_slopes"][0], 3.0, 0.75, toks, heads)
    for name in ("out", "dq", "lse", "delta"):
        np.testing.assert_allclose(part[name], full[name][toks, heads], rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- causal / window masks
# The pages name causal, window_left and window_right without defining them;
# the reading pinned here keeps key j of row i iff
# i + Lk - Lq - window_left <= j <= i + Lk - Lq + window_right (negative = no
# bound, causal = right bound 0).

def _vjp_w(case, causal=False, wl=-1, wr=-1):
    return oracle.vjp(case["q"], case["k"], case["v"], case["cu_q"], case["cu_k"],
                      case["alibi_slopes"], case["dout"], case["softcap"],
                      case["scale_multiplier"], causal=causal, window_left=wl, window_right=wr)


def test_window_bounds_reading():
    assert oracle.window_bounds(False, -1, -1) == (-1, -1)
    assert oracle.window_bounds(True, -1, -1) == (-1, 0)
    assert oracle.window_bounds(True, 5, 7) == (5, 0)
    assert oracle.window_bounds(False, 3, 0) == (3, 0)


def test_window_zero_width_is_one_key():
    """window (0, 0): each row keeps only the key at its centre i + Lk - Lq, so
    out = v_centre, L = its logit, dq = dk = 0 and dv_c = sum of dout over the
    rows centred on c; rows whose centre lies before key 0 keep nothing."""
    rng = np.random.default_rng(31)
    case = _rand_case(rng, [6, 3], [4, 9], hq=3, D=5, scale=1.5)
    res = _vjp_w(case, wl=0, wr=0)
    sigma = case["scale_multiplier"] / math.sqrt(5)
    dv = np.zeros_like(case["v"])
    for b in range(2):
        q0, q1 = case["cu_q"][b], case["cu_q"][b + 1]
        k0, k1 = case["cu_k"][b], case["cu_k"][b + 1]
        Lq, Lk = q1 - q0, k1 - k0
        for i in range(Lq):
            c = i + Lk - Lq
            for h in range(3):
                if c < 0:
                    assert res["lse"][q0 + i, h] == -np.inf
                    assert np.all(res["out"][q0 + i, h] == 0)
                    continue
                np.testing.assert_allclose(res["out"][q0 + i, h], case["v"][k0 + c, 0], atol=1e-15)
                s = sigma * case["q"][q0 + i, h] @ case["k"][k0 + c, 0]
                assert abs(res["lse"][q0 + i, h] - 3.0 * math.tanh(s / 3.0)) < 1e-14
                dv[k0 + c, 0] += case["dout"][q0 + i, h]
    assert np.abs(res["dq"]).max() <= 1e-14 and np.abs(res["dk"]).max() <= 1e-14
    np.testing.assert_allclose(res["dv"], dv, atol=1e-14)


def test_no_bounds_is_noncausal():
    rng = np.random.default_rng(32)
    case = _rand_case(rng, [4, 7], [9, 3], hq=2)
    a, b = _vjp(case), _vjp_w(case, False, -1, -1)
    for key in ("out", "lse", "dq", "dk", "dv"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("lq,lk", [(5, 11), (9, 4), (7, 7)])
@pytest.mark.parametrize("causal,wl,wr", [(True, -1, -1), (True, 2, -1), (False, 3, 0),
                                          (False, 0, 2), (False, 2, 5), (False, -1, 3),
                                          (False, 4, -1)])
def test_window_row_equals_unmasked_slice(lq, lk, causal, wl, wr):
    """Each masked row equals the unmasked oracle on the keys it keeps: row i
    of the masked problem is placed at position i' = c - lo of a square
    problem over keys lo..hi (c = i + Lk - Lq), whose centre i' + 0 sits at
    the same distance from every key; other rows of the square problem are
    zero (zero q and dout rows add nothing to dK / dV).  dK / dV of the masked
    problem are the sums of the slices' dK / dV over rows and heads."""
    rng = np.random.default_rng(100 + lq * 13 + lk)
    hq, D = 2, 4
    case = _rand_case(rng, [lq], [lk], hq=hq, D=D, scale=1.3)
    res = _vjp_w(case, causal, wl, wr)
    ewl, ewr = oracle.window_bounds(causal, wl, wr)
    dk = np.zeros_like(case["k"])
    dv = np.zeros_like(case["v"])
    for i in range(lq):
        c = i + lk - lq
        lo = max(0, c - ewl) if ewl >= 0 else 0
        hi = min(lk - 1, c + ewr) if ewr >= 0 else lk - 1
        for h in range(hq):
            if lo > hi:
                assert res["lse"][i, h] == -np.inf and np.all(res["out"][i, h] == 0)
                assert np.all(res["dq"][i, h] == 0)
                continue
            n = hi - lo + 1
            # a problem over keys lo..hi whose row i' has centre i' + n - Lq' =
            # c - lo (before key 0 when the row's centre is clamped)
            ip = c - lo
            Lqs, ir = n - min(ip, 0), max(ip, 0)
            sq = np.zeros((Lqs, 1, D))
            sd = np.zeros((Lqs, 1, D))
            sq[ir, 0] = case["q"][i, h]
            sd[ir, 0] = case["dout"][i, h]
            part = oracle.sequence_vjp(sq, case["k"][lo:hi + 1], case["v"][lo:hi + 1], sd,
                                       case["alibi_slopes"][0][h:h + 1], case["softcap"],
                                       case["scale_multiplier"])
            np.testing.assert_allclose(res["out"][i, h], part["out"][ir, 0], rtol=0, atol=1e-13)
            np.testing.assert_allclose(res["lse"][i, h], part["lse"][ir, 0], rtol=0, atol=1e-13)
            np.testing.assert_allclose(res["dq"][i, h], part["dq"][ir, 0], rtol=0, atol=1e-13)
            dk[lo:hi + 1] += part["dk"]
            dv[lo:hi + 1] += part["dv"]
    np.testing.assert_allclose(res["dk"], dk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["dv"], dv, rtol=0, atol=1e-12)


def test_window_mirror_symmetry():
    """With Lq = Lk, reversing the order of queries and keys maps centre i to
    centre Lq - 1 - i and swaps the two window bounds."""
    rng = np.random.default_rng(33)
    case = _rand_case(rng, [9], [9], hq=2, D=4)
    a = _vjp_w(case, False, 1, 4)
    rev = dict(case, q=case["q"][::-1].copy(), k=case["k"][::-1].copy(), v=case["v"][::-1].copy(),
               dout=case["dout"][::-1].copy())
    b = _vjp_w(rev, False, 4, 1)
    for key in ("out", "lse", "dq", "dk", "dv"):
        np.testing.assert_allclose(a[key], b[key][::-1], rtol=0, atol=1e-13, err_msg=key)


# ---------------------------------------------------------------- row chunking
def test_row_chunks_do_not_change_the_result():
    """sequence_vjp splits a head's query rows into chunks to bound memory; every
    chunk size gives the same result (each row's softmax spans all keys), which
    exercises the chunk boundaries that long sequences reach."""
    rng = np.random.default_rng(25)
    case = _rand_case(rng, [7], [6], hq=3, D=5, scale=2.0)
    args = (case["q"], case["k"], case["v"], case["dout"], case["alibi_slopes"][0], 3.0, 0.75)
    whole = oracle.sequence_vjp(*args, row_chunk=4096)
    for chunk in (1, 2, 3, 6):
        part = oracle.sequence_vjp(*args, row_chunk=chunk)
        for name in ("out", "lse", "dq", "delta", "dk", "dv"):
            np.testing.assert_allclose(part[name], whole[name], rtol=1e-15, atol=1e-15,
                                       err_msg=f"chunk {chunk} {name}")
    for chunk in (2, 5):
        a = oracle.sequence_vjp(*args, row_chunk=chunk, window=(1, 2))
        b = oracle.sequence_vjp(*args, window=(1, 2))
        for name in ("out", "lse", "dq", "dk", "dv"):
            np.testing.assert_allclose(a[name], b[name], rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("causal,wl,wr", [(True, -1, -1), (False, 2, 1), (False, -1, 0)])
def test_rows_vjp_matches_sequence_with_mask(causal, wl, wr):
    rng = np.random.default_rng(26)
    case = _rand_case(rng, [9], [5], hq=3, D=5, scale=2.0)
    full = oracle.sequence_vjp(case["q"], case["k"], case["v"], case["dout"],
                               case["alibi_slopes"][0], 3.0, 0.75,
                               window=oracle.window_bounds(causal, wl, wr))
    toks = np.array([0, 8, 3, 1, 5, 6])
    heads = np.array([2, 0, 1, 0, 2, 1])
    part = oracle.rows_vjp(case["q"], case["k"], case["v"], case["dout"],
                           case["alibi_slopes"][0], 3.0, 0.75, toks, heads, causal=causal,
                           window_left=wl, window_right=wr)
    for name in ("out", "dq", "lse", "delta"):
        np.testing.assert_array_equal(np.isneginf(part[name]), np.isneginf(full[name][toks, heads]))
        fin = np.isfinite(full[name][toks, heads])
        np.testing.assert_allclose(part[name][fin], full[name][toks, heads][fin],
                                   rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- negative slopes
@pytest.mark.parametrize("lq,lk", [(3, 7), (7, 3), (5, 5)])
def test_alibi_closed_form_negative_slope(lq, lk):
    """A negative slope rewards distance: with q = 0 the weights are r^|c - j|
    with r = e^{-mu} > 1, and the same geometric sums give L and P."""
    D = max(lk, 2)
    mu = -0.45
    case = dict(q=np.zeros((lq, 1, D)), k=np.ones((lk, 1, D)),
                v=np.eye(lk, D)[:, None, :], cu_q=[0, lq], cu_k=[0, lk],
                alibi_slopes=[[mu]], softcap=3.0, scale_multiplier=0.75)
    out, lse = _fwd(case)
    r = math.exp(-mu)
    for i in range(lq):
        c = i + lk - lq
        Z = _alibi_Z(r, c, lk)
        assert abs(lse[i, 0] - math.log(Z)) <= 1e-13 * max(1.0, abs(math.log(Z)))
        for j in range(lk):
            assert abs(out[i, 0, j] - r ** abs(c - j) / Z) <= 1e-14
