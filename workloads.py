"""Seeded synthetic workloads for ragged extreme-GQA attention.

This module only draws inputs: sequence lengths, ALiBi slopes and Gaussian
activations, stored in NaN-poisoned padded buffers and exposed as strided
views.  It holds none of the attention arithmetic, so both the HIP path and
the float64 oracle can consume the same draws.

The shapes follow the problem family on page "Noncausal Global Extreme-GQA
Ragged Attention Full VJP", section "What You Have": 18-52 ragged sequences,
Q much shorter than K in some and the reverse in others; 48/64/80/96 query
heads over one K/V head; head dim 160; FP16 or BF16; views with a padded
feature axis and a token step of 2 or 3; FP32 slopes [batch, q_heads];
scale 0.75/sqrt(160) and soft cap 3.  The page's own panel and sealed cases
are not available; these seeded draws stand in for them.

Recipe (``numpy.random.default_rng([config, trial])``, draws in this order):
lengths, slopes ``2**(-8 (h+1) / Hq) * U(0.5, 1.5)`` per (sequence, head),
then q, k, v, dout as float32 N(0, 1) times the config's value scale, each
rounded to nearest-even into the 16-bit dtype.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

HEAD_DIM = 160

# name, batch, hq, dtype, width, step, value scale, length rule
CONFIGS = {
    0: dict(name="tiny_ragged_gqa", batch=3, hq=48, dtype="f16", width=176, step=2, scale=1.0),
    1: dict(name="q_short_k_long", batch=24, hq=64, dtype="bf16", width=192, step=2, scale=1.0),
    2: dict(name="q_long_k_short", batch=36, hq=80, dtype="f16", width=176, step=3, scale=1.5),
    3: dict(name="mixed_extreme", batch=52, hq=96, dtype="bf16", width=192, step=3, scale=1.0),
    4: dict(name="balanced_long", batch=18, hq=48, dtype="f16", width=176, step=2, scale=1.0),
}

TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


def _loguniform_lengths(rng, n):
    # floor(exp(U(0, ln 4097))) clipped to [1, 4096]
    x = np.floor(np.exp(rng.uniform(0.0, math.log(4097.0), size=n))).astype(np.int64)
    return np.clip(x, 1, 4096)


def draw_lengths(cfg: int, rng: np.random.Generator):
    c = CONFIGS[cfg]
    B = c["batch"]
    if cfg == 0:
        return np.array([5, 17, 33], np.int64), np.array([40, 9, 64], np.int64)
    if cfg == 1:
        return rng.integers(16, 129, size=B), rng.integers(512, 2049, size=B)
    if cfg == 2:
        return rng.integers(512, 2049, size=B), rng.integers(32, 257, size=B)
    if cfg == 3:
        lq = _loguniform_lengths(rng, B)
        lk = _loguniform_lengths(rng, B)
        lq[0] = 0
        lq[B - 1] = 0
        lk[1] = 1
        lk[B // 2] = 1
        return lq, lk
    if cfg == 4:
        lq = rng.integers(4096, 8193, size=B)
        return lq, lq.copy()
    raise ValueError(f"unknown config {cfg}")


def draw_slopes(rng: np.random.Generator, B: int, hq: int) -> np.ndarray:
    base = 2.0 ** (-8.0 * (np.arange(hq) + 1) / hq)
    u = rng.uniform(0.5, 1.5, size=(B, hq))
    return (base[None, :] * u).astype(np.float32)


def _poisoned_view(rng, T, H, width, step, dtype, scale, head_dim=HEAD_DIM, chunk_tokens=8192):
    """NaN-filled buffer [T*step, H, width]; the view [::step, :, :head_dim] holds N(0,1)*scale."""
    buf = torch.full((max(T * step, 1), H, width), float("nan"), dtype=dtype)
    view = buf[::step, :, :head_dim][:T]
    for t0 in range(0, T, chunk_tokens):
        t1 = min(T, t0 + chunk_tokens)
        x = rng.standard_normal(size=(t1 - t0, H, head_dim), dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        view[t0:t1].copy_(torch.from_numpy(x))   # float32 -> 16-bit, nearest-even
    return buf, view


@dataclasses.dataclass
class Workload:
    name: str
    dtype: torch.dtype
    hq: int
    hkv: int
    width: int
    step: int
    lq: np.ndarray
    lk: np.ndarray
    cu_q: torch.Tensor          # int32 [B+1]
    cu_k: torch.Tensor          # int32 [B+1]
    slopes: torch.Tensor        # float32 [B, hq]
    bufs: dict                  # name -> padded backing buffer
    softcap: float = 3.0
    scale_multiplier: float = 0.75
    head_dim: int = HEAD_DIM

    @property
    def batch(self):
        return len(self.lq)

    @property
    def total_q(self):
        return int(self.lq.sum())

    @property
    def total_k(self):
        return int(self.lk.sum())

    def view(self, name):
        T = self.total_q if name in ("q", "dout") else self.total_k
        return self.bufs[name][::self.step, :, :self.head_dim][:T]

    @property
    def q(self):
        return self.view("q")

    @property
    def k(self):
        return self.view("k")

    @property
    def v(self):
        return self.view("v")

    @property
    def dout(self):
        return self.view("dout")

    def to(self, device) -> "Workload":
        return dataclasses.replace(
            self,
            cu_q=self.cu_q.to(device), cu_k=self.cu_k.to(device),
            slopes=self.slopes.to(device),
            bufs={k: v.to(device) for k, v in self.bufs.items()})

    def score_elements(self) -> int:
        """sum_b Lq_b * Lk_b * Hq."""
        return int((self.lq * self.lk).sum()) * self.hq

    def flops(self) -> float:
        """Credited work of forward + full VJP: 14 * sum_b Lq_b Lk_b * Hq * D."""
        return 14.0 * self.score_elements() * self.head_dim

    def min_hbm_bytes(self) -> int:
        """Read q, dout, k, v once; write out, dq, dk, dv once; FP32 lse and delta."""
        e = 2
        tq = self.total_q * self.hq
        tk = self.total_k * self.hkv
        return 4 * tq * self.head_dim * e + 4 * tk * self.head_dim * e + 2 * tq * 4


def _build(name, lq, lk, hq, dtype_name, width, step, scale, rng, softcap=3.0,
           scale_multiplier=0.75, slopes=None, hkv=1, head_dim=HEAD_DIM):
    lq = np.asarray(lq, np.int64)
    lk = np.asarray(lk, np.int64)
    B = len(lq)
    if hq % hkv != 0:
        raise ValueError("hkv must divide hq")
    if width < head_dim:
        raise ValueError("buffer width below the head dimension")
    if slopes is None:
        slopes = draw_slopes(rng, B, hq)
    dtype = TORCH_DTYPES[dtype_name]
    Tq, Tk = int(lq.sum()), int(lk.sum())
    bufs = {}
    for nm, T, H in (("q", Tq, hq), ("k", Tk, hkv), ("v", Tk, hkv), ("dout", Tq, hq)):
        bufs[nm], _ = _poisoned_view(rng, T, H, width, step, dtype, scale, head_dim)
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(lq)]), dtype=torch.int32)
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(lk)]), dtype=torch.int32)
    return Workload(name=name, dtype=dtype, hq=hq, hkv=hkv, width=width, step=step,
                    lq=lq, lk=lk, cu_q=cu_q, cu_k=cu_k,
                    slopes=torch.from_numpy(np.ascontiguousarray(slopes)), bufs=bufs,
                    softcap=softcap, scale_multiplier=scale_multiplier, head_dim=head_dim)


def make_workload(cfg: int, trial: int = 0) -> Workload:
    """One of the five named configurations (or a GQA_VARIANTS index);
    ``trial`` reseeds the draw."""
    if cfg in GQA_VARIANTS:
        return make_gqa_variant(cfg, trial)
    c = CONFIGS[cfg]
    rng = np.random.default_rng([cfg, trial])
    lq, lk = draw_lengths(cfg, rng)
    return _build(c["name"], lq, lk, c["hq"], c["dtype"], c["width"],
                  c["step"], c["scale"], rng)


# Grouped-query variants of the Q-short/K-long draw (same lengths and
# slopes recipe, several K/V heads, head dimensions 128 and 64), used to
# measure the general GQA paths; they are not among the page-derived configs.
GQA_VARIANTS = {
    5: dict(name="q_short_k_long_hkv8_d128", base=1, hkv=8, head_dim=128, width=128, step=2),
    6: dict(name="q_short_k_long_hkv4_d64", base=1, hkv=4, head_dim=64, width=64, step=2),
}


def make_gqa_variant(index: int, trial: int = 0) -> Workload:
    c = GQA_VARIANTS[index]
    b = CONFIGS[c["base"]]
    rng = np.random.default_rng([c["base"], trial])
    lq, lk = draw_lengths(c["base"], rng)
    return _build(c["name"], lq, lk, b["hq"], b["dtype"], c["width"], c["step"],
                  b["scale"], rng, hkv=c["hkv"], head_dim=c["head_dim"])


def fuzz_gqa_workload(seed: int, max_batch: int = 5, max_len: int = 260,
                      budget: int = 2_000_000) -> Workload:
    """Small random case over K/V head counts (hkv divides hq) and head
    dimensions 64 / 128 / 160, with the fuzz lengths of fuzz_workload."""
    rng = np.random.default_rng([1100, seed])
    hq = int(rng.choice([8, 16, 48, 64]))
    hkv = int(rng.choice([h for h in (1, 2, 4, 8) if hq % h == 0]))
    head_dim = int(rng.choice([64, 128, 160]))
    dtype_name = str(rng.choice(["f16", "bf16"]))
    step = int(rng.integers(1, 4))
    width = head_dim + int(rng.choice([0, 16, 32]))
    B = int(rng.integers(1, max_batch + 1))

    def one():
        if rng.uniform() < 0.5:
            return int(rng.choice(_EDGE_LENGTHS))
        return int(rng.integers(0, max_len + 1))

    lq = np.array([one() for _ in range(B)], np.int64)
    lk = np.array([one() for _ in range(B)], np.int64)
    while int((lq * lk).sum()) * hq > budget:
        i = int(np.argmax(lq * lk))
        lq[i] //= 2
        lk[i] //= 2
    scale = float(rng.choice([1.0, 1.5, 3.0]))
    softcap = 3.0 if rng.uniform() < 0.85 else 0.0
    return _build(f"fuzz_gqa{seed}", lq, lk, hq, dtype_name, width, step, scale, rng,
                  softcap=softcap, hkv=hkv, head_dim=head_dim)


# Lengths that sit on and around the 32/64/128 tile edges used on the device.
_EDGE_LENGTHS = np.array([0, 1, 2, 3, 31, 32, 33, 63, 64, 65, 127, 128, 129, 191, 255, 256, 257])


def fuzz_workload(seed: int, max_batch: int = 6, max_len: int = 300,
                  budget: int = 3_000_000) -> Workload:
    """Small random case: ragged lengths incl. 0/1/tile edges, any head count,
    dtype, token step and padded width.  ``budget`` bounds sum Lq*Lk*Hq so the
    oracle stays fast."""
    rng = np.random.default_rng([1000, seed])
    hq = int(rng.choice([48, 64, 80, 96]))
    dtype_name = str(rng.choice(["f16", "bf16"]))
    step = int(rng.integers(1, 4))
    width = int(rng.choice([160, 176, 192]))
    B = int(rng.integers(1, max_batch + 1))

    def one():
        if rng.uniform() < 0.5:
            return int(rng.choice(_EDGE_LENGTHS))
        return int(rng.integers(0, max_len + 1))

    lq = np.array([one() for _ in range(B)], np.int64)
    lk = np.array([one() for _ in range(B)], np.int64)
    while int((lq * lk).sum()) * hq > budget:
        i = int(np.argmax(lq * lk))
        lq[i] //= 2
        lk[i] //= 2
    scale = float(rng.choice([1.0, 1.5, 3.0]))
    softcap = 3.0 if rng.uniform() < 0.85 else 0.0
    return _build(f"fuzz{seed}", lq, lk, hq, dtype_name, width, step, scale, rng,
                  softcap=softcap)


def custom_workload(lq, lk, hq=48, dtype="f16", width=176, step=2, scale=1.0, seed=0,
                    softcap=3.0, scale_multiplier=0.75, slopes=None, hkv=1,
                    head_dim=HEAD_DIM) -> Workload:
    """Explicit lengths (and K/V heads, head dimension), for edge-case tests."""
    rng = np.random.default_rng([2000, seed])
    return _build("custom", lq, lk, hq, dtype, width, step, scale, rng, softcap=softcap,
                  scale_multiplier=scale_multiplier, slopes=slopes, hkv=hkv, head_dim=head_dim)


def oracle_inputs(wl: Workload):
    """The exact 16-bit values of the views, widened to float64 NumPy arrays."""
    def f64(t):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return dict(q=f64(wl.q), k=f64(wl.k), v=f64(wl.v), dout=f64(wl.dout),
                cu_q=wl.cu_q.cpu().numpy().astype(np.int64),
                cu_k=wl.cu_k.cpu().numpy().astype(np.int64),
                alibi_slopes=wl.slopes.cpu().numpy().astype(np.float64),
                softcap=wl.softcap, scale_multiplier=wl.scale_multiplier)
