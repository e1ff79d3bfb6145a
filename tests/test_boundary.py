"""C-ABI boundary checks that need no GPU: the library loads, exports every
function the header declares, and rejects bad arguments with the documented
status codes before launching anything."""
import ctypes
import glob
import os
import re

import pytest

from ragged_gqa_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(attn_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for required in ("attn_varlen_fwd", "attn_varlen_bwd", "attn_varlen_full_vjp",
                     "attn_varlen_workspace_size", "attn_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(_declared_functions()) <= set(_lib.EXPORTED) | set(_declared_functions())


def _problem(**over):
    p = dict(dtype=_lib.ATTN_BF16, batch=2, hq=64, hkv=1, head_dim=160, total_q=10,
             total_k=20, cu_q=0x10000, cu_k=0x20000, alibi_slopes=0x30000, slopes_stride=64,
             causal=0, window_left=-1, window_right=-1, softcap=3.0, scale_multiplier=0.75)
    p.update(over)
    return _lib.AttnProblem(**p)


def _tensor(ptr=0x100000, ts=192 * 64 * 2, hs=192):
    return _lib.AttnTensor(ptr, ts, hs)


def _call_fwd(prob, q=None, k=None, v=None, out=None, ws_bytes=1 << 30, ws=0x4000000):
    lib = _lib.load()
    q = q or _tensor()
    k = k or _tensor(ts=384, hs=192)
    v = v or _tensor(ts=384, hs=192)
    out = out or _tensor(ptr=0x200000, ts=64 * 160, hs=160)
    lse = ctypes.cast(0x300000, ctypes.POINTER(ctypes.c_float))
    return lib.attn_varlen_fwd(ctypes.byref(prob), ctypes.byref(q), ctypes.byref(k),
                               ctypes.byref(v), ctypes.byref(out), lse, ctypes.c_void_p(ws),
                               ws_bytes, None)


@pytest.mark.parametrize("over,status", [
    (dict(causal=2), _lib.ATTN_INVALID_ARG),
    (dict(window_left=-2), _lib.ATTN_INVALID_ARG),
    (dict(window_right=-7), _lib.ATTN_INVALID_ARG),
    (dict(head_dim=96), _lib.ATTN_UNSUPPORTED),
    (dict(head_dim=256), _lib.ATTN_UNSUPPORTED),
    (dict(hkv=3), _lib.ATTN_INVALID_ARG),
    (dict(hkv=0), _lib.ATTN_INVALID_ARG),
    (dict(dtype=7), _lib.ATTN_UNSUPPORTED),
    (dict(hq=0), _lib.ATTN_INVALID_ARG),
    (dict(batch=-1), _lib.ATTN_INVALID_ARG),
    (dict(total_q=-5), _lib.ATTN_INVALID_ARG),
    (dict(cu_q=0), _lib.ATTN_INVALID_ARG),
    (dict(alibi_slopes=0), _lib.ATTN_INVALID_ARG),
    (dict(slopes_stride=10), _lib.ATTN_INVALID_ARG),
    (dict(softcap=-1.0), _lib.ATTN_INVALID_ARG),
    (dict(softcap=float("nan")), _lib.ATTN_INVALID_ARG),
    (dict(scale_multiplier=float("inf")), _lib.ATTN_INVALID_ARG),
])
def test_problem_errors(over, status):
    assert _call_fwd(_problem(**over)) == status
    assert _lib.load().attn_last_error().decode() != ""


def test_tensor_errors():
    prob = _problem()
    assert _call_fwd(prob, q=_tensor(ptr=0x100008)) == _lib.ATTN_MISALIGNED
    assert _call_fwd(prob, q=_tensor(ts=192 * 64 * 2 + 4)) == _lib.ATTN_MISALIGNED
    assert _call_fwd(prob, k=_tensor(ts=100, hs=192)) == _lib.ATTN_INVALID_ARG
    assert _call_fwd(prob, q=_tensor(hs=64)) == _lib.ATTN_INVALID_ARG
    assert _call_fwd(prob, q=_tensor(ptr=0)) == _lib.ATTN_INVALID_ARG
    assert _call_fwd(prob, ws=0x4000010) == _lib.ATTN_MISALIGNED


def test_workspace_size_and_too_small():
    lib = _lib.load()
    prob = _problem()
    sizes = []
    for entry in (_lib.ENTRY_FWD, _lib.ENTRY_BWD, _lib.ENTRY_FULL_VJP):
        n = ctypes.c_size_t(0)
        assert lib.attn_varlen_workspace_size(ctypes.byref(prob), entry, ctypes.byref(n)) == 0
        sizes.append(n.value)
    assert 0 < sizes[0] < sizes[1] < sizes[2]
    assert _call_fwd(prob, ws_bytes=sizes[0] - 1) == _lib.ATTN_WORKSPACE_TOO_SMALL
    n = ctypes.c_size_t(0)
    assert lib.attn_varlen_workspace_size(ctypes.byref(prob), 9, ctypes.byref(n)) == \
        _lib.ATTN_INVALID_ARG


def test_workspace_linear_in_tokens():
    """Auxiliary memory grows linearly with tokens (page "python-20261012-ragged-
    flash-attention-gradient-recompute", section "Verification": linear, not
    quadratic, growth of peak auxiliary memory)."""
    lib = _lib.load()
    sizes = []
    for scale in (1, 2, 4, 8):
        prob = _problem(total_q=10000 * scale, total_k=20000 * scale)
        n = ctypes.c_size_t(0)
        assert lib.attn_varlen_workspace_size(ctypes.byref(prob), _lib.ENTRY_FULL_VJP,
                                              ctypes.byref(n)) == 0
        sizes.append(n.value)
    growth = [sizes[i + 1] - sizes[i] for i in range(3)]
    assert growth[1] == pytest.approx(2 * growth[0], rel=0.02)
    assert growth[2] == pytest.approx(4 * growth[0], rel=0.02)


def test_status_strings():
    lib = _lib.load()
    for st in range(-6, 1):
        assert lib.attn_status_string(st).decode() not in ("", "unknown status")
    assert lib.attn_status_string(-99).decode() == "unknown status"


def test_workspace_size_with_stored_ds():
    """Room for dS: ceil(Lq hq / 256) ceil(Lk / 64) images of 32 KiB per
    sequence with rows and keys, on top of the minimum; the forward needs none;
    malformed host offsets are rejected."""
    lib = _lib.load()
    i32 = ctypes.c_int32
    lq, lk = [3, 0, 9, 5], [70, 4, 0, 64]
    cq = (i32 * 5)(*[sum(lq[:i]) for i in range(5)])
    ck = (i32 * 5)(*[sum(lk[:i]) for i in range(5)])
    prob = _problem(batch=4, total_q=sum(lq), total_k=sum(lk))
    for entry in (_lib.ENTRY_FWD, _lib.ENTRY_BWD, _lib.ENTRY_FULL_VJP):
        base, full = ctypes.c_size_t(0), ctypes.c_size_t(0)
        assert lib.attn_varlen_workspace_size(ctypes.byref(prob), entry, ctypes.byref(base)) == 0
        assert lib.attn_varlen_workspace_size_ds(ctypes.byref(prob), entry, cq, ck,
                                                 ctypes.byref(full)) == 0
        images = (1 * 2) + (2 * 1) if entry != _lib.ENTRY_FWD else 0   # seqs 0 and 3
        assert full.value - base.value == images * 64 * 256 * 2
    bad = (i32 * 5)(0, 3, 2, 12, 17)
    n = ctypes.c_size_t(0)
    assert lib.attn_varlen_workspace_size_ds(ctypes.byref(prob), _lib.ENTRY_BWD, bad, ck,
                                             ctypes.byref(n)) == _lib.ATTN_BAD_SEQLENS
    short = (i32 * 5)(0, 3, 3, 12, 16)
    assert lib.attn_varlen_workspace_size_ds(ctypes.byref(prob), _lib.ENTRY_BWD, short, ck,
                                             ctypes.byref(n)) == _lib.ATTN_BAD_SEQLENS
