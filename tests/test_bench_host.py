"""Host logic of bench.py: the profile readers and the one-GPU guard.

`bench.py` folds figures from the committed rocprofv3 summaries into its JSON
line (the dominant kernel's fabric traffic and SQ busy fractions, every
kernel's fabric bytes) only while the kernel sources are the ones the
summaries were taken from; these tests pin that behaviour on a scratch tree.
"""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

TRAFFIC = """# HBM-side traffic per launch: full VJP, wl

| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | written MB (scaled) | read MB (by request size) | L2 hit rate | unique read MB | unique written MB |
|---|---|---|---|---|---|---|---|---|
| `fwd_kernel<BF16, 160, true, true, false, false>` | 79141.8 | 38576.2 | 162.1 | 39.5 | 161.8 | 0.627 | 91.4 | 36.7 |
| `dkdv_kernel<BF16, 160, true, false, false>` | 184845.4 | 300568.3 | 378.6 | 307.8 | 378.2 | 0.670 | 91.4 | 18.0 |
| `dq_kernel<BF16, 160, true, false, false>` | 201952.5 | 50033.8 | 413.6 | 51.2 | 412.4 | 0.206 | 9.0 | 36.7 |

traffic_bytes_per_launch: 686336902
kernel_source_sha256: {digest}
"""

COUNTERS = """# SQ counters: wl

busy dkdv_kernel: mfma=0.340 valu=0.400 coissue=0.115 lds=0.094 clock_mhz=2082
kernel_source_sha256: {digest}
"""


@pytest.fixture
def tree(tmp_path, monkeypatch):
    csrc = tmp_path / "ragged_gqa_attention_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("// kernel source\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def _write(tree, digest):
    (tree / "profiles" / "dkdv_kernel_wl_hbm_traffic.md").write_text(TRAFFIC.format(digest=digest))
    (tree / "profiles" / "sq_counters_wl.md").write_text(COUNTERS.format(digest=digest))


def test_profiles_read_while_sources_match(tree):
    _write(tree, bench.kernel_source_digest())
    assert bench.measured_traffic("dkdv_kernel", "wl") == 686336902.0
    kb = bench.measured_kernel_bytes("wl")
    assert kb == {"fwd_kernel": (162.1e6, 39.5e6), "dkdv_kernel": (378.6e6, 307.8e6),
                  "dq_kernel": (413.6e6, 51.2e6)}
    busy = bench.measured_busy("dkdv_kernel", "wl")
    assert busy == {"mfma": 0.34, "valu": 0.4, "coissue": 0.115, "lds": 0.094, "clock_mhz": 2082.0}
    assert bench.measured_busy("fwd_kernel", "wl") is None   # no line for it


def test_profiles_ignored_once_sources_change(tree):
    _write(tree, bench.kernel_source_digest())
    (tree / "ragged_gqa_attention_amd" / "csrc" / "k.hip").write_text("// edited\n")
    assert bench.measured_traffic("dkdv_kernel", "wl") is None
    assert bench.measured_kernel_bytes("wl") is None
    assert bench.measured_busy("dkdv_kernel", "wl") is None


def test_missing_profiles(tree):
    assert bench.measured_traffic("dkdv_kernel", "wl") is None
    assert bench.measured_kernel_bytes("wl") is None
    assert bench.measured_busy("dkdv_kernel", "wl") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr
