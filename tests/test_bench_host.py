"""Host-side checks of bench.py that need no GPU: the one-GPU guard, the algorithmic
byte counts per launch, and the reading of the committed traffic summary."""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, timeout=120)
    assert r.returncode == 2
    assert b"one GPU" in r.stderr
    assert r.stdout == b""


@pytest.mark.parametrize("kernel,per_elem", [
    ("quantize", 2 + 1 / 2 + 1 / 32),      # BF16 in, codes + MX scales out
    ("rows", 1 / 2 + 1 / 32 + 1 + 1 / 128),  # codes + MX scales in, FP8 + block scales out
    ("fp8q_rows", 2 + 1 + 1 / 128),        # BF16 in, FP8 + block scales out
])
def test_row_kernel_bytes_per_element(kernel, per_elem):
    M, K = 4096, 7168
    assert bench.alg_bytes(kernel, M, K) == round(M * K * per_elem)


def test_column_kernel_bytes_count_each_scale_byte_once():
    M, K = 1000, 2048
    col_scales = 8 * K                      # e.g. 8 blocks of 128 rows over all columns
    assert bench.alg_bytes("cols", M, K, col_scales) == M * K // 2 + M * K // 32 + M * K + col_scales
    assert bench.alg_bytes("fp8q_cols", M, K, col_scales) == 3 * M * K + col_scales
    with pytest.raises(ValueError):
        bench.alg_bytes("gemm", M, K)


def test_traffic_summary_is_read_only_for_matching_sources(tmp_path, monkeypatch):
    text = open(os.path.join(ROOT, "profiles", "hbm_traffic_config5.md")).read()
    data = json.loads(re.search(r"<!-- traffic-json (\{.*\}) -->", text).group(1))
    for key, ent in data.items():
        assert abs(ent["bytes_per_launch"] - ent["fetch_bytes"] - ent["write_bytes"]) <= 1
        # counters never read fewer bytes than the method must move
        assert ent["bytes_per_launch"] >= 0.99 * ent["alg_bytes"], key
    # a summary whose recorded hash differs from the sources is ignored
    fake = dict(data)
    fake["rows/hidden"] = dict(data["rows/hidden"], source_sha="0" * 16)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "hbm_traffic_config5.md").write_text("<!-- traffic-json " + json.dumps(fake) + " -->")
    assert bench.read_traffic("rows", "config5", "hidden") is None
    (tmp_path / "hbm_traffic_config5.md").write_text("<!-- traffic-json " + json.dumps(
        {"rows/hidden": dict(data["rows/hidden"], source_sha=bench.source_hash("rows"))}) + " -->")
    assert bench.read_traffic("rows", "config5", "hidden") == data["rows/hidden"]["bytes_per_launch"]


def test_strip_table_covers_every_row_once_in_the_transposed_layout():
    """The memory-only ceiling kernel's strips: every routed row in exactly one strip, in
    expert order, each strip 1..128 rows of one expert, and its output byte is where the
    transposed layout puts (column 0, the strip's first row): K * offs[g] + the row's
    index within the expert."""
    import numpy as np
    K = 384
    counts = [0, 1, 127, 128, 129, 0, 300, 5]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    t = bench.strip_table(offs, K)
    assert t.shape == (sum((c + 127) // 128 for c in counts), 4)
    seen = np.zeros(offs[-1], np.int64)
    for row, n, a0, mg in t:
        assert 1 <= n <= 128
        g = int(np.searchsorted(offs, row, side="right")) - 1
        assert mg == offs[g + 1] - offs[g] and row + n <= offs[g + 1]
        assert a0 == K * offs[g] + (row - offs[g])
        seen[row:row + n] += 1
    assert (seen == 1).all()
    assert list(t[:, 0]) == sorted(t[:, 0])
    assert bench.strip_table(np.zeros(4, np.int32), K).shape == (0, 4)
