"""The measured form of page 1's section-4 table (one head, bf16, d = 128),
run small: the materialising forward really holds S and P in device memory,
the fused forward only O, L and its O(n) key-split workspace, and both
compute the same attention (to the bf16 rounding of S and P in the
materialising one)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.gpu
def test_io_compare_small():
    n, d = 1024, 128
    e = bench.io_compare(n, calls=2, warmup=1)
    # S and P: two n x n bf16 matrices
    assert e["materialising"]["peak_extra_bytes"] >= 2 * n * n * 2
    # O (bf16) and L (fp32), with the allocator's rounding
    assert e["fused"]["peak_extra_bytes"] <= n * d * 2 + n * 4 + (64 << 10)
    assert e["fused"]["max_abs_diff_vs_materialising"] <= 5e-2
    assert e["page_io_elements"]["materialising"] == 4 * n * n
    for path in ("materialising", "fused"):
        assert e[path]["ms"]["median"] > 0


@pytest.mark.gpu
def test_io_compare_split():
    # one head of 4096: the forward splits its keys; its extra memory is O, L
    # and the O(n) workspace of the partials
    n, d = 4096, 128
    e = bench.io_compare(n, calls=2, warmup=1, paths=("fused", "fused_split"))
    ws = e["fused_split_workspace_bytes"]
    assert ws > 0
    assert e["fused_split"]["peak_extra_bytes"] <= n * d * 2 + n * 4 + ws + (64 << 10)
    assert "materialising" not in e
