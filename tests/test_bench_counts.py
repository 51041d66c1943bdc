"""The work counts behind bench.py's rates and roofline fractions.

`prefill_flops` is the numerator of every prefill TFLOP/s figure and of
roofline.achieved; `decode_cost` gives the decode bytes.  They are checked
here against the sizes the workloads fix (4*d FLOPs per visible (query, key)
pair and head; decode reads each visible cache row once) and, for the pair
counts, against a brute-force count of the causal / band mask.
"""
import numpy as np
import pytest

import bench
from attention_g4attn_amd import inputs


def brute_pairs(S, W):
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    vis = (j <= i) if W == 0 else ((i - j >= 0) & (i - j < W))
    return int(vis.sum())


@pytest.mark.parametrize("S,W", [(1, 0), (1, 5), (37, 0), (37, 1), (37, 7), (37, 36), (37, 37),
                                 (37, 100), (200, 64), (257, 32)])
def test_visible_pairs_match_the_mask(S, W):
    layer = inputs.Layer("local", 1, S, 1, 1, 1, W, inputs.LOCAL_THETA, 1.0)
    assert bench.prefill_flops(layer) == 4.0 * brute_pairs(S, W)


def test_local_prefill_b4_s8192_work():
    # 1024*1025/2 + (8192-1024)*1024 visible pairs per (b, h)
    pairs = 1024 * 1025 // 2 + (8192 - 1024) * 1024
    assert pairs == 7_864_832
    f = bench.prefill_flops(inputs.LOCAL_PREFILL)
    assert f == 4.0 * 256 * 16 * 4 * pairs
    assert f == pytest.approx(5.154e11, rel=1e-3)


def test_global_prefill_s32768_work():
    pairs = 32768 * 32769 // 2
    assert pairs == 536_887_296
    f = bench.prefill_flops(inputs.GLOBAL_PREFILL)
    assert f == 4.0 * 512 * 32 * pairs
    assert f == pytest.approx(3.5185e13, rel=1e-4)


def test_group_layers_s262144_work():
    g = bench.prefill_flops(inputs.GROUP_GLOBAL)
    loc = bench.prefill_flops(inputs.GROUP_LOCAL)
    assert g == 4.0 * 512 * 16 * (262144 * 262145 // 2)
    assert g == pytest.approx(1.1259e15, rel=1e-4)
    assert loc == 4.0 * 256 * 16 * (1024 * 1025 // 2 + (262144 - 1024) * 1024)
    assert loc == pytest.approx(4.3895e12, rel=1e-4)
    # the global layer is 98.1% of the group's five local and one global layers
    assert g / (g + 5 * loc) == pytest.approx(0.981, abs=1e-3)


def test_decode_bytes_batch64():
    lengths = [4096, 65536, 30000, 512, 100]
    glo = inputs.DecodeLayer("global", len(lengths), 16, 2, 512, 65536, 0, inputs.GLOBAL_THETA, 0.25)
    loc = inputs.DecodeLayer("local", len(lengths), 16, 8, 256, 512, 512, inputs.LOCAL_THETA, 1.0)
    qo = len(lengths) * 16  # query heads: bf16 q in, fp32 out
    # K=V: one 2 KiB row (2 KV heads x 512 dims x 2 B) per visible position
    f, b = bench.decode_cost(glo, lengths)
    assert b == sum(lengths) * 2 * 512 * 2 + qo * 512 * 6
    assert f == 4.0 * 512 * 16 * sum(lengths)
    # ring of 512 slots: at most 512 rows of K and of V per sequence
    f, b = bench.decode_cost(loc, lengths)
    rows = sum(min(L, 512) for L in lengths)
    assert b == rows * 8 * 256 * 2 * 2 + qo * 256 * 6
    assert f == 4.0 * 256 * 16 * rows


def test_decode_local_ring_batch64_reads_268_mb():
    loc = inputs.DecodeLayer("local", 64, 16, 8, 256, 512, 512, inputs.LOCAL_THETA, 1.0)
    _, b = bench.decode_cost(loc, [4096] * 64)
    assert b - 64 * 16 * 256 * 6 == 64 * 8 * 512 * 256 * 2 * 2 == 268_435_456
