"""The benchmark's algorithmic work and byte counts, checked against brute-force counts on
small cases (CPU only; no GPU call).  These are the numerators of every reported rate and
roofline fraction."""
import numpy as np
import pytest

import bench
from attn_inputs import (BF16, decode_case, log_uniform_ctx, paged_prefill_case,
                         prefill_case)


def visible_pairs_causal(N):
    return sum(1 for i in range(N) for j in range(N) if j <= i)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_flops_and_bytes(causal):
    c = prefill_case(2, 4, 2, 64, 16, causal, BF16)
    pairs = 2 * 4 * (visible_pairs_causal(64) if causal else 64 * 64)
    # the convention: causal counts N^2 / 2 pairs (within 1/N of the exact count)
    want = 4.0 * 16 * (2 * 4 * 64 * 64 * (0.5 if causal else 1.0))
    assert bench.prefill_flops(c) == want
    assert abs(bench.prefill_flops(c) / (4.0 * 16 * pairs) - 1) < (1.0 / 64 if causal else 1e-12)
    # Q + O (2 B each per element of [B, Hq, N, d]), K + V ([B, Hkv, N, d]), LSE fp32
    assert bench.prefill_bytes(c) == 2 * 2 * 4 * 64 * 16 * 2 + 2 * 2 * 2 * 64 * 16 * 2 + 2 * 4 * 64 * 4


def test_decode_bytes_count_every_kv_element_once():
    ctx = [1, 17, 300, 0]
    c = decode_case(4, 8, 2, 64, ctx, 16, BF16)
    total, kv = bench.decode_bytes(c)
    kv_brute = sum(t * 2 * 64 * 2 * 2 for t in ctx)        # tokens x Hkv x d x 2 B x (K, V)
    assert kv == kv_brute
    pages = sum((t + 15) // 16 for t in ctx)
    assert total == kv_brute + 2 * 4 * 8 * 64 * 2 + pages * 4 + 4 * 4 + 4 * 8 * 4
    assert bench.decode_flops(c) == 4.0 * 8 * 64 * sum(ctx)


def test_cascade_bytes_add_the_prefix_once():
    c = decode_case(3, 8, 2, 64, [5, 0, 40], 16, BF16)
    total, _ = bench.decode_bytes(c)
    assert bench.cascade_bytes(c, 100) == total + 100 * 2 * 64 * 2 * 2


def test_paged_prefill_flops_count_visible_pairs():
    for causal in (True, False):
        c = paged_prefill_case(4, 2, 16, [5, 0, 9, 1], [30, 7, 9, 2], 16, BF16, causal)
        pairs = 0
        for ql, kl in zip(c.q_lens, c.kv_lens):
            for i in range(ql):
                pos = kl - ql + i
                pairs += sum(1 for j in range(kl) if (not causal or j <= pos))
        assert bench.paged_prefill_flops(c) == 4.0 * 4 * 16 * pairs


def test_variant_flops_count_the_window():
    v = dict(B=2, Hq=3, d=16, N=50, window=7)
    pairs = sum(1 for i in range(50) for j in range(50) if i - 7 < j <= i)
    assert bench.variant_flops(v) == 4.0 * 2 * 3 * 16 * pairs
