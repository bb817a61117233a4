"""Host-side pieces of bench.py (no GPU): FLOP and byte accounting."""

import numpy as np
import pytest
import torch

import bench
from exact_attention_forward_fa_amd import inputs
from oracle import ref


@pytest.mark.parametrize("sq,sk", [(4096, 4096), (100, 37), (37, 100), (1, 50), (5, 5), (1, 1), (300, 299)])
def test_causal_pair_count_matches_oracle_mask(sq, sk):
    assert bench.causal_pairs(sq, sk) == int(ref.allowed_mask(np.arange(sq), sq, sk, True).sum())


def test_metric_flops():
    # 4 * D per allowed pair, B*H heads: the causal B4 S4096 H32 D64 workload
    assert 4 * 64 * bench.causal_pairs(4096, 4096) * 4 * 32 == 274945015808


def test_decode_bytes_counts_each_cached_token_once():
    pc = inputs.paged_cache(3, 1, 8, 2, 64, torch.bfloat16, seed=1, page_size=16, lengths=[5, 16, 40])
    c = dict(q=pc.q, k_pool=pc.k_pool, cache_seqlens=pc.cache_seqlens, page_size=16)
    kv = (5 + 16 + 40) * 2 * 64 * 2 * 2
    assert bench.decode_bytes(c) == kv + 2 * pc.q.numel() * 2 + (1 + 1 + 3) * 4 + 3 * 4


def test_median_and_cpu_model():
    import bench
    assert bench.median([3.0, 1.0, 2.0]) == 2.0
    assert bench.median([4.0, 1.0, 2.0, 3.0]) == 2.5
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


@pytest.mark.parametrize("sq,sk,causal,window", [
    (4096, 4096, True, (256, 0)), (4096, 4096, False, (256, 256)), (300, 299, True, (-1, -1)),
    (100, 37, False, (5, 3)), (37, 100, True, (10, -1)), (64, 64, False, (-1, -1)), (8, 8, False, (0, 0))])
def test_allowed_pair_count_matches_oracle_mask(sq, sk, causal, window):
    """The bench's pair counts (the FLOP denominators of every prefill leg) equal the
    number of True entries of the oracle's mask, and the config 3 window counts
    equal the closed forms 257*S - 256*257/2 and 513*S - 256*257."""
    assert bench.allowed_pairs(sq, sk, causal, window) == int(
        ref.allowed_mask(np.arange(sq), sq, sk, causal, window).sum())
    if (sq, sk, causal, window) == (4096, 4096, True, (256, 0)):
        assert bench.allowed_pairs(sq, sk, causal, window) == 257 * 4096 - 256 * 257 // 2
    if (sq, sk, causal, window) == (4096, 4096, False, (256, 256)):
        assert bench.allowed_pairs(sq, sk, causal, window) == 513 * 4096 - 256 * 257
