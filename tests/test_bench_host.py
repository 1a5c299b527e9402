"""Host-side helpers of bench.py (no GPU): work counting of the chunked and windowed prefill lines."""
import types

import pytest

import torch

import bench


def test_chunked_prefill_flops_counts_visible_pairs():
    # token i of a chunk of 4 tokens at the end of a cache of L tokens sees L - 4 + i + 1 keys
    pc = types.SimpleNamespace(seq_lens=torch.tensor([5, 3, 4]), sq=4, hq=3)
    brute = 0
    for L in (5, 3, 4):
        for i in range(4):
            brute += sum(1 for j in range(L) if j <= L - 4 + i)
    assert brute == (2 + 3 + 4 + 5) + (0 + 1 + 2 + 3) + (1 + 2 + 3 + 4)
    assert bench.chunked_prefill_flops(pc) == 2.0 * 256 * brute * 3


@pytest.mark.parametrize("causal", [True, False])
def test_window_prefill_flops_counts_visible_pairs(causal):
    lq, lk = [5, 9, 3, 0], [7, 4, 3, 2]
    for w in (0, 1, 3, 100):
        brute = 0
        for a, b in zip(lq, lk):
            for i in range(a):
                d = i + b - a
                brute += sum(1 for j in range(b)
                             if (not causal or j <= d) and (w <= 0 or j >= d - w + 1))
        assert bench.window_prefill_flops(lq, lk, 2, 64, 32, causal, w) == brute * 2 * 2 * 96
    assert (bench.window_prefill_flops(lq, lk, 2, 64, 64, causal, 0)
            == bench.prefill_flops(lq, lk, 2, 64, 64, causal))


@pytest.mark.parametrize("causal", [True, False])
def test_decode_visible_pairs_counts_by_brute_force(causal):
    lens, sq = [1, 2, 5, 64], 2
    brute = 0
    for L in lens:
        for t in range(sq):
            pos = L - sq + t
            brute += sum(1 for j in range(L) if not causal or j <= pos)
    assert bench.decode_visible_pairs(lens, sq, causal) == brute


def test_ms_stats_median_and_min():
    assert bench.ms_stats([3.0, 1.0, 2.0]) == {"mean": 2.0, "median": 2.0, "min": 1.0}
    assert bench.ms_stats([4.0, 1.0, 2.0, 3.0]) == {"mean": 2.5, "median": 2.5, "min": 1.0}
