"""Host-side helpers of bench.py (no GPU): work counting of the chunked-prefill line."""
import types

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
