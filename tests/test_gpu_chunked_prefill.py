"""GPU parity of chunked prefill over the paged cache (sdpa_decode_paged with many query
tokens per sequence) against the fp64 oracle.

A query chunk of s_q tokens is the last s_q tokens of a cache of L tokens (bottom-right
causal: token i sees keys 0 .. L - s_q + i).  For d_qk = d_v = 128 and page sizes that are
multiples of 64, once s_q covers a work item of the prefill kernel, the library runs the
ping-pong prefill kernel with K/V tiles addressed through the two page tables (and fp32
split partials merged by the LSE combine); these cases pin that path, including shapes the
few-row decode kernels refuse (more than 512 query rows per KV head).  With fewer tokens
than an item holds and more than 16 query rows per KV head, the
same kernel folds the (token, head) rows of the whole group, token-major, into its 256-row
items; the folded cases pin that mapping (partial items, several items, every group size).
"""
import numpy as np
import pytest
import torch

from scaled_dot_product_19_amd import inputs, sdpa
from tests.helpers import check_lse, check_o, log, oracle_decode, path_of, sample_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sdpa.load()


def run(pc, splits=None):
    S = pc.num_splits if splits is None else splits
    o, l = sdpa.decode_paged(to_dev(pc.q), to_dev(pc.k_pool), to_dev(pc.v_pool),
                             to_dev(pc.pt_k), to_dev(pc.pt_v), to_dev(pc.seq_lens), pc.max_kv,
                             pc.scale, pc.causal, num_splits=S)
    torch.cuda.synchronize()
    return o, l


def parity(pc, sel_rows=None):
    log("chunked prefill parity: %s lens=%s sq=%d hq=%d hkv=%d page=%d splits=%d causal=%s "
        "scale=%g kernel=%s" % (pc.name, pc.seq_lens.tolist()[:8], pc.sq, pc.hq, pc.hkv,
                                pc.page_size, pc.num_splits, pc.causal, pc.scale, path_of(pc)))
    o, l = run(pc)
    rows = pc.batch * pc.sq * pc.hq
    o_ref, l_ref = oracle_decode(pc, sel_rows=sel_rows)
    if sel_rows is None:
        e_o = check_o(o, o_ref)
        e_l = check_lse(l, l_ref)
    else:
        idx = torch.from_numpy(sel_rows).cuda()
        e_o = check_o(o.reshape(rows, -1)[idx], o_ref)
        e_l = check_lse(l.reshape(rows)[idx], l_ref)
    log("  max|dO|=%.3g max|dLSE|=%.3g" % (e_o, e_l))
    return o, l


CASES = [
    # G = 4, one 64-token item per (sequence, head group); L < s_q leaves early tokens keyless
    dict(seed=2101, sq=64, hq=8, hkv=2, page=64, lengths=[40, 300, 1000], splits=1, causal=True),
    # ragged last item (200 = 3 x 64 + 8), page 128, three splits
    dict(seed=2102, sq=200, hq=8, hkv=2, page=128, lengths=[700, 2100], splits=3, causal=True),
    # G = 8 (two head groups of 4 per KV head), non-causal, two splits
    dict(seed=2103, sq=96, hq=16, hkv=2, page=64, lengths=[96, 1500], splits=2, causal=False),
    # G = 1: items of 256 tokens of one head
    dict(seed=2104, sq=256, hq=4, hkv=4, page=64, lengths=[900], splits=1, causal=True),
    # 1200 query rows per KV head (refused by the few-row kernels); more splits than pages
    # for the short sequence
    dict(seed=2105, sq=300, hq=8, hkv=2, page=64, lengths=[320, 5000], splits=8, causal=True),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c["seed"]) for c in CASES])
def test_chunked_prefill_paged(case):
    pc = inputs.paged_case(case["seed"], len(case["lengths"]), case["sq"], case["hq"],
                           case["hkv"], 128, 128, case["page"], lengths=case["lengths"],
                           num_splits=case["splits"], causal=case["causal"], poison=True,
                           name="chunked_%d" % case["seed"])
    o, l = parity(pc)
    assert torch.isfinite(o).all()


@pytest.mark.parametrize("scale", [-0.07, 0.0])
def test_chunked_prefill_scale_edges(scale):
    pc = inputs.paged_case(2106, 2, 128, 8, 2, 128, 128, 64, lengths=[128, 700], num_splits=2,
                           scale=scale, poison=True, name="chunked_scale")
    parity(pc)


def test_chunked_prefill_rows_without_keys_are_empty():
    # L = 30 < s_q = 64: tokens 0..33 of the chunk see no key (O = 0, LSE = -inf)
    pc = inputs.paged_case(2107, 1, 64, 8, 2, 128, 128, 64, lengths=[30], num_splits=3,
                           poison=True, name="chunked_short")
    o, l = parity(pc)
    assert torch.all(o[0, :34] == 0)
    assert torch.all(l[0, :34] == float("-inf"))
    assert torch.all(torch.isfinite(l[0, 34:]))


def test_full_size_chunked_prefill_sampled():
    pc = inputs.chunked_prefill_paged()
    log("full-size %s pages=%d" % (pc.name, pc.k_pool.shape[0]))
    rows = pc.batch * pc.sq * pc.hq
    sel = sample_rows(rows, 96, 7, must=[0, rows - 1])
    o, l = parity(pc, sel_rows=sel)
    assert torch.isfinite(o).all() and torch.isfinite(l).all()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("chunk,cache", [(512, 131072), (1024, 65536)])
def test_context_phase_chunk_sampled(chunk, cache):
    # the context phase of serving: a 512- or 1024-token chunk at the end of 64k / 128k caches
    pc = inputs.context_chunk(chunk, cache, poison=True)
    rows = pc.batch * pc.sq * pc.hq
    sel = sample_rows(rows, 96, chunk + cache, must=[0, rows - 1])
    o, l = parity(pc, sel_rows=sel)
    assert torch.isfinite(o).all() and torch.isfinite(l).all()


# Folded rows: s_q * G query rows per KV head (s_q below an item's token count, more than
# 16 rows), token-major in items of 256 rows
FOLDED = [
    # MTP-like: 4 tokens x G 32 = 128 rows, half an item; L = 2 < s_q leaves tokens keyless
    dict(seed=2121, sq=4, hq=32, hkv=1, lengths=[2, 190, 1200], splits=1, causal=True),
    # 3 tokens x G 32 = 96 rows over two KV heads, three splits
    dict(seed=2122, sq=3, hq=64, hkv=2, lengths=[0, 77, 900], splits=3, causal=True),
    # 40 tokens x G 8 = 320 rows: a full item and a ragged one, non-causal
    dict(seed=2123, sq=40, hq=16, hkv=2, lengths=[41, 700], splits=2, causal=False),
    # 2 tokens x G 64 = 128 rows, causal across two tokens
    dict(seed=2124, sq=2, hq=64, hkv=1, lengths=[1, 333], splits=1, causal=True),
    # G 2: 33 tokens x 2 = 66 rows; G 1: 100 tokens of one head
    dict(seed=2125, sq=33, hq=4, hkv=2, lengths=[20, 500], splits=4, causal=True),
    dict(seed=2126, sq=100, hq=2, hkv=2, lengths=[150, 260], splits=1, causal=True),
    # 16 tokens x G 8 = 128 rows per KV head, 4 KV heads, page 128
    dict(seed=2127, sq=16, hq=32, hkv=4, lengths=[16, 1000, 3000], splits=8, causal=True,
         page=128),
    # the fewest rows that fold: 17 tokens of one head; 8 tokens x G 4 = 32 rows; 6 x 8 = 48
    dict(seed=2129, sq=17, hq=2, hkv=2, lengths=[5, 400], splits=2, causal=True),
    dict(seed=2130, sq=8, hq=32, hkv=8, lengths=[7, 130, 2000], splits=4, causal=True),
    dict(seed=2131, sq=6, hq=16, hkv=2, lengths=[6, 64, 65], splits=1, causal=True),
    # groups that are not powers of two: 5 tokens x G 7 = 35 rows; 30 x G 6 = 180 rows
    # (an item of 128 tokens when not folded); 3 x G 96 = 288 rows
    dict(seed=2132, sq=5, hq=28, hkv=4, lengths=[3, 444, 1900], splits=3, causal=True),
    dict(seed=2133, sq=30, hq=12, hkv=2, lengths=[31, 1000], splits=1, causal=True),
    dict(seed=2134, sq=3, hq=96, hkv=1, lengths=[2, 800], splits=2, causal=True),
]


@pytest.mark.parametrize("case", FOLDED, ids=["%d_%dx%d" % (c["seed"], c["sq"], c["hq"] // c["hkv"])
                                              for c in FOLDED])
def test_folded_rows(case):
    pc = inputs.paged_case(case["seed"], len(case["lengths"]), case["sq"], case["hq"],
                           case["hkv"], 128, 128, case.get("page", 64), lengths=case["lengths"],
                           num_splits=case["splits"], causal=case["causal"], poison=True,
                           name="folded_%d" % case["seed"])
    log("folded rows: %d per KV head" % (case["sq"] * case["hq"] // case["hkv"]))
    o, l = parity(pc)
    if case["lengths"][0] < case["sq"] and case["causal"]:
        # sequence 0 holds fewer keys than tokens: its first token sees none
        assert torch.all(o[0, 0] == 0) and torch.all(l[0, 0] == -np.inf)


@pytest.mark.timeout(600)
def test_folded_rows_decode_workload_sampled():
    # the paged decode workload's sequences (B = 64, 32/8 heads, D = 128, page 64,
    # L U[512, 32768], 8 splits) with 32 query tokens: 128 folded rows per KV head
    pc = inputs.paged_case(inputs.SEED_BASE + 3, 64, 32, 32, 8, 128, 128, 64, lo=512,
                           hi=32768, num_splits=8, poison=True, name="folded_decode_workload")
    rows = pc.batch * pc.sq * pc.hq
    sel = sample_rows(rows, 256, 2128, must=[0, rows - 1])
    o, _ = parity(pc, sel_rows=sel)
    assert torch.isfinite(o.float()).all()


# D = 256: the sequential 4-wave prefill kernel over the page tables (32-key tiles, so pages
# of a multiple of 32 keys), items of 32 tokens x 4 heads or, folded, 128 rows
D256 = [
    # chunk of 40 tokens, G 4 (two items per head group), page 32, three splits
    dict(seed=2141, sq=40, hq=8, hkv=2, page=32, lengths=[50, 900], splits=3, causal=True),
    # folded: 2 tokens x G 16 = 32 rows; 3 x G 12 = 36; 5 x G 32 = 160 (two items)
    dict(seed=2142, sq=2, hq=16, hkv=1, page=64, lengths=[1, 300, 1500], splits=1, causal=True),
    dict(seed=2143, sq=3, hq=24, hkv=2, page=32, lengths=[2, 777], splits=4, causal=True),
    dict(seed=2144, sq=5, hq=64, hkv=2, page=64, lengths=[9, 1200], splits=2, causal=False),
]


@pytest.mark.parametrize("case", D256, ids=[str(c["seed"]) for c in D256])
def test_d256_paged_prefill_kernel(case):
    pc = inputs.paged_case(case["seed"], len(case["lengths"]), case["sq"], case["hq"],
                           case["hkv"], 256, 256, case["page"], lengths=case["lengths"],
                           num_splits=case["splits"], causal=case["causal"], poison=True,
                           name="d256_paged_%d" % case["seed"])
    o, l = parity(pc)
    if case["causal"] and case["lengths"][0] < case["sq"]:
        assert torch.all(o[0, 0] == 0) and torch.all(l[0, 0] == -np.inf)


# D = 64: the ping-pong kernel with 64-key tiles over the page tables (pages of a multiple
# of 64 keys): a chunk of 64 tokens (G 4), and folded rows
D64 = [
    dict(seed=2151, sq=64, hq=8, hkv=2, page=64, lengths=[70, 900], splits=2, causal=True),
    dict(seed=2152, sq=4, hq=32, hkv=1, page=128, lengths=[3, 500, 2000], splits=1, causal=True),
    dict(seed=2153, sq=3, hq=12, hkv=2, page=64, lengths=[2, 640], splits=3, causal=False),
]


@pytest.mark.parametrize("case", D64, ids=[str(c["seed"]) for c in D64])
def test_d64_paged_prefill_kernel(case):
    pc = inputs.paged_case(case["seed"], len(case["lengths"]), case["sq"], case["hq"],
                           case["hkv"], 64, 64, case["page"], lengths=case["lengths"],
                           num_splits=case["splits"], causal=case["causal"], poison=True,
                           name="d64_paged_%d" % case["seed"])
    parity(pc)


# Pages of 16 or 32 keys: a tile spans several pages and each wave of the prefill kernel
# reads its 8 rows through the page that holds them
SMALL_PAGES = [
    # (seed, d, sq, hq, hkv, page, lengths, splits, causal)
    (2161, 128, 100, 8, 2, 16, [120, 1500], 3, True),    # chunk of 100 tokens
    (2162, 128, 8, 32, 8, 16, [7, 130, 2000], 4, True),   # folded 32 rows
    (2163, 128, 4, 32, 1, 32, [3, 900], 1, False),        # folded 128 rows
    (2164, 64, 64, 8, 2, 16, [70, 900], 2, True),         # D 64 chunk
    (2165, 256, 40, 8, 2, 16, [50, 700], 3, True),        # D 256 chunk
    (2166, 256, 2, 16, 1, 16, [1, 333], 2, True),         # D 256 folded 32 rows
]


@pytest.mark.parametrize("case", SMALL_PAGES, ids=[str(c[0]) for c in SMALL_PAGES])
def test_prefill_kernel_on_small_pages(case):
    seed, d, sq, hq, hkv, page, lengths, splits, causal = case
    pc = inputs.paged_case(seed, len(lengths), sq, hq, hkv, d, d, page, lengths=lengths,
                           num_splits=splits, causal=causal, poison=True,
                           name="small_pages_%d" % seed)
    assert path_of(pc) in ("prefill", "prefill_folded")
    o, l = parity(pc)
    if causal and lengths[0] < sq:
        assert torch.all(o[0, 0] == 0) and torch.all(l[0, 0] == -np.inf)


def test_fp8_prefill_kernel_on_16_key_pages():
    pc = inputs.fp8_paged_case(2167, 3, 16, 32, 8, 128, 16, lengths=[10, 400, 1800],
                               num_splits=3, poison=True, name="fp8_small_pages")
    assert path_of(pc, fp8=True) == "prefill_folded"
    dq, dk, dv = [torch.tensor([x], dtype=torch.float32, device="cuda") for x in pc.descale]
    o, l = sdpa.decode_paged_fp8(to_dev(pc.q), to_dev(pc.k_pool), to_dev(pc.v_pool),
                                 to_dev(pc.pt_k), to_dev(pc.pt_v), to_dev(pc.seq_lens),
                                 pc.max_kv, pc.scale, dq, dk, dv, causal=True, num_splits=3)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_decode(pc, descale=pc.descale)
    check_o(o, o_ref)
    check_lse(l, l_ref)
