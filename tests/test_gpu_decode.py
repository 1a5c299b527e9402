"""GPU parity of sdpa_decode_paged and sdpa_splitkv_combine against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from scaled_dot_product_19_amd import inputs, sdpa
from tests.helpers import check_lse, check_o, log, oracle_decode, path_of, sample_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sdpa.load()


def run(pc: inputs.PagedCase, splits=None, workspace=None, out=None, lse=None, stream=None):
    S = pc.num_splits if splits is None else splits
    o, l = sdpa.decode_paged(to_dev(pc.q), to_dev(pc.k_pool), to_dev(pc.v_pool),
                             to_dev(pc.pt_k), to_dev(pc.pt_v), to_dev(pc.seq_lens), pc.max_kv,
                             pc.scale, pc.causal, num_splits=S, workspace=workspace, out=out,
                             lse=lse, stream=stream)
    torch.cuda.synchronize()
    return o, l


def parity(pc, splits=None):
    S = pc.num_splits if splits is None else splits
    log("decode parity: %s lens=%s sq=%d hq=%d hkv=%d d=%d/%d page=%d splits=%d kernel=%s" % (
        pc.name, pc.seq_lens.tolist()[:8], pc.sq, pc.hq, pc.hkv, pc.q.shape[3],
        pc.v_pool.shape[3], pc.page_size, S, path_of(pc, S)))
    o, l = run(pc, splits=S)
    o_ref, l_ref = oracle_decode(pc)
    e_o = check_o(o, o_ref)
    e_l = check_lse(l, l_ref)
    log("  max|dO|=%.3g max|dLSE|=%.3g" % (e_o, e_l))
    return o, l, o_ref, l_ref


@pytest.mark.parametrize("splits", [1, 3, 8])
def test_d128_gqa4_poisoned_pools(splits):
    pc = inputs.paged_case(2001, 7, 1, 32, 8, 128, 128, 64,
                           lengths=[1, 63, 64, 65, 130, 1000, 2047], num_splits=splits,
                           poison=True, name="d128_g4")
    parity(pc)


def test_page16_and_more_splits_than_pages():
    pc = inputs.paged_case(2002, 3, 1, 8, 2, 128, 128, 16, lengths=[5, 40, 300],
                           num_splits=24, poison=True, name="page16")
    parity(pc)


@pytest.mark.parametrize("splits", [1, 16])
def test_mla_576_512_two_tokens_causal(splits):
    pc = inputs.paged_case(2003, 3, 2, 128, 1, 576, 512, 64, lengths=[1, 65, 700],
                           num_splits=splits, poison=True, name="mla_small")
    o, l, _, _ = parity(pc)
    # L=1 < s_q=2: token 0 sees no key
    assert torch.all(l[0, 0] == -math.inf) and torch.all(o[0, 0] == 0)


@pytest.mark.parametrize("shape", [(64, 64, 4, 4, 3, False), (64, 64, 2, 1, 1, True),
                                   (64, 64, 16, 1, 1, True), (64, 64, 32, 1, 2, True),
                                   (64, 64, 64, 1, 2, True),
                                   (256, 256, 8, 2, 2, True), (128, 128, 64, 4, 1, True),
                                   (128, 128, 16, 1, 4, True)])
def test_other_head_shapes(shape):
    d, dv, hq, hkv, sq, causal = shape
    pc = inputs.paged_case(2004, 3, sq, hq, hkv, d, dv, 32, lengths=[3, 77, 500], num_splits=4,
                           causal=causal, poison=True, name="shape")
    parity(pc)


def test_zero_length_sequences():
    pc = inputs.paged_case(2005, 4, 1, 8, 2, 128, 128, 64, lengths=[0, 10, 0, 70], num_splits=4,
                           poison=True, name="zero_len")
    o, l, _, _ = parity(pc)
    assert torch.all(o[0] == 0) and torch.all(l[0] == -math.inf)


def test_split_partials_match_oracle_partials():
    pc = inputs.paged_case(2006, 3, 2, 8, 2, 128, 128, 64, lengths=[10, 300, 1000],
                           num_splits=5, poison=True, name="partials")
    need = sdpa.decode_workspace_bytes(3, 2, 8, 128, 5)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN-patterned workspace
    o, l = run(pc, workspace=ws)
    rows = 3 * 2 * 8
    o_bytes = ((5 * rows * 128 * 4 + 255) // 256) * 256
    o_part = ws[:5 * rows * 128 * 4].view(torch.float32).view(5, rows, 128)
    lse_part = ws[o_bytes:o_bytes + 5 * rows * 4].view(torch.float32).view(5, rows)
    _, _, op_ref, lp_ref = oracle_decode(pc, num_splits=5, want_partials=True)
    check_lse(lse_part, lp_ref, "LSE partials")
    check_o(o_part, op_ref, "O partials")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("S,dv", [(7, 512), (19, 512), (16, 100)])
def test_combine_matches_oracle_definition(dtype, S, dv):
    g = torch.Generator().manual_seed(2007)
    rows = 100
    o_part = torch.randn(S, rows, dv, generator=g)
    lse_part = torch.randn(S, rows, generator=g) * 4
    lse_part[2, :50] = -math.inf                      # some empty splits
    lse_part[:, 60] = -math.inf                       # a row where every split is empty
    o_part[2, :50] = float("nan")                     # empty splits' partials are never read
    o_ref, l_ref = oracle.combine(o_part.double().numpy(), lse_part.double().numpy())
    o, l = sdpa.splitkv_combine(to_dev(o_part), to_dev(lse_part), out_dtype=dtype)
    torch.cuda.synchronize()
    check_o(o, o_ref)
    check_lse(l, l_ref)
    assert torch.all(o[60] == 0)


@pytest.mark.parametrize("case", [
    # page 32, 3 tokens x 16 heads = 48 rows per KV head (two waves without rows)
    dict(seed=2008, sq=3, hq=16, hkv=1, page=32, lengths=[33, 2100], splits=2, causal=True),
    # page 128, 64 rows per KV head, 2 KV heads, one chunk of 71 pages (page-window reload)
    dict(seed=2009, sq=1, hq=128, hkv=2, page=128, lengths=[9000, 40], splits=1, causal=False),
    # 3 row blocks (2 x 160 = 320 rows), lengths not multiples of a tile
    dict(seed=2010, sq=2, hq=160, hkv=1, page=64, lengths=[97, 1301], splits=3, causal=True),
])
def test_mla_wide_row_edges(case):
    pc = inputs.paged_case(case["seed"], len(case["lengths"]), case["sq"], case["hq"], case["hkv"],
                           576, 512, case["page"], lengths=case["lengths"],
                           num_splits=case["splits"], causal=case["causal"], poison=True,
                           name="mla_edges")
    parity(pc)


# few rows per KV head (e.g. 16 heads of one token when the 128 heads are split over GPUs):
# up to 32 rows the wide kernel computes one row block of O^T per wave
@pytest.mark.parametrize("shape", [(1, 16, 64, 1, True), (1, 1, 32, 3, True), (2, 8, 64, 4, True),
                                   (1, 32, 128, 16, False), (3, 11, 64, 2, True)],
                         ids=["16_rows", "1_row", "2x8_rows", "32_rows", "33_rows"])
def test_mla_few_rows(shape):
    sq, hq, page, splits, causal = shape
    pc = inputs.paged_case(2013, 3, sq, hq, 1, 576, 512, page, lengths=[1, 300, 2500],
                           num_splits=splits, causal=causal, poison=True, name="mla_few_rows")
    parity(pc)


@pytest.mark.parametrize("scale", [-0.05, 0.0])
def test_mla_negative_and_zero_scale(scale):
    pc = inputs.paged_case(2011, 2, 2, 128, 1, 576, 512, 64, lengths=[70, 500], num_splits=2,
                           causal=True, poison=True, scale=scale, name="mla_scale")
    parity(pc)


@pytest.mark.parametrize("splits", [1, 3])
def test_mla_16_key_pages(splits):
    # 16-key pages: a 32-key tile spans two pages, each wave's 8 rows come from one
    pc = inputs.paged_case(2015, 3, 2, 64, 1, 576, 512, 16, lengths=[9, 333, 2100],
                           num_splits=splits, causal=True, poison=True, name="mla_page16")
    assert path_of(pc) == "wide"
    parity(pc)


def test_mla_second_pass_reloads_the_page_window():
    # one chunk of 188 16-key pages (the page-id window of 64 reloads twice) and a late
    # large logit, so the work-group runs the chunk a second time from its first page
    pc = inputs.paged_case(2016, 1, 2, 128, 1, 576, 512, 16, lengths=[3000], num_splits=1,
                           causal=True, poison=True, name="mla_rerun_window")
    key = 40
    page = int(pc.pt_k[0, key // pc.page_size])
    pc.k_pool[page, key % pc.page_size, 0] = (1.5 * pc.q[0, 1, 3].float()).to(pc.k_pool.dtype)
    o, l, _, _ = parity(pc)
    assert float(l[0, 1, 3]) > 30.0


def test_mla_late_large_logit_takes_second_pass():
    # key 40 of sequence 0 is 1.5 x the query of (token 1, head 3): its logit
    # (~36 nats) exceeds the first tile's maxima by far more than 2^32, so the
    # work-group reruns its chunk with the exact max as reference
    pc = inputs.paged_case(2012, 2, 2, 128, 1, 576, 512, 64, lengths=[300, 90], num_splits=2,
                           causal=True, poison=True, name="mla_big_logit")
    key = 40
    page = int(pc.pt_k[0, key // pc.page_size])
    pc.k_pool[page, key % pc.page_size, 0] = (1.5 * pc.q[0, 1, 3].float()).to(pc.k_pool.dtype)
    o, l, o_ref, l_ref = parity(pc)
    assert float(l[0, 1, 3]) > 30.0


def test_d64_decode_workload_sampled():
    # the paged decode workload's shape at D = 64 (B = 64, 32/8 heads, page 64,
    # L U[512, 32768], 8 splits): the few-row kernel's D = 64 instantiation
    pc = inputs.paged_case(inputs.SEED_BASE + 3, 64, 1, 32, 8, 64, 64, 64, lo=512, hi=32768,
                           num_splits=8, poison=True, name="paged_decode_d64")
    o, l = run(pc)
    rows = pc.batch * pc.sq * pc.hq
    sel = sample_rows(rows, 192, 64, must=[0, rows - 1])
    o_ref, l_ref = oracle_decode(pc, sel_rows=sel)
    si = torch.from_numpy(sel).cuda()
    check_o(o.reshape(rows, -1)[si], o_ref)
    check_lse(l.reshape(rows)[si], l_ref)
    assert torch.isfinite(o.float()).all()


# ---- row groups: up to 64 rows per KV head take the few-row kernel in groups of 16 rows,
# each group a unit of its own (a partial last group; causal limits per group).  In bf16
# that is the 192/128 pools: square head dims past 16 rows go to the prefill kernel ------

@pytest.mark.parametrize("shape", [(17, 1, 2, 1), (3, 11, 1, 1), (4, 12, 2, 3), (4, 16, 1, 8)],
                         ids=["17_rows", "33_rows", "48_rows", "64_rows"])
def test_row_groups(shape):
    sq, group, hkv, splits = shape
    pc = inputs.paged_case(2040 + sq * group, 3, sq, group * hkv, hkv, 192, 128, 32,
                           lengths=[2, 130, 1900], num_splits=splits, poison=True,
                           name="row_groups")
    assert path_of(pc) == "row_groups"
    log("row groups: %d rows per KV head" % (sq * group))
    o, l, _, _ = parity(pc)
    # sequence 0 holds 2 keys: with s_q > 2 its first token sees none
    assert torch.all(o[0, 0] == 0) and torch.all(l[0, 0] == -math.inf)


@pytest.mark.timeout(600)
def test_mla_sixteen_heads_workload_sampled():
    # the MLA-shaped workload's sequences with 16 heads of one token (the 128 heads split
    # over 8 GPUs): 16 rows per KV head, one row block of O^T per wave in the wide kernel
    pc = inputs.paged_case(inputs.SEED_BASE + 5, 32, 1, 16, 1, 576, 512, 64, lo=4096, hi=16384,
                           num_splits=16, poison=True, name="mla_decode_16_heads")
    assert path_of(pc) == "wide"
    o, l = run(pc)
    rows = pc.batch * pc.sq * pc.hq
    sel = sample_rows(rows, 192, 2014, must=[0, rows - 1])
    o_ref, l_ref = oracle_decode(pc, sel_rows=sel)
    si = torch.from_numpy(sel).cuda()
    check_o(o.reshape(rows, -1)[si], o_ref)
    check_lse(l.reshape(rows)[si], l_ref)
