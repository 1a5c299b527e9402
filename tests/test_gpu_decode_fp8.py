"""GPU parity of sdpa_decode_paged_fp8 (per-tensor FP8 E4M3 Q/K/V, bf16 O) against the
fp64 oracle on the same codes and descales, through the C-ABI.

The bar is the decode one: O within |g-o| <= 2e-2 + 2e-2|o|, LSE within 1e-3, -inf
exactly where the oracle has -inf.  Pools are poisoned (NaN codes in unused pages and
past each sequence's end) so a stray read shows up as a non-finite output.
"""
import numpy as np
import pytest
import torch

from scaled_dot_product_19_amd import inputs, sdpa
from tests.helpers import check_lse, check_o, log, oracle_decode, sample_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sdpa.load()  # raises if the HIP library is missing: no fallback


def descales(pc):
    return [torch.tensor([x], dtype=torch.float32, device="cuda") for x in pc.descale]


def run(pc, splits=None):
    S = pc.num_splits if splits is None else splits
    dq, dk, dv = descales(pc)
    o, l = sdpa.decode_paged_fp8(to_dev(pc.q), to_dev(pc.k_pool), to_dev(pc.v_pool),
                                 to_dev(pc.pt_k), to_dev(pc.pt_v), to_dev(pc.seq_lens),
                                 pc.max_kv, pc.scale, dq, dk, dv, causal=pc.causal,
                                 num_splits=S)
    torch.cuda.synchronize()
    return o, l


def parity(pc):
    log("fp8 decode parity: %s lens=%s sq=%d hq=%d hkv=%d d=%d page=%d splits=%d descale=%s" % (
        pc.name, pc.seq_lens.tolist()[:8], pc.sq, pc.hq, pc.hkv, pc.q.shape[3], pc.page_size,
        pc.num_splits, pc.descale))
    o, l = run(pc)
    o_ref, l_ref = oracle_decode(pc, descale=pc.descale)
    e_o = check_o(o, o_ref)
    e_l = check_lse(l, l_ref)
    log("  max|dO|=%.3g max|dLSE|=%.3g" % (e_o, e_l))
    return o, l, o_ref, l_ref


@pytest.mark.parametrize("splits", [1, 3, 8])
def test_d128_gqa4_poisoned_pools(splits):
    pc = inputs.fp8_paged_case(3001, 7, 1, 32, 8, 128, 64,
                               lengths=[1, 63, 64, 65, 130, 1000, 2047], num_splits=splits,
                               poison=True, name="fp8_d128_g4")
    parity(pc)


def test_d128_page16_more_splits_than_pages():
    pc = inputs.fp8_paged_case(3002, 3, 1, 8, 2, 128, 16, lengths=[5, 40, 300],
                               num_splits=24, poison=True, name="fp8_page16")
    parity(pc)


@pytest.mark.parametrize("splits", [1, 4])
def test_d256_two_tokens_gqa8(splits):
    # 2 tokens x 8 heads = 16 rows per KV head, bottom-right causal
    pc = inputs.fp8_paged_case(3003, 4, 2, 16, 2, 256, 32, lengths=[1, 2, 77, 900],
                               num_splits=splits, poison=True, name="fp8_d256_mtp")
    parity(pc)


@pytest.mark.parametrize("causal", [True, False])
def test_mtp_tokens_and_keyless_rows(causal):
    # s_q = 4 > L for the first sequence: its first tokens see no key when causal
    pc = inputs.fp8_paged_case(3004, 3, 4, 8, 2, 128, 64, lengths=[2, 64, 515], num_splits=2,
                               causal=causal, poison=True, name="fp8_mtp4")
    o, l, _, _ = parity(pc)
    if causal:
        assert torch.all(l[0, :2] == float("-inf")) and torch.all(o[0, :2] == 0)


@pytest.mark.parametrize("scale", [0.0, -0.125])
def test_scale_edges(scale):
    pc = inputs.fp8_paged_case(3005, 2, 1, 8, 8, 128, 64, lengths=[100, 333], num_splits=2,
                               scale=scale, poison=True, name="fp8_scale")
    parity(pc)


def test_empty_batch_entry_and_zero_length_sequence():
    pc = inputs.fp8_paged_case(3006, 3, 1, 8, 2, 128, 64, lengths=[0, 17, 0], num_splits=3,
                               poison=True, name="fp8_zero_len")
    o, l, _, _ = parity(pc)
    assert torch.all(l[0] == float("-inf")) and torch.all(o[0] == 0)


def test_descales_read_on_the_device():
    # the same codes with descales doubled / halved: O doubles with descale_v (exactly,
    # a power of two), LSE moves with descale_q * descale_k
    pc = inputs.fp8_paged_case(3007, 2, 1, 8, 2, 128, 64, lengths=[50, 700], num_splits=1,
                               name="fp8_descale")
    o1, l1 = run(pc)
    import dataclasses
    dq, dk, dv = pc.descale
    pc2 = dataclasses.replace(pc, descale=(dq * 2.0, dk * 0.5, dv * 2.0))
    o2, l2 = run(pc2)
    assert torch.equal(o2.float(), o1.float() * 2.0)
    assert torch.equal(l2, l1)


def test_full_size_fp8_decode_sampled():
    pc = inputs.paged_decode_d128_fp8()
    log("full-size %s pages=%d" % (pc.name, pc.k_pool.shape[0]))
    o, l = run(pc)
    rows = pc.batch * pc.sq * pc.hq
    sel = sample_rows(rows, 192, 3, must=[0, rows - 1])
    o_ref, l_ref = oracle_decode(pc, sel_rows=sel, descale=pc.descale)
    check_o(o.reshape(rows, -1)[torch.from_numpy(sel).cuda()], o_ref)
    check_lse(l.reshape(rows)[torch.from_numpy(sel).cuda()], l_ref)
    assert torch.isfinite(o.float()).all() and torch.isfinite(l).all()
