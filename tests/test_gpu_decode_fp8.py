"""GPU parity of sdpa_decode_paged_fp8 (per-tensor FP8 E4M3 Q/K/V, bf16 O) against the
fp64 oracle on the same codes and descales, through the C-ABI: the few-row kernel (D = 64,
128, 256 and 192/128, up to 64 query rows per KV head in groups of 16), the FP8 prefill
kernel over the page tables (D = 128 with page sizes that are multiples of 64, past 32 rows
per KV head and without an upper limit; with few tokens, the (token, head) rows of a GQA
group are folded into its items) and the general decode kernel (the rest, up to
512 rows per KV head, e.g. 576/512).

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


# ---- the general decode kernel in FP8: more than 16 rows per KV head, D = 64, 192/128 and
# the absorbed-MLA 576/512 (cuDNN Frontend v1.32.0 Release Notes, "SDPA: wider native
# forward support": native D64 per-tensor FP8 and Q/K 576 with V 512) -------------------

@pytest.mark.parametrize("splits", [1, 3])
def test_d128_mtp_rows_in_two_row_groups(splits):
    # 4 tokens x 8 heads = 32 rows per KV head: two 16-row groups of the few-row kernel
    # (page 32 keeps the shape off the prefill kernel)
    pc = inputs.fp8_paged_case(3011, 3, 4, 32, 4, 128, 32, lengths=[2, 300, 1400],
                               num_splits=splits, poison=True, name="fp8_mtp_g8")
    o, _, _, _ = parity(pc)
    assert torch.all(o[0, :2] == 0)


@pytest.mark.parametrize("splits", [1, 4])
def test_d256_rows_in_two_row_groups(splits):
    # 4 tokens x 8 heads = 32 rows per KV head at D = 256
    pc = inputs.fp8_paged_case(3012, 2, 4, 16, 2, 256, 32, lengths=[90, 1100],
                               num_splits=splits, poison=True, name="fp8_d256_g8")
    parity(pc)


@pytest.mark.parametrize("shape", [(1, 8, 2, 32, 1), (3, 16, 4, 64, 3)],
                         ids=["sq1_g4", "sq3_g4_split3"])
def test_d64(shape):
    sq, hq, hkv, page, splits = shape
    pc = inputs.fp8_paged_case(3013 + sq, 3, sq, hq, hkv, 64, page, lengths=[1, 250, 1700],
                               num_splits=splits, poison=True, name="fp8_d64")
    parity(pc)


@pytest.mark.parametrize("splits", [1, 4])
@pytest.mark.parametrize("hq", [16, 32], ids=["16_rows", "32_rows"])
def test_d192_d128_pools(splits, hq):
    # 2 tokens x hq / 2 heads per KV head: the few-row kernel (16 rows), the general one (32)
    pc = inputs.fp8_paged_case(3017, 3, 2, hq, 2, 192, 32, lengths=[5, 333, 1200],
                               num_splits=splits, poison=True, name="fp8_d192x128", d_v=128)
    parity(pc)


@pytest.mark.parametrize("splits", [1, 4])
def test_absorbed_mla_aliased_fp8_cache(splits):
    # one 576-wide E4M3 pool, V = the first 512 columns of each K row (descale_v = descale_k)
    import dataclasses
    pc = inputs.fp8_paged_case(3018, 3, 2, 32, 1, 576, 64, lengths=[1, 700, 2000],
                               num_splits=splits, poison=True, name="fp8_mla_aliased")
    dq, dk, _ = pc.descale
    pc = dataclasses.replace(pc, v_pool=pc.k_pool[..., :512], pt_v=pc.pt_k, descale=(dq, dk, dk))
    log("fp8 aliased MLA: lens=%s splits=%d" % (pc.seq_lens.tolist(), splits))
    kp = to_dev(pc.k_pool)
    d_q, d_k, d_v = descales(pc)
    o, l = sdpa.decode_paged_fp8(to_dev(pc.q), kp, kp[..., :512], to_dev(pc.pt_k),
                                 to_dev(pc.pt_k), to_dev(pc.seq_lens), pc.max_kv, pc.scale,
                                 d_q, d_k, d_v, causal=pc.causal, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_decode(pc, descale=pc.descale)
    log("  max|dO|=%.3g max|dLSE|=%.3g" % (check_o(o, o_ref), check_lse(l, l_ref)))


def test_512_rows_per_kv_head_and_past_them():
    # 4 tokens x 128 heads over one KV head on 32-key pages (general kernel): the most rows
    # it serves; past them only the prefill kernel (pages of 64k keys) takes the call
    pc = inputs.fp8_paged_case(3019, 2, 4, 128, 1, 128, 32, lengths=[6, 900], num_splits=2,
                               poison=True, name="fp8_512rows")
    parity(pc)
    pc5 = inputs.fp8_paged_case(3020, 1, 5, 128, 1, 128, 32, lengths=[900], name="fp8_640rows")
    with pytest.raises(sdpa.SdpaError) as ei:
        run(pc5)
    assert ei.value.status == sdpa.SDPA_ERR_UNSUPPORTED


# ---- the FP8 prefill kernel over the page tables (D = 128, pages of a multiple of 64 keys):
# chunked prefill, and few tokens of a GQA group with their (token, head) rows
# folded into the 256-row items --------------------------------------------------------------

FP8_PAGED_PREFILL = [
    # (seed, batch, s_q, h_q, h_kv, page, lengths, splits, causal, scale)
    (3021, 3, 8, 32, 4, 64, [2, 300, 1400], 1, True, None),      # folded: 64 rows
    (3022, 3, 5, 32, 4, 64, [2, 300, 1400], 3, True, None),      # folded: 40 rows
    (3023, 1, 5, 128, 1, 64, [900], 2, True, None),              # folded: 640 rows, 3 items
    (3024, 2, 3, 64, 2, 128, [0, 777], 1, True, None),           # folded: 96 rows, page 128
    (3025, 2, 100, 8, 2, 64, [120, 1500], 1, True, None),        # chunk of 100 tokens, G 4
    (3026, 2, 100, 8, 2, 64, [120, 1500], 4, False, None),
    (3027, 2, 16, 32, 4, 64, [40, 900], 2, True, -0.07),         # negative scale
    (3028, 2, 16, 32, 4, 64, [40, 900], 1, True, 0.0),           # zero scale
]


@pytest.mark.parametrize("case", FP8_PAGED_PREFILL, ids=[str(c[0]) for c in FP8_PAGED_PREFILL])
def test_fp8_paged_prefill_kernel(case):
    seed, batch, sq, hq, hkv, page, lengths, splits, causal, scale = case
    pc = inputs.fp8_paged_case(seed, batch, sq, hq, hkv, 128, page, lengths=lengths,
                               num_splits=splits, causal=causal, scale=scale, poison=True,
                               name="fp8_paged_prefill_%d" % seed)
    log("fp8 paged prefill: %d rows per KV head" % (sq * hq // hkv))
    o, l, _, _ = parity(pc)
    assert torch.isfinite(o.float()).all()
    if causal and lengths[0] < sq:
        assert torch.all(o[0, 0] == 0) and torch.all(l[0, 0] == -np.inf)
