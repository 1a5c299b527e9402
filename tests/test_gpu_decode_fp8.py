"""GPU parity of sdpa_decode_paged_fp8 (per-tensor FP8 E4M3 Q/K/V, bf16 O) against the
fp64 oracle on the same codes and descales, through the C-ABI and every kernel it takes:
- the few-row kernel (D = 64, 128, 256 and 192/128, up to 64 query rows per KV head in
  groups of 16);
- the FP8 prefill kernel over the page tables (D = 128 with page sizes that are multiples
  of 64, past 32 rows per KV head and without an upper limit; with few tokens, the
  (token, head) rows of a GQA group are folded into its items);
- the absorbed-MLA wide kernel (576/512, the codes widened to bf16 in LDS and in
  registers);
- the general decode kernel (the rest, up to 512 rows per KV head).

The bar is the decode one: O within |g-o| <= 2e-2 + 2e-2|o|, LSE within 1e-3, -inf
exactly where the oracle has -inf.  Pools are poisoned (NaN codes in unused pages and
past each sequence's end) so a stray read shows up as a non-finite output.
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
    log("fp8 decode parity: %s lens=%s sq=%d hq=%d hkv=%d d=%d page=%d splits=%d descale=%s "
        "kernel=%s" % (pc.name, pc.seq_lens.tolist()[:8], pc.sq, pc.hq, pc.hkv, pc.q.shape[3],
                       pc.page_size, pc.num_splits, pc.descale, path_of(pc, fp8=True)))
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


# ---- FP8 past 16 rows per KV head: row groups of the few-row kernel, the general decode
# kernel, D = 64, 192/128 and the absorbed-MLA 576/512 (cuDNN Frontend v1.32.0 Release
# Notes, "SDPA: wider native forward support": native D64 per-tensor FP8 and Q/K 576 with
# V 512) --------------------------------------------------------------------------------

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
    # 4 tokens x 128 heads over one KV head at D = 64 (general kernel): the most rows it
    # serves; past them only the FP8 prefill kernel (D = 128) takes a call
    pc = inputs.fp8_paged_case(3019, 2, 4, 128, 1, 64, 32, lengths=[6, 900], num_splits=2,
                               poison=True, name="fp8_512rows")
    assert path_of(pc, fp8=True) == "general"
    parity(pc)
    pc5 = inputs.fp8_paged_case(3020, 1, 5, 128, 1, 64, 32, lengths=[900], name="fp8_640rows")
    with pytest.raises(sdpa.SdpaError) as ei:
        run(pc5)
    assert ei.value.status == sdpa.SDPA_ERR_UNSUPPORTED


# ---- the absorbed-MLA wide kernel in FP8 (576/512 codes, more than 16 rows per KV head,
# any page size) ----------------------------------------------------------------------------

def mla8(seed, batch, sq, hq, lengths=None, page=64, splits=1, causal=True, scale=None,
         lo=0, hi=0, name="fp8_mla"):
    return inputs.fp8_paged_case(seed, batch, sq, hq, 1, 576, page, lo=lo, hi=hi, lengths=lengths,
                                 num_splits=splits, causal=causal, scale=scale, poison=True,
                                 name=name, d_v=512)


@pytest.mark.parametrize("splits", [1, 16])
def test_mla_wide_fp8_two_tokens_causal(splits):
    pc = mla8(3031, 3, 2, 128, lengths=[1, 65, 700], splits=splits)
    o, l, _, _ = parity(pc)
    # L = 1 < s_q = 2: token 0 sees no key
    assert torch.all(l[0, 0] == -np.inf) and torch.all(o[0, 0] == 0)


@pytest.mark.parametrize("case", [
    # 3 tokens x 16 heads = 48 rows (two waves without rows), page 32, two splits
    dict(seed=3032, sq=3, hq=16, page=32, lengths=[33, 2100], splits=2, causal=True),
    # 320 rows in 3 row blocks, page 128, lengths not multiples of a tile
    dict(seed=3033, sq=2, hq=160, page=128, lengths=[97, 1301], splits=3, causal=True),
    # one chunk of 71 pages (the page-id window reloads), non-causal
    dict(seed=3034, sq=1, hq=64, page=128, lengths=[9000, 40], splits=1, causal=False),
])
def test_mla_wide_fp8_row_edges(case):
    pc = mla8(case["seed"], len(case["lengths"]), case["sq"], case["hq"], lengths=case["lengths"],
              page=case["page"], splits=case["splits"], causal=case["causal"])
    parity(pc)


@pytest.mark.parametrize("shape", [(1, 16, 64, 1, True), (1, 1, 32, 3, True), (2, 8, 64, 4, True),
                                   (1, 32, 128, 16, False), (3, 11, 64, 2, True)],
                         ids=["16_rows", "1_row", "2x8_rows", "32_rows", "33_rows"])
def test_mla_wide_fp8_few_rows(shape):
    sq, hq, page, splits, causal = shape
    parity(mla8(3041, 3, sq, hq, lengths=[1, 300, 2500], page=page, splits=splits, causal=causal,
                name="fp8_mla_few_rows"))


@pytest.mark.parametrize("scale", [-0.05, 0.0])
def test_mla_wide_fp8_negative_and_zero_scale(scale):
    pc = mla8(3035, 2, 2, 128, lengths=[70, 500], splits=2, scale=scale)
    parity(pc)


def test_mla_wide_fp8_late_large_logit_takes_second_pass():
    # as the bf16 case: key 40 of sequence 0 is 1.5 x the query of (token 1, head 3) before
    # quantization, a logit far above the first tile's maxima, so the work-group reruns
    # its chunk with the exact max as reference
    import dataclasses
    pc = inputs.paged_case(3036, 2, 2, 128, 1, 576, 512, 64, lengths=[300, 90], num_splits=2,
                           causal=True, dtype=torch.float32, poison=True, name="fp8_mla_big")
    key = 40
    page = int(pc.pt_k[0, key // pc.page_size])
    pc.k_pool[page, key % pc.page_size, 0] = 1.5 * pc.q[0, 1, 3]
    q8, dq = inputs.quantize_e4m3(pc.q)
    k8, dk = inputs.quantize_e4m3(pc.k_pool)
    v8, dv = inputs.quantize_e4m3(pc.v_pool)
    pc = dataclasses.replace(pc, q=q8, k_pool=k8, v_pool=v8, descale=(dq, dk, dv))
    o, l, _, _ = parity(pc)
    assert float(l[0, 1, 3]) > 30.0


@pytest.mark.parametrize("splits", [1, 3])
def test_mla_wide_fp8_16_key_pages(splits):
    pc = mla8(3043, 3, 2, 64, lengths=[9, 333, 2100], page=16, splits=splits)
    assert path_of(pc, fp8=True) == "wide"
    parity(pc)


def test_mla_wide_fp8_descales_read_on_the_device():
    import dataclasses
    pc = mla8(3037, 2, 2, 64, lengths=[300, 1000], splits=4)
    o1, l1 = run(pc)
    dq, dk, dv = pc.descale
    o2, l2 = run(dataclasses.replace(pc, descale=(dq * 2.0, dk * 0.5, dv * 2.0)))
    assert torch.equal(o2.float(), o1.float() * 2.0)
    assert torch.equal(l2, l1)


def test_mla_wide_fp8_seq_lens_past_the_table_are_nan():
    pc = mla8(3038, 3, 2, 64, lengths=[90, 700, 1500], splits=3)
    reach = pc.pt_k.shape[1] * pc.page_size
    lens = pc.seq_lens.clone()
    lens[1] = reach + 5
    dq, dk, dv = descales(pc)
    o, l = sdpa.decode_paged_fp8(to_dev(pc.q), to_dev(pc.k_pool), to_dev(pc.v_pool),
                                 to_dev(pc.pt_k), to_dev(pc.pt_v), to_dev(lens), reach, pc.scale,
                                 dq, dk, dv, causal=pc.causal, num_splits=3)
    torch.cuda.synchronize()
    assert torch.isnan(o[1].float()).all() and torch.isnan(l[1]).all()
    o_ref, l_ref = oracle_decode(pc, descale=pc.descale)
    for b in (0, 2):
        check_o(o[b], o_ref[b])
        check_lse(l[b], l_ref[b])


@pytest.mark.timeout(600)
def test_mla_wide_fp8_full_size_sampled():
    # the MLA-shaped decode workload (B = 32, 2 tokens, 128/1 heads, L U[4096, 16384],
    # page 64, 16 splits) in per-tensor FP8
    pc = mla8(inputs.SEED_BASE + 5, 32, 2, 128, lo=4096, hi=16384, splits=16,
              name="fp8_mla_decode_workload")
    o, l = run(pc)
    rows = pc.batch * pc.sq * pc.hq
    sel = sample_rows(rows, 256, 3039, must=[0, rows - 1])
    o_ref, l_ref = oracle_decode(pc, sel_rows=sel, descale=pc.descale)
    si = torch.from_numpy(sel).cuda()
    log("fp8 MLA full size: max|dO|=%.3g max|dLSE|=%.3g" % (
        check_o(o.reshape(rows, -1)[si], o_ref), check_lse(l.reshape(rows)[si], l_ref)))
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_mla_wide_repeated_calls_are_bitwise_equal(fp8):
    # the wide kernel's S^T MFMAs are hand-scheduled inline asm: repeated calls on the same
    # inputs (one and several splits) must give the same bits
    for splits in (1, 8):
        if fp8:
            pc = mla8(3040, 4, 2, 128, lengths=[5, 900, 2000, 3100], splits=splits)
            outs = [run(pc) for _ in range(4)]
        else:
            pc = inputs.paged_case(3040, 4, 2, 128, 1, 576, 512, 64, lengths=[5, 900, 2000, 3100],
                                   num_splits=splits, poison=True, name="mla_repeat")
            args = [to_dev(x) for x in (pc.q, pc.k_pool, pc.v_pool, pc.pt_k, pc.pt_v, pc.seq_lens)]
            outs = []
            for _ in range(4):
                outs.append(sdpa.decode_paged(*args, pc.max_kv, pc.scale, True, num_splits=splits))
                torch.cuda.synchronize()
        for o, l in outs[1:]:
            assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


# ---- the FP8 prefill kernel over the page tables (D = 128, any page size):
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


@pytest.mark.timeout(600)
def test_fp8_folded_rows_decode_workload_sampled():
    # the paged decode workload's sequences in FP8 (B = 64, 32/8 heads, D = 128, page 64,
    # L U[512, 32768], 8 splits) with 16 query tokens: 64 folded rows per KV head on the FP8
    # prefill kernel over the page tables
    pc = inputs.fp8_paged_case(inputs.SEED_BASE + 3, 64, 16, 32, 8, 128, 64, lo=512, hi=32768,
                               num_splits=8, poison=True, name="fp8_folded_decode_workload")
    assert path_of(pc, fp8=True) == "prefill_folded"
    o, l = run(pc)
    rows = pc.batch * pc.sq * pc.hq
    sel = sample_rows(rows, 256, 3042, must=[0, rows - 1])
    o_ref, l_ref = oracle_decode(pc, sel_rows=sel, descale=pc.descale)
    si = torch.from_numpy(sel).cuda()
    check_o(o.reshape(rows, -1)[si], o_ref)
    check_lse(l.reshape(rows)[si], l_ref)
    assert torch.isfinite(o.float()).all()
