"""GPU parity of the decode variants against the fp64 oracle: multi-token (MTP) decode with
q_tokens = 1..4, the non-absorbed MLA pools (d_qk 192, d_v 128), and the absorbed-MLA
aliased cache (V = the first 512 columns of the 576-wide K rows, one page table).

Sources: q_tokens = 1 + MTP for MTP 0..3 in the generation phase of the attention benchmark
(cuDNN Frontend v1.28.0 release notes, "Samples, Benchmarks, and Tests"); d_qk 192 / d_v 128
(v1.28.0 "New: FROST SDPA on Ampere, Ada/Blackwell-consumer, and Rubin"); Q/K 576 with V 512
over independent or shared K/V layouts (v1.32.0 "SDPA: wider native forward support").
"""
import dataclasses

import pytest
import torch

from scaled_dot_product_19_amd import inputs, sdpa
from tests.helpers import check_lse, check_o, log, oracle_decode, sample_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sdpa.load()


def run(pc, k_pool=None, v_pool=None):
    kp = to_dev(pc.k_pool) if k_pool is None else k_pool
    vp = to_dev(pc.v_pool) if v_pool is None else v_pool
    o, l = sdpa.decode_paged(to_dev(pc.q), kp, vp, to_dev(pc.pt_k), to_dev(pc.pt_v),
                             to_dev(pc.seq_lens), pc.max_kv, pc.scale, pc.causal,
                             num_splits=pc.num_splits)
    torch.cuda.synchronize()
    return o, l


def parity(pc, sel_rows=None, **kw):
    log("decode variant parity: %s lens=%s sq=%d hq=%d hkv=%d d=%d/%d page=%d splits=%d" % (
        pc.name, pc.seq_lens.tolist()[:8], pc.sq, pc.hq, pc.hkv, pc.q.shape[3],
        pc.v_pool.shape[3], pc.page_size, pc.num_splits))
    o, l = run(pc, **kw)
    o_ref, l_ref = oracle_decode(pc, sel_rows=sel_rows)
    if sel_rows is None:
        e_o, e_l = check_o(o, o_ref), check_lse(l, l_ref)
    else:
        rows = pc.batch * pc.sq * pc.hq
        idx = torch.from_numpy(sel_rows).cuda()
        e_o = check_o(o.reshape(rows, -1)[idx], o_ref)
        e_l = check_lse(l.reshape(rows)[idx], l_ref)
    log("  max|dO|=%.3g max|dLSE|=%.3g" % (e_o, e_l))
    return o, l


@pytest.mark.parametrize("q_tokens", [1, 2, 3, 4])
def test_mtp_decode_d128(q_tokens):
    # 32/8 heads: 4 .. 16 query rows per KV head; L = 2 < q_tokens leaves leading tokens keyless
    pc = inputs.paged_case(2201 + q_tokens, 6, q_tokens, 32, 8, 128, 128, 64,
                           lengths=[2, 64, 65, 700, 3000, 9000], num_splits=8, poison=True,
                           name="mtp%d" % q_tokens)
    parity(pc)


@pytest.mark.parametrize("shape", [(1, 16, 1, 64, 1), (2, 8, 2, 32, 4), (4, 64, 4, 64, 3)],
                         ids=["sq1_g16", "sq2_g4_page32", "sq4_g16_split3"])
def test_d192_d128_pools(shape):
    sq, hq, hkv, page, splits = shape
    pc = inputs.paged_case(2210 + sq, 3, sq, hq, hkv, 192, 128, page, lengths=[3, 200, 1500],
                           num_splits=splits, poison=True, name="d192x128")
    parity(pc)


def aliased_mla(seed, lengths, sq=2, hq=128, splits=4):
    """Absorbed-MLA cache with V aliased into K: one 576-wide pool and one page table; V is
    the first 512 columns of each K row."""
    pc = inputs.paged_case(seed, len(lengths), sq, hq, 1, 576, 576, 64, lengths=lengths,
                           num_splits=splits, poison=True, name="mla_aliased")
    return dataclasses.replace(pc, v_pool=pc.k_pool[..., :512], pt_v=pc.pt_k)


@pytest.mark.parametrize("splits", [1, 4])
def test_absorbed_mla_aliased_cache(splits):
    pc = aliased_mla(2220 + splits, [1, 65, 700, 3000], splits=splits)
    kp = to_dev(pc.k_pool)
    o, l = parity(pc, k_pool=kp, v_pool=kp[..., :512])
    assert torch.isfinite(o).all()


def test_absorbed_mla_aliased_cache_full_size_sampled():
    base = inputs.mla_decode()
    pc = aliased_mla(2225, base.seq_lens.tolist(), splits=16)
    rows = pc.batch * pc.sq * pc.hq
    sel = sample_rows(rows, 96, 9, must=[0, rows - 1])
    kp = to_dev(pc.k_pool)
    parity(pc, sel_rows=sel, k_pool=kp, v_pool=kp[..., :512])


# ---- fewer, longer chunks in the absorbed-MLA kernel ---------------------------------------
# When num_splits would give more than two work-groups per CU, the 576/512 kernel gives
# `merge` adjacent chunks to one work-group: slot cg * merge holds the partial of their union,
# the group's other slots are empty (LSE -inf, O never written and never read by the merge).

def mla_merge_factor(batch, splits, n_rb=2):
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    return max(1, min(splits, batch * splits * n_rb // (2 * n_cu)))


@pytest.mark.parametrize("splits", [16, 17, 40])
def test_mla_merged_chunks_partials_and_result(splits):
    import numpy as np
    import oracle
    lengths = [int(x) for x in np.random.default_rng(2230 + splits).integers(1, 2600, 32)]
    lengths[3] = 1   # a one-key sequence: every group but the first is empty
    pc = inputs.paged_case(2230 + splits, 32, 2, 128, 1, 576, 512, 64, lengths=lengths,
                           num_splits=splits, poison=True, name="mla_merge")
    m = mla_merge_factor(pc.batch, splits)
    log("MLA merged chunks: splits=%d merge=%d lens=%s" % (splits, m, lengths[:6]))
    rows = pc.batch * pc.sq * pc.hq
    need = sdpa.decode_workspace_bytes(pc.batch, pc.sq, pc.hq, 512, splits)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN-patterned
    o, l = sdpa.decode_paged(to_dev(pc.q), to_dev(pc.k_pool), to_dev(pc.v_pool), to_dev(pc.pt_k),
                             to_dev(pc.pt_v), to_dev(pc.seq_lens), pc.max_kv, pc.scale,
                             pc.causal, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    o_ref, l_ref, op_ref, lp_ref = oracle_decode(pc, num_splits=splits, want_partials=True)
    check_o(o, o_ref)
    check_lse(l, l_ref)
    o_bytes = ((splits * rows * 512 * 4 + 255) // 256) * 256
    o_part = ws[:splits * rows * 512 * 4].view(torch.float32).view(splits, rows, 512)
    lse_part = ws[o_bytes:o_bytes + splits * rows * 4].view(torch.float32).view(splits, rows)
    for c0 in range(0, splits, m):
        group = list(range(c0, min(splits, c0 + m)))
        # the union's partial = the oracle's LSE merge of the group's chunk partials
        og, lg = oracle.combine(op_ref[group], lp_ref[group])
        check_lse(lse_part[c0], lg, "LSE partial of chunks %s" % group)
        live = np.isfinite(lg)
        check_o(o_part[c0][torch.from_numpy(live).cuda()], og[live], "O partial of chunks %s" % group)
        for c in group[1:]:
            assert torch.all(lse_part[c] == float("-inf")), "slot %d of a merged group" % c
