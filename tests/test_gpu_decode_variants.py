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
