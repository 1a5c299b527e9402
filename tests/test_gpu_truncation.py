"""Rows a call cannot compute come out as NaN, never as a silent partial result.

- THD prefill: the grid covers ceil(max_seqlen_q / R) * R query rows of each sequence (R: rows
  of one work item); rows of a longer sequence past that are written as NaN O and NaN LSE,
  and every covered row still matches the oracle.
- Paged decode: a seq_lens[b] past the page table's reach (table_stride * page_size) is
  clamped for reading, and all of sequence b's output rows are NaN (O and LSE), through every
  decode kernel and with split-KV (a NaN partial makes the merged row NaN); the other
  sequences match the oracle.
"""
import numpy as np
import pytest
import torch

from scaled_dot_product_19_amd import inputs, sdpa
from tests.helpers import check_lse, check_o, log, oracle_decode, oracle_prefill, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sdpa.load()


# rows of one prefill work item: D = 64/128 (8 waves, 4 heads) -> 64, D = 256 (4 waves) -> 32,
# fp32 -> 1
@pytest.mark.parametrize("d,dtype,rows", [(64, torch.bfloat16, 64), (128, torch.bfloat16, 64),
                                          (256, torch.bfloat16, 32), (64, torch.float32, 1)])
def test_prefill_rows_past_max_seqlen_q_are_nan(d, dtype, rows):
    case = inputs.thd_case(3100 + d, hq=8, hkv=2, d_qk=d, lengths=[300, 90], dtype=dtype,
                           name="trunc_q")
    max_q = 90  # below the first sequence's 300 rows
    cover = -(-max_q // rows) * rows
    log("prefill truncation: D=%d %s lengths %s, max_seqlen_q=%d -> rows >= %d of sequence 0 NaN"
        % (d, dtype, case.lengths_q, max_q, cover))
    o, l = sdpa.prefill_thd(to_dev(case.q), to_dev(case.k), to_dev(case.v), to_dev(case.cu_q),
                            to_dev(case.cu_kv), max_q, case.max_kv, case.scale, True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_prefill(case)
    t0, t1 = int(case.cu_q[1]), int(case.cu_q[2])
    assert torch.isnan(o[cover:t0].float()).all() and torch.isnan(l[cover:t0]).all()
    keep = torch.cat([torch.arange(cover), torch.arange(t0, t1)]).cuda()
    kn = keep.cpu().numpy()
    check_o(o[keep], o_ref[kn])
    check_lse(l[keep], l_ref[kn])


def test_fp8_prefill_rows_past_max_seqlen_q_are_nan():
    case = inputs.fp8_thd_case(3199, 8, 2, 128, lengths=[300, 90], name="trunc_q_fp8")
    dq, dk, dv = (torch.tensor([x], dtype=torch.float32, device="cuda") for x in case.descale)
    o, l = sdpa.prefill_thd_fp8(to_dev(case.q), to_dev(case.k), to_dev(case.v),
                                to_dev(case.cu_q), to_dev(case.cu_kv), 90, case.max_kv,
                                case.scale, dq, dk, dv, causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_prefill(case, descale=case.descale)
    assert torch.isnan(o[128:300].float()).all() and torch.isnan(l[128:300]).all()
    keep = torch.cat([torch.arange(128), torch.arange(300, 390)]).cuda()
    check_o(o[keep], o_ref[keep.cpu().numpy()])
    check_lse(l[keep], l_ref[keep.cpu().numpy()])


# (name, factory, splits): one case per decode kernel
DECODE = {
    "few_row_d128": lambda: inputs.paged_case(3201, 3, 1, 32, 8, 128, 128, 64,
                                              lengths=[100, 700, 1500], name="trunc_few"),
    "wide_mla": lambda: inputs.paged_case(3202, 3, 2, 128, 1, 576, 512, 64,
                                          lengths=[90, 700, 1500], name="trunc_wide"),
    "few_row_d64": lambda: inputs.paged_case(3203, 3, 1, 4, 4, 64, 64, 32,
                                             lengths=[77, 300, 900], name="trunc_few_d64"),
    "row_groups_d192_128": lambda: inputs.paged_case(3205, 3, 4, 16, 2, 192, 128, 32,
                                                     lengths=[77, 300, 900],
                                                     name="trunc_row_groups"),
    "general_d192_128": lambda: inputs.paged_case(3206, 3, 4, 32, 1, 192, 128, 32,
                                                  lengths=[77, 300, 900], name="trunc_general"),
    "folded_d64_page32": lambda: inputs.paged_case(3210, 3, 4, 32, 1, 64, 64, 32,
                                                   lengths=[77, 300, 900],
                                                   name="trunc_folded_d64_page32"),
    "chunked_prefill": lambda: inputs.paged_case(3204, 3, 128, 8, 2, 128, 128, 64,
                                                 lengths=[200, 700, 1500], name="trunc_chunked"),
    "folded_rows": lambda: inputs.paged_case(3207, 3, 4, 32, 1, 128, 128, 64,
                                             lengths=[90, 700, 1500], name="trunc_folded"),
    "folded_rows_d64": lambda: inputs.paged_case(3209, 3, 4, 32, 1, 64, 64, 64,
                                                 lengths=[77, 300, 900], name="trunc_folded_d64"),
    "folded_rows_d256": lambda: inputs.paged_case(3208, 3, 2, 32, 2, 256, 256, 32,
                                                  lengths=[90, 700, 1500], name="trunc_folded_d256"),
}


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("path", list(DECODE))
def test_decode_seq_lens_past_the_table_are_nan(path, splits):
    pc = DECODE[path]()
    reach = pc.pt_k.shape[1] * pc.page_size
    lens = pc.seq_lens.clone()
    lens[1] = reach + 5  # sequence 1 claims more keys than its table can address
    log("decode truncation: %s splits=%d reach=%d seq_lens=%s" % (path, splits, reach,
                                                                   lens.tolist()))
    ws = torch.empty(max(1, sdpa.decode_workspace_bytes(pc.batch, pc.sq, pc.hq,
                                                        pc.v_pool.shape[3], splits)),
                     dtype=torch.uint8, device="cuda")
    o, l = sdpa.decode_paged(to_dev(pc.q), to_dev(pc.k_pool), to_dev(pc.v_pool), to_dev(pc.pt_k),
                             to_dev(pc.pt_v), to_dev(lens), reach, pc.scale, pc.causal,
                             num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isnan(o[1].float()).all() and torch.isnan(l[1]).all()
    o_ref, l_ref = oracle_decode(pc, num_splits=splits)
    for b in (0, 2):
        check_o(o[b], o_ref[b])
        check_lse(l[b], l_ref[b])
    assert not torch.isnan(o[0].float()).any() and not torch.isnan(o[2].float()).any()
