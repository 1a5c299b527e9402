"""GPU check of sdpa_decode_paged_noalloc (through the C-ABI) against sdpa_decode_paged.

The no-allocation entry point runs the same kernels with the split partials in the
library-owned device array.  Two calls in a row, the second on a smaller input, each
compared with the workspace entry point on the same inputs (and with the oracle) to the
parity bar; a call whose split workspace exceeds the array is declined before launch.
"""
import pytest
import torch

from scaled_dot_product_19_amd import inputs, sdpa
from tests.helpers import check_lse, check_o, log, oracle_decode, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sdpa.load()


def _both(pc):
    q, kp, vp = to_dev(pc.q), to_dev(pc.k_pool), to_dev(pc.v_pool)
    ptk, ptv, sl = to_dev(pc.pt_k), to_dev(pc.pt_v), to_dev(pc.seq_lens)
    dv = int(pc.v_pool.shape[3])
    o_ref, l_ref = sdpa.decode_paged(q, kp, vp, ptk, ptv, sl, pc.max_kv, pc.scale, pc.causal,
                                     num_splits=pc.num_splits)
    o = torch.full((pc.batch, pc.sq, pc.hq, dv), 3.0, dtype=torch.bfloat16, device="cuda")
    l = torch.full((pc.batch, pc.sq, pc.hq), 3.0, dtype=torch.float32, device="cuda")
    sdpa.decode_paged_noalloc(q, kp, vp, ptk, ptv, sl, pc.max_kv, pc.scale, out=o, lse=l,
                              causal=pc.causal, num_splits=pc.num_splits)
    torch.cuda.synchronize()
    return o, l, o_ref, l_ref


def test_noalloc_matches_the_workspace_entry_twice_second_smaller():
    # the second call is smaller in input and in workspace, so it reuses the start of the
    # array the first call filled; the third runs the wide (576/512) decode kernel
    cases = [
        inputs.paged_case(3001, 16, 1, 32, 8, 128, 128, 64, lo=512, hi=8192, num_splits=8,
                          poison=True, name="noalloc_first"),
        inputs.paged_case(3002, 5, 1, 32, 8, 128, 128, 64, lengths=[33, 700, 64, 1, 2000],
                          num_splits=4, poison=True, name="noalloc_second_smaller"),
        inputs.paged_case(3005, 3, 2, 128, 1, 576, 512, 64, lengths=[70, 700, 1300],
                          num_splits=4, poison=True, name="noalloc_wide_kernel"),
    ]
    for pc in cases:
        need = sdpa.decode_workspace_bytes(pc.batch, pc.sq, pc.hq, int(pc.v_pool.shape[3]),
                                           pc.num_splits)
        log("noalloc: %s B=%d sq=%d hq=%d splits=%d workspace=%d bytes" % (
            pc.name, pc.batch, pc.sq, pc.hq, pc.num_splits, need))
        o, l, o_ref, l_ref = _both(pc)
        check_o(o, o_ref.double().cpu().numpy(), "O vs sdpa_decode_paged")
        check_lse(l, l_ref.double().cpu().numpy(), "LSE vs sdpa_decode_paged")
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref), "same kernels: same bits"
        o_or, l_or = oracle_decode(pc)
        check_o(o, o_or)
        check_lse(l, l_or)


def test_noalloc_one_split_and_oversized_workspace():
    pc = inputs.paged_case(3003, 4, 1, 8, 2, 128, 128, 64, lengths=[5, 64, 300, 1000],
                           num_splits=1, poison=True, name="noalloc_one_split")
    o, l, o_ref, l_ref = _both(pc)
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    # 16 splits x 8192 rows x 512 fp32 = 268 MB of partials: more than the 32 MiB array
    big = inputs.paged_case(3004, 32, 2, 128, 1, 576, 512, 64, lengths=[64] * 32,
                            num_splits=16, name="noalloc_too_big")
    out = torch.empty((32, 2, 128, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sdpa.SdpaError) as ei:
        sdpa.decode_paged_noalloc(to_dev(big.q), to_dev(big.k_pool), to_dev(big.v_pool),
                                  to_dev(big.pt_k), to_dev(big.pt_v), to_dev(big.seq_lens),
                                  big.max_kv, big.scale, out=out, num_splits=16)
    assert ei.value.status == sdpa.SDPA_ERR_WORKSPACE
