"""GPU parity of sdpa_prefill_thd against the fp64 oracle (through the C-ABI).

Each case: seeded synthetic inputs -> HIP path on cuda:0 and the oracle on the
same values -> O within |g-o| <= 2e-2 + 2e-2|o|, LSE within 1e-3 (finite rows),
-inf exactly on empty rows, padded rows and masking exact.
"""
import math

import numpy as np
import pytest
import torch

from scaled_dot_product_19_amd import inputs, sdpa
from tests.helpers import check_lse, check_o, log, oracle_prefill, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sdpa.load()  # raises if the HIP library is missing: no fallback


def run(case: inputs.ThdCase, lse_layout=sdpa.LSE_PACKED, lse_s_max=0, q=None, k=None, v=None,
        out=None, lse=None, stream=None):
    q = to_dev(case.q) if q is None else q
    k = to_dev(case.k) if k is None else k
    v = to_dev(case.v) if v is None else v
    o, l = sdpa.prefill_thd(q, k, v, to_dev(case.cu_q), to_dev(case.cu_kv), case.max_q,
                            case.max_kv, case.scale, case.causal, out=out, lse=lse,
                            lse_layout=lse_layout, lse_s_max=lse_s_max, stream=stream)
    torch.cuda.synchronize()
    return o, l


def parity(case, **kw):
    log("prefill parity: %s lengths=%s kv=%s hq=%d hkv=%d d=%d causal=%s scale=%g" % (
        case.name, case.lengths_q[:8], case.lengths_kv[:8], case.hq, case.hkv, case.q.shape[2],
        case.causal, case.scale))
    o, l = run(case, **kw)
    o_ref, l_ref = oracle_prefill(case)
    e_o = check_o(o, o_ref)
    e_l = check_lse(l, l_ref)
    log("  max|dO|=%.3g max|dLSE|=%.3g" % (e_o, e_l))
    return o, l, o_ref, l_ref


@pytest.mark.parametrize("seed", [inputs.SEED_BASE + 1, inputs.SEED_ALT + 1])
def test_tiny_fp32_workload(seed):
    parity(inputs.tiny_fp32(seed))


@pytest.mark.parametrize("seed", [inputs.SEED_BASE + 2, inputs.SEED_ALT + 2])
def test_d128_gqa4_ragged_tiles_and_tails(seed):
    case = inputs.thd_case(seed, hq=32, hkv=8, d_qk=128, lengths=[1, 31, 33, 100, 257, 640],
                           name="d128_gqa4_ragged")
    parity(case)


@pytest.mark.parametrize("seed", [inputs.SEED_BASE + 2, inputs.SEED_ALT + 2])
def test_d128_random_lengths(seed):
    case = inputs.thd_case(seed, hq=32, hkv=8, d_qk=128, batch=4, lo=128, hi=700,
                           name="d128_rand")
    parity(case)


@pytest.mark.parametrize("seed", [inputs.SEED_BASE + 4, inputs.SEED_ALT + 4])
def test_d256_gqa12_padded_lse(seed):
    case = inputs.thd_case(seed, hq=24, hkv=2, d_qk=256, lengths=[300, 77], name="d256_gqa12")
    s_max = 320
    lse = torch.full((2, s_max, 24), 12345.0, device="cuda")  # dirty allocator
    o, l = run(case, lse_layout=sdpa.LSE_PADDED, lse_s_max=s_max, lse=lse)
    o_ref, l_ref = oracle_prefill(case)
    check_o(o, o_ref)
    lp = l.cpu().numpy()
    for b, L in enumerate(case.lengths_q):
        t0 = int(case.cu_q[b])
        check_lse(l[b, :L], l_ref[t0:t0 + L], "padded LSE b=%d" % b)
        assert np.all(lp[b, L:] == -np.inf), "padded rows past Lq must be -inf"


@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (6, 2), (3, 1)])
@pytest.mark.parametrize("causal", [True, False])
def test_d64_gqa_groups(hq, hkv, causal):
    case = inputs.thd_case(77, hq=hq, hkv=hkv, d_qk=64, lengths=[70, 5, 129], causal=causal,
                           name="d64_g%d" % (hq // hkv))
    parity(case)


@pytest.mark.parametrize("lq,lk", [([10, 40], [50, 40]), ([40, 3], [20, 3]), ([96], [1000])])
def test_bottom_right_causal_lq_ne_lk(lq, lk):
    case = inputs.thd_case(88, hq=8, hkv=2, d_qk=128, lengths=lq, lengths_kv=lk,
                           name="bottom_right")
    parity(case)


@pytest.mark.parametrize("scale", [0.0, -0.3, 3.0])
def test_scale_edge_values(scale):
    case = inputs.thd_case(99, hq=8, hkv=2, d_qk=128, lengths=[65, 200], scale=scale,
                           name="scale")
    o, l, o_ref, l_ref = parity(case)
    if scale == 0.0:  # closed form: LSE = ln(number of visible keys)
        lp = l.cpu().numpy()
        for t in (0, 10, 64):
            assert abs(lp[t, 0] - math.log(t + 1)) < 1e-3


def test_empty_sequences_and_rows_without_keys():
    case = inputs.thd_case(5, hq=8, hkv=2, d_qk=128, lengths=[5, 0, 0, 40, 3],
                           lengths_kv=[0, 0, 7, 20, 3], name="empty")
    o, l, _, l_ref = parity(case)
    on = o.float().cpu().numpy()
    assert np.all(on[:5] == 0.0)                                  # Lk = 0
    assert np.all(on[5:5 + 20] == 0.0)                            # Lq=40 > Lk=20: first 20 rows see nothing
    assert np.all(l.cpu().numpy()[:5] == -np.inf)


def test_capacity_tails_poison_and_output_sentinel():
    case = inputs.thd_case(6, hq=8, hkv=2, d_qk=128, lengths=[100, 37], name="capacity")
    extra = 64
    qp, kp, vp = inputs.thd_with_capacity(case, extra)             # NaN capacity rows
    out = torch.full((qp.shape[0], 8, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    o, l = run(case, q=to_dev(qp), k=to_dev(kp), v=to_dev(vp), out=out)
    o_ref, l_ref = oracle_prefill(case)
    T = int(case.cu_q[-1])
    check_o(o[:T], o_ref)
    check_lse(l[:T], l_ref)
    assert torch.all(o[T:] == 7.0), "rows past the last sequence must stay untouched"


def test_strided_token_and_head_gaps():
    case = inputs.thd_case(8, hq=8, hkv=2, d_qk=128, lengths=[50, 90], name="strided")

    def gapped(t):
        T, H, D = t.shape
        big = torch.zeros(T, 2 * H + 1, D + 24, dtype=t.dtype, device="cuda")
        view = big[:, 1:2 * H + 1:2, 8:8 + D]
        view.copy_(to_dev(t))
        return view
    q, k, v = gapped(case.q), gapped(case.k), gapped(case.v)
    obig = torch.zeros(q.shape[0], 3 * 8, 128 + 16, dtype=torch.bfloat16, device="cuda")
    out = obig[:, ::3, 16:]
    o, l = run(case, q=q, k=k, v=v, out=out)
    o_ref, l_ref = oracle_prefill(case)
    check_o(o, o_ref)
    check_lse(l, l_ref)
    assert torch.all(obig[:, 1::3] == 0) and torch.all(obig[:, :, :16] == 0)


def test_non_default_stream():
    case = inputs.thd_case(9, hq=8, hkv=2, d_qk=128, lengths=[64, 65], name="stream")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
        o, l = sdpa.prefill_thd(q, k, v, to_dev(case.cu_q), to_dev(case.cu_kv), case.max_q,
                                case.max_kv, case.scale, True, stream=s)
    s.synchronize()
    o_ref, l_ref = oracle_prefill(case)
    check_o(o, o_ref)
    check_lse(l, l_ref)


def test_deterministic_and_causal_future_keys_bitwise():
    case = inputs.thd_case(10, hq=8, hkv=2, d_qk=128, lengths=[200], name="determinism")
    o1, l1 = run(case)
    o2, l2 = run(case)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    k2, v2 = case.k.clone(), case.v.clone()
    k2[150:] = torch.randn_like(k2[150:].float()).to(torch.bfloat16)
    v2[150:] = torch.randn_like(v2[150:].float()).to(torch.bfloat16)
    o3, l3 = run(case, k=to_dev(k2), v=to_dev(v2))
    assert torch.equal(o1[:150], o3[:150]) and torch.equal(l1[:150], l3[:150])
    assert not torch.equal(l1[150:], l3[150:])


@pytest.mark.parametrize("d", [64, 128, 256])
def test_repeated_calls_are_bitwise_equal(d):
    # identical calls give identical bits, at every head dim (the softmax must read each
    # score accumulator only once its MFMAs are done); large logits (scale 2) included
    for scale in (None, 2.0):
        case = inputs.thd_case(12 + d, hq=8, hkv=2, d_qk=d, lengths=[700, 129, 65, 1],
                               scale=scale, name="repeat_d%d" % d)
        outs = [run(case) for _ in range(4)]
        log("bf16 repeat: D=%d scale=%s, %d calls on lengths %s" % (d, scale, len(outs),
                                                                     case.lengths_q))
        for o, l in outs[1:]:
            assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
        assert torch.isfinite(outs[0][1]).all()


def test_first_causal_row_is_v0_exactly():
    case = inputs.thd_case(11, hq=8, hkv=2, d_qk=128, lengths=[40, 33], name="first_row")
    o, _ = run(case)
    for b in range(2):
        t0 = int(case.cu_q[b])
        for h in range(8):
            assert torch.equal(o[t0, h].cpu(), case.v[t0, h // 4])
