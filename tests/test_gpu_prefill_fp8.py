"""GPU parity of sdpa_prefill_thd_fp8 (per-tensor FP8 E4M3 Q/K/V, bf16 O) against the
fp64 oracle on the same codes and descales, through the C-ABI.

The bar is the prefill one: O within |g-o| <= 2e-2 + 2e-2|o|, LSE within 1e-3 (a base-2
LSE compared after multiplying by ln 2), -inf exactly where the oracle has -inf.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

from scaled_dot_product_19_amd import inputs, sdpa
from tests.helpers import check_lse, check_o, log, oracle_prefill, thd_sample, to_dev

pytestmark = pytest.mark.gpu

LN2 = math.log(2.0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sdpa.load()  # raises if the HIP library is missing: no fallback


def run(case, window=0, sinks=None, lse_layout=sdpa.LSE_PACKED, stats_log2=False):
    dq, dk, dv = (torch.tensor([x], dtype=torch.float32, device="cuda") for x in case.descale)
    o, l = sdpa.prefill_thd_fp8(to_dev(case.q), to_dev(case.k), to_dev(case.v),
                                to_dev(case.cu_q), to_dev(case.cu_kv), case.max_q, case.max_kv,
                                case.scale, dq, dk, dv, causal=case.causal, window_left=window,
                                sinks=None if sinks is None else to_dev(sinks),
                                lse_layout=lse_layout, stats_log2=stats_log2)
    torch.cuda.synchronize()
    return o, l


def parity(case, window=0, sinks=None, lse_layout=sdpa.LSE_PACKED, stats_log2=False):
    log("fp8 prefill parity: %s lengths=%s kv=%s hq=%d hkv=%d causal=%s scale=%g W=%d sinks=%s "
        "descale=%s" % (case.name, case.lengths_q[:8], case.lengths_kv[:8], case.hq, case.hkv,
                        case.causal, case.scale, window, sinks is not None, case.descale))
    o, l = run(case, window, sinks, lse_layout, stats_log2)
    s = None if sinks is None else sinks.double().numpy()
    o_ref, l_ref = oracle_prefill(case, window=window, sinks=s, descale=case.descale)
    if lse_layout == sdpa.LSE_HEAD_MAJOR:
        l = l[:, :int(case.cu_q[-1])].t()
    if stats_log2:
        l = l * LN2
    e_o = check_o(o, o_ref)
    e_l = check_lse(l, l_ref)
    log("  max|dO|=%.3g max|dLSE|=%.3g" % (e_o, e_l))
    return o, l, o_ref, l_ref


RAGGED = [1, 31, 33, 100, 257, 640]


@pytest.mark.parametrize("seed", [4001, 4101])
def test_d128_gqa4_ragged(seed):
    parity(inputs.fp8_thd_case(seed, 32, 8, 128, lengths=RAGGED, name="fp8_d128_gqa4"))


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (24, 2)])
def test_head_groupings(hq, hkv):
    parity(inputs.fp8_thd_case(4002, hq, hkv, 128, lengths=[65, 300, 7],
                               name="fp8_d128_h%dx%d" % (hq, hkv)))


@pytest.mark.parametrize("causal", [True, False])
def test_unequal_query_and_key_lengths(causal):
    # shift = Lk - Lq > 0, < 0 and 0; causal rows before the diagonal see no key
    case = inputs.fp8_thd_case(4003, 8, 2, 128, lengths=[50, 200, 129],
                               lengths_kv=[300, 150, 129], causal=causal, name="fp8_shift")
    parity(case)


def test_window_sinks_log2_head_major():
    case = inputs.fp8_thd_case(4004, 32, 8, 128, lengths=RAGGED, name="fp8_swa")
    parity(case, window=100, sinks=inputs.sink_logits(4004, 32), lse_layout=sdpa.LSE_HEAD_MAJOR,
           stats_log2=True)


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5])
def test_scale_edges(scale):
    parity(inputs.fp8_thd_case(4005, 8, 2, 128, lengths=[1, 65, 190], scale=scale,
                               name="fp8_scale"))


# The gfx950 FP8 MFMAs do not return fp32-exact dot products: an in-bounds probe of
# v_mfma_scale_f32_32x32x64_f8f6f4 and v_mfma_f32_16x16x32_fp8_fp8 on known E4M3 codes
# measured errors up to 4.1e-5 of sum_d |q_d k_d| (the bf16 MFMA was exact on the same kind
# of probe).  A logit of scale * dq * dk * sum_d q_d k_d thus carries up to
# FP8_DOT_EPS * |scale * dq * dk| * sum_d |q_d k_d|, and the LSE (1-Lipschitz in the
# logits) at most the largest of those over the keys a row sees.
FP8_DOT_EPS = 2.0 ** -14


def fp8_lse_slack(case):
    """Per (token, head): FP8_DOT_EPS * |scale dq dk| * max over visible keys of
    sum_d |q_d||k_d| (THD, bottom-right causal or not)."""
    dq, dk, _ = case.descale
    qa = case.q.view(torch.float8_e4m3fn).float().abs()
    ka = case.k.view(torch.float8_e4m3fn).float().abs()
    g = case.hq // case.hkv
    out = np.zeros((int(case.cu_q[-1]), case.hq))
    for b in range(case.batch):
        q0, q1 = int(case.cu_q[b]), int(case.cu_q[b + 1])
        k0, k1 = int(case.cu_kv[b]), int(case.cu_kv[b + 1])
        lq, lk = q1 - q0, k1 - k0
        for h in range(case.hq):
            m = qa[q0:q1, h] @ ka[k0:k1, h // g].t()  # [lq, lk]
            if case.causal:
                i = torch.arange(lq)[:, None]
                j = torch.arange(lk)[None, :]
                m = torch.where(j <= i + lk - lq, m, torch.zeros_like(m))
            out[q0:q1, h] = m.max(dim=1).values.numpy() if lk else 0.0
    return FP8_DOT_EPS * abs(case.scale * dq * dk) * out


def test_large_logits_within_the_fp8_dot_product_bound():
    # scale 3: logits up to ~160, so the FP8 MFMA's dot-product error reaches a few 1e-3 in
    # the LSE.  O is held to the prefill bar; the LSE to 1e-3 plus the per-row bound above.
    case = inputs.fp8_thd_case(4005, 8, 2, 128, lengths=[1, 65, 190], scale=3.0,
                               name="fp8_large_logits")
    o, l = run(case)
    o_ref, l_ref = oracle_prefill(case, descale=case.descale)
    check_o(o, o_ref)
    g = l.cpu().numpy().astype(np.float64)
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(g), fin)
    slack = fp8_lse_slack(case)
    err = np.abs(g - l_ref)[fin]
    bound = (1e-3 + slack)[fin]
    log("fp8 large logits: max|dLSE| %.3g, max bound %.3g, max logit-scale LSE %.1f"
        % (err.max(), bound.max(), np.abs(l_ref[fin]).max()))
    assert np.all(err <= bound), (err.max(), bound[np.argmax(err - bound)])


def test_negative_descale_product():
    # Q codes with flipped signs and a negated descale_q stand for the same values
    case = inputs.fp8_thd_case(4006, 8, 2, 128, lengths=[70, 129], name="fp8_neg_descale")
    dq, dk, dv = case.descale
    flipped = dataclasses.replace(case, q=case.q ^ 0x80, descale=(-dq, dk, dv))
    o1, l1, _, _ = parity(case)
    o2, l2, _, _ = parity(flipped)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_full_size_fp8_prefill_sampled():
    base = inputs.thd_prefill_d128()
    case = inputs.fp8_thd_case(inputs.SEED_BASE + 2, 32, 8, 128, lengths=base.lengths_q,
                               name="fp8_" + base.name)
    log("full-size %s T=%d" % (case.name, int(case.cu_q[-1])))
    o, l = run(case)
    toks, heads = thd_sample(case, 384, 4007)
    o_ref, l_ref = oracle_prefill(case, sel_tok=toks, sel_head=heads, descale=case.descale)
    ti, hi = torch.from_numpy(toks).cuda(), torch.from_numpy(heads).long().cuda()
    e_o = check_o(o[ti, hi], o_ref)
    e_l = check_lse(l[ti, hi], l_ref)
    log("  max|dO|=%.3g max|dLSE|=%.3g" % (e_o, e_l))
    assert torch.isfinite(l).all()


def test_repeated_calls_are_bitwise_equal():
    # identical calls give identical bits, on the first launch as on later ones (the
    # scores' MFMAs must stay ahead of the softmax that reads them)
    case = inputs.fp8_thd_case(4007, 32, 8, 128, lengths=[3000, 2500, 70, 129, 640],
                               name="fp8_repeat")
    outs = [run(case) for _ in range(5)]
    log("fp8 repeat: %d calls on lengths %s" % (len(outs), case.lengths_q))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
