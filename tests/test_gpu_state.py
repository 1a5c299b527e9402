"""GPU checks of the library's device-side state (work-queue counters): captured launches
replayed on changed inputs, and many calls in flight at once on several streams.

The persistent prefill and decode grids draw their work items from counters in a static
device array; every launch tags the counters it uses and the last work-group of a launch
returns them to zero.  A replayed captured launch (same arguments, same tag) must find its
counters free again, and calls overlapping on different streams must not share counters.
"""
import pytest
import torch

from scaled_dot_product_19_amd import inputs, sdpa
from tests.helpers import path_of, check_lse, check_o, log, oracle_decode, oracle_prefill, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sdpa.load()


def test_captured_prefill_and_decode_replayed_on_new_inputs():
    # one prefill (padded LSE: the -inf fill kernel is captured too), one split decode
    # (split kernel + combine) and one multi-token decode on the paged prefill kernel
    # (folded rows, its persistent work queue) captured once, replayed on three different
    # inputs, with eager work between the replays
    pre = [inputs.thd_case(4100 + r, hq=8, hkv=2, d_qk=128, lengths=[100, 37, 260],
                           name="graph_prefill") for r in range(3)]
    dec = [inputs.paged_case(4200 + r, 3, 1, 32, 8, 128, 128, 64, lengths=[90, 700, 1500],
                             num_splits=4, poison=True, name="graph_decode") for r in range(3)]
    fol = [inputs.paged_case(4300 + r, 2, 4, 32, 1, 128, 128, 64, lengths=[3, 900],
                             num_splits=2, poison=True, name="graph_folded") for r in range(3)]
    assert path_of(fol[0]) == "prefill_folded"
    # the captured launches read these buffers; each replay copies new inputs into them
    q, k, v = to_dev(pre[0].q), to_dev(pre[0].k), to_dev(pre[0].v)
    cu = to_dev(pre[0].cu_q)
    s_max = 260
    o_p = torch.empty((q.shape[0], 8, 128), dtype=torch.bfloat16, device="cuda")
    l_p = torch.empty((3, s_max, 8), dtype=torch.float32, device="cuda")
    dq, kp, vp = to_dev(dec[0].q), to_dev(dec[0].k_pool), to_dev(dec[0].v_pool)
    ptk, ptv, sl = to_dev(dec[0].pt_k), to_dev(dec[0].pt_v), to_dev(dec[0].seq_lens)
    o_d = torch.empty((3, 1, 32, 128), dtype=torch.bfloat16, device="cuda")
    l_d = torch.empty((3, 1, 32), dtype=torch.float32, device="cuda")
    ws = torch.empty(sdpa.decode_workspace_bytes(3, 1, 32, 128, 4), dtype=torch.uint8,
                     device="cuda")
    fq, fkp, fvp = to_dev(fol[0].q), to_dev(fol[0].k_pool), to_dev(fol[0].v_pool)
    fptk, fptv, fsl = to_dev(fol[0].pt_k), to_dev(fol[0].pt_v), to_dev(fol[0].seq_lens)
    o_f = torch.empty((2, 4, 32, 128), dtype=torch.bfloat16, device="cuda")
    l_f = torch.empty((2, 4, 32), dtype=torch.float32, device="cuda")
    ws_f = torch.empty(sdpa.decode_workspace_bytes(2, 4, 32, 128, 2), dtype=torch.uint8,
                       device="cuda")

    def calls():
        sdpa.prefill_thd(q, k, v, cu, cu, 260, 260, pre[0].scale, True, out=o_p, lse=l_p,
                         lse_layout=sdpa.LSE_PADDED, lse_s_max=s_max)
        sdpa.decode_paged(dq, kp, vp, ptk, ptv, sl, 1500, dec[0].scale, True, num_splits=4,
                          workspace=ws, out=o_d, lse=l_d)
        sdpa.decode_paged(fq, fkp, fvp, fptk, fptv, fsl, 900, fol[0].scale, True, num_splits=2,
                          workspace=ws_f, out=o_f, lse=l_f)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()  # eager warm-up (per-kernel attributes, occupancy) before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side, capture_error_mode="thread_local"):
        calls()
    torch.cuda.synchronize()
    for r in range(3):
        log("graph replay %d" % r)
        q.copy_(to_dev(pre[r].q))
        k.copy_(to_dev(pre[r].k))
        v.copy_(to_dev(pre[r].v))
        dq.copy_(to_dev(dec[r].q))
        kp.copy_(to_dev(dec[r].k_pool))
        vp.copy_(to_dev(dec[r].v_pool))
        ptk.copy_(to_dev(dec[r].pt_k))
        ptv.copy_(to_dev(dec[r].pt_v))
        fq.copy_(to_dev(fol[r].q))
        fkp.copy_(to_dev(fol[r].k_pool))
        fvp.copy_(to_dev(fol[r].v_pool))
        fptk.copy_(to_dev(fol[r].pt_k))
        fptv.copy_(to_dev(fol[r].pt_v))
        o_f.fill_(5.0)
        l_f.fill_(5.0)
        o_p.fill_(5.0)
        l_p.fill_(5.0)
        o_d.fill_(5.0)
        l_d.fill_(5.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o_p, l_p, o_d, l_d, o_f, l_f)]
        calls()  # the same calls eagerly, on the same inputs
        torch.cuda.synchronize()
        for g, e in zip(got, (o_p, l_p, o_d, l_d, o_f, l_f)):
            assert torch.equal(g, e), "replay %d differs from the eager call" % r
        o_ref, l_ref = oracle_prefill(pre[r])
        check_o(got[0], o_ref)
        for b, L in enumerate(pre[r].lengths_q):
            t0 = int(pre[r].cu_q[b])
            check_lse(got[1][b, :L], l_ref[t0:t0 + L])
            assert torch.all(got[1][b, L:] == -float("inf"))
        od_ref, ld_ref = oracle_decode(dec[r])
        check_o(got[2], od_ref)
        check_lse(got[3], ld_ref)
        of_ref, lf_ref = oracle_decode(fol[r])
        check_o(got[4], of_ref)
        check_lse(got[5], lf_ref)


def test_many_calls_in_flight_on_four_streams():
    # 16 input sets x 5 rounds of prefill and decode calls = 80 + 80 launches spread over
    # four streams of the default priority; every output is checked
    n_sets, rounds = 16, 5
    g = torch.Generator().manual_seed(4300)
    pre, dec = [], []
    for i in range(n_sets):
        lens = torch.randint(1, 300, (3,), generator=g).tolist()
        pre.append(inputs.thd_case(4300 + i, hq=8, hkv=2, d_qk=128, lengths=lens,
                                   name="overlap_prefill"))
        dlens = torch.randint(1, 2000, (3,), generator=g).tolist()
        dec.append(inputs.paged_case(4400 + i, 3, 1, 32, 8, 128, 128, 64, lengths=dlens,
                                     num_splits=4, poison=True, name="overlap_decode"))
    dev_pre = [(to_dev(c.q), to_dev(c.k), to_dev(c.v), to_dev(c.cu_q)) for c in pre]
    dev_dec = [tuple(to_dev(t) for t in (c.q, c.k_pool, c.v_pool, c.pt_k, c.pt_v, c.seq_lens))
               for c in dec]
    out_pre, out_dec = [], []
    for r in range(rounds):
        for i in range(n_sets):
            c, d = pre[i], dec[i]
            T = int(c.cu_q[-1])
            out_pre.append((i, torch.empty((T, 8, 128), dtype=torch.bfloat16, device="cuda"),
                            torch.empty((T, 8), dtype=torch.float32, device="cuda")))
            out_dec.append((i, torch.empty((3, 1, 32, 128), dtype=torch.bfloat16, device="cuda"),
                            torch.empty((3, 1, 32), dtype=torch.float32, device="cuda"),
                            torch.empty(sdpa.decode_workspace_bytes(3, 1, 32, 128, 4),
                                        dtype=torch.uint8, device="cuda")))
    streams = [torch.cuda.Stream() for _ in range(4)]
    torch.cuda.synchronize()
    for n, ((i, o, l), (j, od, ld, ws)) in enumerate(zip(out_pre, out_dec)):
        s = streams[n % 4]
        q, k, v, cu = dev_pre[i]
        sdpa.prefill_thd(q, k, v, cu, cu, pre[i].max_q, pre[i].max_kv, pre[i].scale, True,
                         out=o, lse=l, stream=s)
        dq, kp, vp, ptk, ptv, sl = dev_dec[j]
        sdpa.decode_paged(dq, kp, vp, ptk, ptv, sl, dec[j].max_kv, dec[j].scale, True,
                          num_splits=4, workspace=ws, out=od, lse=ld, stream=s)
    torch.cuda.synchronize()
    log("80 prefill + 80 decode calls done on 4 streams")
    first_pre, first_dec = {}, {}
    for (i, o, l), (j, od, ld, _) in zip(out_pre, out_dec):
        if i not in first_pre:
            first_pre[i] = (o, l)
            first_dec[j] = (od, ld)
            o_ref, l_ref = oracle_prefill(pre[i])
            check_o(o, o_ref)
            check_lse(l, l_ref)
            od_ref, ld_ref = oracle_decode(dec[j])
            check_o(od, od_ref)
            check_lse(ld, ld_ref)
        else:
            assert torch.equal(o, first_pre[i][0]) and torch.equal(l, first_pre[i][1])
            assert torch.equal(od, first_dec[j][0]) and torch.equal(ld, first_dec[j][1])
