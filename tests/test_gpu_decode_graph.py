"""GPU parity of the decode graph (gqa_decode_graph_*: one generation step captured as a HIP
graph, replayed per token) against eager gqa_decode calls, bit for bit, and against the fp64
oracle of successive decode steps. Every replay is checked, with the program's own eager work
and synchronisations between replays as well as back-to-back."""
import numpy as np
import pytest
import torch

import workloads as W

from _gpu import check, device_steps_inputs, oracle_decode_steps, say, to_f64

pytestmark = pytest.mark.gpu


def _eager_steps(case, dev):
    """The same S steps by gqa_decode: seq_lens advanced by a torch op before each call."""
    import attention_head_qk_amd as gqa
    kc, vc = dev["k_cache"].clone(), dev["v_cache"].clone()
    sl = dev["seq_lens"].clone()
    outs = []
    for s in range(case.S):
        sl.add_(1).clamp_(max=case.max_seq)
        outs.append(gqa.decode(dev["q"][s], kc, vc, sl, k_new=dev["k"][s], v_new=dev["v"][s],
                               q_norm_w=dev["q_norm_w"], k_norm_w=dev["k_norm_w"],
                               eps=case.eps, theta=case.theta))
    return torch.stack(outs), kc, vc, sl


def _graph(case, dev, kc, vc, sl):
    import attention_head_qk_amd as gqa
    B, H, G, d = case.B, case.H, case.G, case.d
    tdt = dev["q"].dtype
    bufs = dict(q=torch.empty((B, H, d), dtype=tdt, device="cuda"),
                k=torch.empty((B, G, d), dtype=tdt, device="cuda"),
                v=torch.empty((B, G, d), dtype=tdt, device="cuda"))
    g = gqa.DecodeGraph(bufs["q"], kc, vc, sl, bufs["k"], bufs["v"], q_norm_w=dev["q_norm_w"],
                        k_norm_w=dev["k_norm_w"], eps=case.eps, theta=case.theta)
    return g, bufs


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_graph_steps_equal_eager_and_oracle(dtype):
    # starting lengths around the 1024-key split edges, an empty sequence and a short one
    case = W.make_decode_steps("graph_steps", 110, [0, 1, 1023, 1024, 2000, 37], 6, 2100,
                               H=32, G=8, d=128, dtype=dtype)
    dev = device_steps_inputs(case)
    say("decode graph vs eager vs oracle", dtype)
    want_out, want_kc, want_vc, want_sl = _eager_steps(case, dev)
    torch.cuda.synchronize()
    kc, vc, sl = dev["k_cache"].clone(), dev["v_cache"].clone(), dev["seq_lens"].clone()
    g, bufs = _graph(case, dev, kc, vc, sl)
    with g:
        for s in range(case.S):
            # the program's own eager work between replays, then a synchronisation
            bufs["q"].copy_(dev["q"][s])
            bufs["k"].copy_(dev["k"][s])
            bufs["v"].copy_(dev["v"][s])
            out = g.launch().clone()
            torch.cuda.synchronize()
            assert torch.equal(out, want_out[s]), f"replay {s}"
            assert torch.equal(sl, dev["seq_lens"] + s + 1)
    assert torch.equal(kc, want_kc) and torch.equal(vc, want_vc) and torch.equal(sl, want_sl)
    o_out, o_kc, o_vc = oracle_decode_steps(case)
    got = to_f64(want_out)
    for s in range(case.S):
        check(got[s], o_out[s], dtype, f"step {s}")
    for b in range(case.B):
        L = int(case.cache_lens[b]) + case.S
        new_k = to_f64(kc[b, L - case.S:L])
        ref = o_kc[b, L - case.S:L]
        tol = 2.0 ** -8 if dtype == W.BF16 else 1e-6
        assert np.all(np.abs(new_k - ref) <= tol * np.abs(ref) + 1e-6)
        assert np.array_equal(to_f64(vc[b, :L]), o_vc[b, :L])


def test_graph_back_to_back_replays():
    # 24 launches with no host synchronisation: inputs refilled and outputs saved in stream
    # order, as a generation loop runs
    case = W.make_decode_steps("graph_b2b", 111, [300, 5, 1500, 64, 999, 2047, 1, 700], 24,
                               2100, H=16, G=4, d=128)
    dev = device_steps_inputs(case)
    say("decode graph back-to-back replays")
    want_out, want_kc, want_vc, want_sl = _eager_steps(case, dev)
    kc, vc, sl = dev["k_cache"].clone(), dev["v_cache"].clone(), dev["seq_lens"].clone()
    g, bufs = _graph(case, dev, kc, vc, sl)
    outs = torch.empty_like(want_out)
    for s in range(case.S):
        bufs["q"].copy_(dev["q"][s])
        bufs["k"].copy_(dev["k"][s])
        bufs["v"].copy_(dev["v"][s])
        outs[s].copy_(g.launch())
    g.close()
    assert torch.equal(outs, want_out)
    assert torch.equal(kc, want_kc) and torch.equal(vc, want_vc) and torch.equal(sl, want_sl)


def test_graph_d64_mqa_and_positions():
    import attention_head_qk_amd as gqa
    case = W.make_decode_steps("graph_d64", 112, [10, 0, 513], 4, 600, H=8, G=1, d=64)
    dev = device_steps_inputs(case)
    say("decode graph d=64 MQA, explicit positions")
    pos = torch.tensor([100000, 7, 3], dtype=torch.int32, device="cuda")
    kc, vc, sl = dev["k_cache"].clone(), dev["v_cache"].clone(), dev["seq_lens"].clone()
    q = torch.empty_like(dev["q"][0])
    k = torch.empty_like(dev["k"][0])
    v = torch.empty_like(dev["v"][0])
    g = gqa.DecodeGraph(q, kc, vc, sl, k, v, positions=pos, q_norm_w=dev["q_norm_w"],
                        k_norm_w=dev["k_norm_w"])
    kc_e, vc_e, sl_e = dev["k_cache"].clone(), dev["v_cache"].clone(), dev["seq_lens"].clone()
    for s in range(case.S):
        q.copy_(dev["q"][s])
        k.copy_(dev["k"][s])
        v.copy_(dev["v"][s])
        pos.add_(1)
        out = g.launch().clone()
        sl_e.add_(1)
        want = gqa.decode(dev["q"][s], kc_e, vc_e, sl_e, k_new=dev["k"][s], v_new=dev["v"][s],
                          positions=pos, q_norm_w=dev["q_norm_w"], k_norm_w=dev["k_norm_w"])
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"step {s}"
    g.close()
    assert torch.equal(kc, kc_e) and torch.equal(vc, vc_e)


def test_graph_full_cache_stays_at_max_seq():
    case = W.make_decode_steps("graph_full", 113, [62, 10], 2, 64, H=8, G=4, d=128)
    dev = device_steps_inputs(case)
    say("decode graph at max_seq")
    kc, vc, sl = dev["k_cache"].clone(), dev["v_cache"].clone(), dev["seq_lens"].clone()
    g, bufs = _graph(case, dev, kc, vc, sl)
    for s in range(3):  # the third step finds sequence 0 full
        src = min(s, case.S - 1)
        bufs["q"].copy_(dev["q"][src])
        bufs["k"].copy_(dev["k"][src])
        bufs["v"].copy_(dev["v"][src])
        g.launch()
    g.close()
    assert sl.tolist() == [64, 13]
    assert not torch.isnan(kc.float()).any()


@pytest.mark.parametrize("per,dtype,d", [(4, W.BF16, 128), (6, W.BF16, 128), (3, W.F32, 64),
                                         (2, W.BF16, 64)])
def test_multi_step_graph_equals_eager(per, dtype, d):
    # gqa_decode_graph_create_steps: `per` steps per launch over [per, B, ...] blocks; two
    # launches (the second with new inputs written between them) equal 2 * per eager steps bit
    # for bit, caches and lengths included
    import attention_head_qk_amd as gqa
    S = 2 * per
    case = W.make_decode_steps(f"graph_multi{per}_{dtype}_{d}", 113 + per, [0, 900, 1023, 2080, 5],
                               S, 2096, H=32, G=8, d=d, dtype=dtype)
    dev = device_steps_inputs(case)
    say("multi-step decode graph", per)
    want_out, want_kc, want_vc, want_sl = _eager_steps(case, dev)
    kc, vc, sl = dev["k_cache"].clone(), dev["v_cache"].clone(), dev["seq_lens"].clone()
    q = torch.empty((per,) + tuple(dev["q"].shape[1:]), dtype=dev["q"].dtype, device="cuda")
    k = torch.empty((per,) + tuple(dev["k"].shape[1:]), dtype=dev["k"].dtype, device="cuda")
    v = torch.empty_like(k)
    g = gqa.DecodeGraph(q, kc, vc, sl, k, v, q_norm_w=dev["q_norm_w"], k_norm_w=dev["k_norm_w"],
                        eps=case.eps, theta=case.theta, steps=per)
    with g:
        for rep in range(2):
            blk = slice(rep * per, (rep + 1) * per)
            q.copy_(dev["q"][blk])
            k.copy_(dev["k"][blk])
            v.copy_(dev["v"][blk])
            out = g.launch().clone()
            torch.cuda.synchronize()
            assert torch.equal(out, want_out[blk]), f"launch {rep}"
            assert torch.equal(sl, dev["seq_lens"] + (rep + 1) * per)
    assert torch.equal(kc, want_kc) and torch.equal(vc, want_vc) and torch.equal(sl, want_sl)
    o_out, _, _ = oracle_decode_steps(case)
    got = to_f64(want_out)
    for s in range(S):
        check(got[s], o_out[s], dtype, f"step {s}")


def test_multi_step_graph_rejects_bad_shapes():
    import attention_head_qk_amd as gqa
    B, H, G, d, S = 2, 8, 2, 128, 64
    kc = torch.zeros((B, S, G, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    sl = torch.zeros(B, dtype=torch.int32, device="cuda")
    q = torch.zeros((3, B, H, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((3, B, G, d), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    with pytest.raises(ValueError):
        gqa.DecodeGraph(q, kc, vc, sl, k, v, steps=0)
    with pytest.raises(ValueError):
        gqa.DecodeGraph(q, kc, vc, sl, k, v, steps=4)   # q holds 3 steps
    with pytest.raises(ValueError):
        gqa.DecodeGraph(q, kc, vc, sl, k[:2], v[:2], steps=3)
    with pytest.raises(ValueError):
        gqa.DecodeGraph(q, kc, vc, sl, k, v, steps=3,
                        positions=torch.zeros((3, B + 1), dtype=torch.int32, device="cuda"))
    g = gqa.DecodeGraph(q, kc, vc, sl, k, v, steps=3)  # B empty caches: three appends each
    out = g.launch()
    g.close()
    assert out.shape == (3, B, H, d)
    assert torch.equal(sl, torch.full((B,), 3, dtype=torch.int32, device="cuda"))
