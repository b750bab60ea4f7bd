"""The library on caller streams and inside caller-captured HIP graphs: it allocates nothing,
never synchronises and records no memset, so a prefill or a decode call can be captured into
a graph by the caller (torch.cuda.CUDAGraph here) and replayed, and calls on two streams with
their own workspaces do not disturb each other. Every replay and every stream's result is
compared bit for bit with the eager call on the default stream."""
import pytest
import torch

import workloads as W

from _gpu import device_decode_inputs, device_prefill_inputs, say

pytestmark = pytest.mark.gpu


def _prefill(gqa, case, dev, out, ws):
    return gqa.prefill(dev["q"].view(1, case.N, case.H, case.d), dev["k"].view(1, case.N, case.G, case.d),
                       dev["v"].view(1, case.N, case.G, case.d), None, q_norm_w=dev["q_norm_w"],
                       k_norm_w=dev["k_norm_w"], eps=case.eps, theta=case.theta, out=out,
                       workspace=ws)


def test_prefill_captured_in_a_graph():
    import attention_head_qk_amd as gqa
    case = W.make_prefill("graph_prefill", 401, lengths=[1000], H=16, G=8)
    dev = device_prefill_inputs(case)
    ws = torch.empty(gqa.workspace_bytes("prefill", 1, case.N, case.H, case.G, case.d),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((1, case.N, case.H, case.d), dtype=torch.bfloat16, device="cuda")
    say("prefill captured in a HIP graph")
    eager = _prefill(gqa, case, dev, out, ws).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            _prefill(gqa, case, dev, out, ws)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
    # new inputs in the same buffers: the replay sees them
    dev["q"].mul_(-1.0)
    eager2 = _prefill(gqa, case, dev, torch.empty_like(out), torch.empty_like(ws)).clone()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, eager2) and not torch.equal(eager2, eager)


def test_decode_captured_in_a_graph():
    import attention_head_qk_amd as gqa
    case = W.make_decode("graph_decode", 402, B=6, max_seq=2048, H=32, G=8, d=128,
                         seq_lens=[1, 100, 700, 2048, 1500, 33])
    dev = device_decode_inputs(case)
    ws = torch.empty(gqa.workspace_bytes("decode", case.B, case.max_seq, case.H, case.G, case.d),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev["q"])
    kc0, vc0 = dev["k_cache"].clone(), dev["v_cache"].clone()

    def call():
        return gqa.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["seq_lens"],
                          k_new=dev["k_new"], v_new=dev["v_new"], q_norm_w=dev["q_norm_w"],
                          k_norm_w=dev["k_norm_w"], eps=case.eps, theta=case.theta, out=out,
                          workspace=ws)
    say("decode captured in a HIP graph")
    eager = call().clone()
    kc1 = dev["k_cache"].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    for i in range(3):
        dev["k_cache"].copy_(kc0)
        dev["v_cache"].copy_(vc0)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        assert torch.equal(dev["k_cache"], kc1), f"replay {i}: appended rows"


def test_two_streams_do_not_interfere():
    import attention_head_qk_amd as gqa
    cases = [W.make_prefill(f"stream_{i}", 410 + i, lengths=[1500], H=16, G=8) for i in range(2)]
    devs = [device_prefill_inputs(c) for c in cases]
    wss = [torch.empty(gqa.workspace_bytes("prefill", 1, c.N, c.H, c.G, c.d), dtype=torch.uint8,
                       device="cuda") for c in cases]
    say("prefill on two streams")
    eager = [_prefill(gqa, c, dv, torch.empty((1, c.N, c.H, c.d), dtype=torch.bfloat16,
                                              device="cuda"), w).clone()
             for c, dv, w in zip(cases, devs, wss)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(e) for e in eager]
    torch.cuda.synchronize()
    for rep in range(4):
        for c, dv, w, st, o in zip(cases, devs, wss, streams, outs):
            with torch.cuda.stream(st):
                _prefill(gqa, c, dv, o, w)
    torch.cuda.synchronize()
    for o, e in zip(outs, eager):
        assert torch.equal(o, e)


def test_stream_argument_allocates_on_that_stream():
    # prefill(..., stream=s) and decode(..., stream=s) with no workspace or out: the binding
    # allocates both on s, so memory the current stream grabs (and writes) right after the
    # call can never be the workspace or the output still in use by s's kernels
    import attention_head_qk_amd as gqa
    case = W.make_prefill("stream_arg", 420, lengths=[3000], H=16, G=8)
    dev = device_prefill_inputs(case)
    shp = lambda t, G: t.view(1, case.N, G, case.d)  # noqa: E731
    eager = gqa.prefill(shp(dev["q"], case.H), shp(dev["k"], case.G), shp(dev["v"], case.G),
                        None, q_norm_w=dev["q_norm_w"], k_norm_w=dev["k_norm_w"], eps=case.eps,
                        theta=case.theta).clone()
    dcase = W.make_decode("stream_arg_dec", 421, B=4, max_seq=4096, H=32, G=8, d=128,
                          seq_lens=[4096, 17, 2000, 1025])
    ddev = device_decode_inputs(dcase)
    dkw = dict(q_norm_w=ddev["q_norm_w"], k_norm_w=ddev["k_norm_w"], eps=dcase.eps,
               theta=dcase.theta)
    d_eager = gqa.decode(ddev["q"], ddev["k_cache"], ddev["v_cache"], ddev["seq_lens"],
                         **dkw).clone()
    torch.cuda.synchronize()
    say("prefill and decode with stream= and binding-allocated buffers")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        # keep s busy first, so its prefill is still running when the current stream moves on
        with torch.cuda.stream(s):
            torch.cuda._sleep(2_000_000)
        out = gqa.prefill(shp(dev["q"], case.H), shp(dev["k"], case.G), shp(dev["v"], case.G),
                          None, q_norm_w=dev["q_norm_w"], k_norm_w=dev["k_norm_w"],
                          eps=case.eps, theta=case.theta, stream=s)
        d_out = gqa.decode(ddev["q"], ddev["k_cache"], ddev["v_cache"], ddev["seq_lens"],
                           stream=s, **dkw)
        junk = [torch.full((int(n),), 7.0, dtype=torch.bfloat16, device="cuda")
                for n in (case.N * case.H * case.d, case.N * case.G * case.d,
                          dcase.B * dcase.H * dcase.d, 1 << 22)]
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"prefill, repetition {rep}"
        assert torch.equal(d_out, d_eager), f"decode, repetition {rep}"
        del junk
