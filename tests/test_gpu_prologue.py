"""Step-level parity of the QK prologue (RMSNorm then RoPE) on the GPU against the oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import gqa_oracle as O

from _gpu import i32, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _case(seed, N, H, G, d, dtype, pos_hi=32768):
    rng = np.random.default_rng(seed)
    q = W.encode(rng.standard_normal((N, H, d), dtype=np.float32) * 2, dtype)
    k = W.encode(rng.standard_normal((N, G, d), dtype=np.float32) * 0.5, dtype)
    gq = W.encode(rng.uniform(0.5, 1.5, d).astype(np.float32), dtype)
    gk = W.encode(rng.uniform(0.5, 1.5, d).astype(np.float32), dtype)
    pos = rng.integers(0, pos_hi, N).astype(np.int32)
    pos[:3] = [0, 1, pos_hi - 1]
    return q, k, gq, gk, pos


def _cmp(got, want, dtype, what):
    err = np.abs(got - want)
    if dtype == W.F32:
        assert err.max() <= 1e-5, (what, err.max())
    else:
        # one bf16 rounding of a value computed in fp32: within 1 ulp (2^-8 relative)
        assert np.all(err <= 2.0 ** -8 * np.abs(want) + 1e-6), (what, err.max())


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,G", [(16, 8), (64, 4), (5, 5)])
def test_prologue_matches_oracle(dtype, d, H, G):
    import attention_head_qk_amd as gqa
    q, k, gq, gk, pos = _case(7 + d + H, 67, H, G, d, dtype)
    say(f"prologue dtype={dtype} d={d} H={H} G={G}")
    qo, ko = gqa.qk_norm_rope(to_dev(q, dtype), to_dev(k, dtype), i32(pos),
                              q_norm_w=to_dev(gq, dtype), k_norm_w=to_dev(gk, dtype),
                              eps=1e-6, theta=1e6)
    wq, wk = O.qk_norm_rope(W.to_f64(q, dtype), W.to_f64(k, dtype), pos, W.to_f64(gq, dtype),
                            W.to_f64(gk, dtype), 1e-6, 1e6)
    _cmp(to_f64(qo), wq, dtype, "q")
    _cmp(to_f64(ko), wk, dtype, "k")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_prologue_without_norm_or_rope(dtype):
    import attention_head_qk_amd as gqa
    q, k, gq, gk, pos = _case(3, 33, 8, 2, 128, dtype)
    say(f"prologue switches dtype={dtype}")
    # no RoPE (theta = 0): RMSNorm only
    qo, ko = gqa.qk_norm_rope(to_dev(q, dtype), to_dev(k, dtype), i32(pos),
                              q_norm_w=to_dev(gq, dtype), k_norm_w=to_dev(gk, dtype), theta=0.0)
    _cmp(to_f64(qo), O.rms_norm(W.to_f64(q, dtype), W.to_f64(gq, dtype), 1e-6), dtype, "q")
    _cmp(to_f64(ko), O.rms_norm(W.to_f64(k, dtype), W.to_f64(gk, dtype), 1e-6), dtype, "k")
    # no norm weights: RoPE only; positions None -> 0..N-1
    qo, ko = gqa.qk_norm_rope(to_dev(q, dtype), to_dev(k, dtype), None, theta=1e6)
    ar = np.arange(33)
    _cmp(to_f64(qo), O.rope(W.to_f64(q, dtype), ar, 1e6), dtype, "q")
    _cmp(to_f64(ko), O.rope(W.to_f64(k, dtype), ar, 1e6), dtype, "k")


def test_prologue_in_several_launches():
    # more than 2^22 (token, head) rows: the launcher splits the pass into launches of whole
    # token slots; rows on both sides of each launch boundary are checked against the oracle
    import torch
    import attention_head_qk_amd as gqa
    N, H, G, d = 480_000, 16, 2, 128   # 8.6M rows: two launches of 233,016 tokens and a rest
    g = torch.Generator(device="cuda").manual_seed(501)
    q = torch.randn((N, H, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((N, G, d), generator=g, device="cuda").to(torch.bfloat16)
    gq = (torch.rand((d,), generator=g, device="cuda") + 0.5).to(torch.bfloat16)
    gk = (torch.rand((d,), generator=g, device="cuda") + 0.5).to(torch.bfloat16)
    say("prologue over 8.6M rows in three launches")
    qo, ko = gqa.qk_norm_rope(q, k, None, q_norm_w=gq, k_norm_w=gk)
    torch.cuda.synchronize()
    per = (1 << 22) // (H + G)
    toks = sorted({0, 1, per - 1, per, per + 1, 2 * per - 1, 2 * per, N - 1, 12345, 250_001})
    assert 2 * per < N and all(0 <= t < N for t in toks)  # every sampled token exists
    idx = torch.tensor(toks, device="cuda")

    def host(t):
        return t.index_select(0, idx).float().cpu().numpy().astype(np.float64)
    qt, kt = O.qk_norm_rope(host(q), host(k), np.array(toks, np.int32),
                            gq.float().cpu().numpy().astype(np.float64),
                            gk.float().cpu().numpy().astype(np.float64), 1e-6, 1e6)
    for got, want in ((host(qo), qt), (host(ko), kt)):
        assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-6)
