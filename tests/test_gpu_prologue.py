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
