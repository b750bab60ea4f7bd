"""GPU parity of the RoPE frequency-table hook (gqa_params.rope_inv_freq) against the fp64
oracle: linear position interpolation, the architecture article's YaRN-named formula and the
NTK base change, through the prefill (bf16 and fp32), cached prefill, decode and the
stand-alone prologue; a table equal to the base frequencies reproduces the theta path bit
for bit."""
import numpy as np
import pytest
import torch

import workloads as W

from _gpu import (check, device_cached_inputs, device_decode_inputs, device_prefill_inputs,
                  oracle_decode_seq, run_decode, run_prefill, run_prefill_cached, say, to_f64)

pytestmark = pytest.mark.gpu


def _tables(d):
    """The library's tables (gqa_rope_freq_table): what the GPU side is given."""
    import attention_head_qk_amd as gqa
    return {"linear": gqa.rope_freq_table(d, 1e6, "linear", alpha=4.0),
            "yarn": gqa.rope_freq_table(d, 1e6, "yarn", train_len=32768, infer_len=131072),
            "ntk": gqa.rope_freq_table(d, 1e6, "ntk", alpha=8.0)}


def _oracle_tables(d):
    """The same rules from the oracle's own functions: what the oracle side is given."""
    from oracle import gqa_oracle as O
    return {"linear": O.inv_freq_linear(d, 1e6, 4.0),
            "yarn": O.inv_freq_yarn_page(d, 1e6, 32768, 131072),
            "ntk": O.rope_inv_freq(d, O.ntk_theta(1e6, 8.0, d))}


def _with_theta(case, table):
    """The same case with the oracle's theta replaced by the frequency table."""
    import copy
    c = copy.copy(case)
    c.theta = table
    return c


@pytest.mark.parametrize("kind", ["linear", "yarn", "ntk"])
@pytest.mark.parametrize("dtype,d", [(W.BF16, 128), (W.BF16, 64), (W.F32, 128)])
def test_prefill_with_table(kind, dtype, d):
    from _gpu import oracle_prefill
    # positions far apart, where the scaled frequencies differ most from the base ones
    lengths = [70, 0, 150]
    pos = np.concatenate([np.arange(70) * 97 + 5000, np.arange(150) * 211]).astype(np.int32)
    case = W.make_prefill(f"rope_{kind}", 200 + d, lengths=lengths, H=16, G=4, d=d, dtype=dtype,
                          positions=pos)
    say("prefill rope table", kind, dtype, d)
    got = to_f64(run_prefill(case, rope_inv_freq=_tables(d)[kind]))
    check(got, oracle_prefill(_with_theta(case, _oracle_tables(d)[kind])), dtype,
          f"{kind} {dtype} d={d}")


def test_base_table_is_the_theta_path():
    import attention_head_qk_amd as gqa
    case = W.make_prefill("rope_base", 210, lengths=[300], H=16, G=8)
    dev = device_prefill_inputs(case)
    say("prefill base table vs theta")
    a = run_prefill(case, dev=dev)
    b = run_prefill(case, dev=dev, rope_inv_freq=gqa.rope_freq_table(128, case.theta))
    assert torch.equal(a, b)


def test_decode_and_cached_prefill_with_table():
    from oracle import gqa_oracle as O
    table = _tables(128)["yarn"]
    otable = _oracle_tables(128)["yarn"]
    # decode
    dcase = W.make_decode("rope_dec", 220, B=4, max_seq=3000, H=32, G=8, d=128,
                          seq_lens=[1, 700, 2999, 64])
    dev = device_decode_inputs(dcase)
    say("decode rope table")
    out = to_f64(run_decode(dcase, dev, rope_inv_freq=table))
    dcase_t = _with_theta(dcase, otable)
    for b in range(dcase.B):
        want, k_slot, _ = oracle_decode_seq(dcase_t, b)
        check(out[b], want, W.BF16, f"decode b={b}")
        L = int(dcase.seq_lens[b])
        got_k = to_f64(dev["k_cache"][b, L - 1])
        assert np.all(np.abs(got_k - k_slot) <= 2.0 ** -8 * np.abs(k_slot) + 1e-6)
    # cached prefill
    ccase = W.make_cached_prefill("rope_cached", 221, [90, 33], [400, 17], 512, H=16, G=8)
    cdev = device_cached_inputs(ccase)
    say("cached prefill rope table")
    got = to_f64(run_prefill_cached(ccase, cdev, rope_inv_freq=table))
    from _gpu import oracle_prefill_cached_seq
    ct = _with_theta(ccase, otable)
    for b in range(ccase.B):
        s, e = int(ccase.cu_seqlens[b]), int(ccase.cu_seqlens[b + 1])
        want, kc, _ = oracle_prefill_cached_seq(ct, b)
        check(got[s:e], want, W.BF16, f"cached b={b}")
        past = int(ccase.cache_lens[b])
        gk = to_f64(cdev["k_cache"][b, past:past + e - s])
        assert np.all(np.abs(gk - kc[past:]) <= 2.0 ** -8 * np.abs(kc[past:]) + 1e-6)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_prologue_with_table(dtype):
    import attention_head_qk_amd as gqa
    from oracle import gqa_oracle as O
    from _gpu import to_dev, i32
    table = _tables(128)["linear"]
    otable = _oracle_tables(128)["linear"]
    case = W.make_prefill("rope_pro", 230, lengths=[257], H=8, G=2, d=128, dtype=dtype,
                          positions=(np.arange(257) * 31).astype(np.int32))
    say("prologue rope table", dtype)
    qo, ko = gqa.qk_norm_rope(to_dev(case.q, dtype), to_dev(case.k, dtype), i32(case.positions),
                              q_norm_w=to_dev(case.q_norm_w, dtype),
                              k_norm_w=to_dev(case.k_norm_w, dtype), rope_inv_freq=table)
    qt, kt = O.qk_norm_rope(case.f64("q"), case.f64("k"), case.positions, case.f64("q_norm_w"),
                            case.f64("k_norm_w"), case.eps, otable)
    tol = 2.0 ** -8 if dtype == W.BF16 else 1e-6
    for got, want in ((to_f64(qo), qt), (to_f64(ko), kt)):
        assert np.all(np.abs(got - want) <= tol * np.abs(want) + 1e-6)
