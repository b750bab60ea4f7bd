"""GPU parity of gqa_decode (prologue + KV append + split-KV pass + combine) against the
fp64 oracle, on the 64-sequence workload and on edge cases of the split partition."""
import numpy as np
import pytest
import torch

import workloads as W

from _gpu import (check, device_decode_inputs, i32, oracle_decode_seq, run_decode, say,
                  to_f64)

pytestmark = pytest.mark.gpu


def test_decode_64_sequences_sampled():
    case = W.decode_64()
    say("decode 64 seqs, cache", case.max_seq, "lens", int(case.seq_lens.min()), int(case.seq_lens.max()))
    dev = device_decode_inputs(case)
    out = to_f64(run_decode(case, dev))
    order = np.argsort(case.seq_lens)
    picks = sorted({int(order[0]), int(order[1]), int(order[-1]), int(order[-2]), 0, 17, 40, 63})
    for b in picks:
        want, k_slot, v_slot = oracle_decode_seq(case, b)
        check(out[b], want, W.BF16, f"seq {b} L={case.seq_lens[b]}")
        L = int(case.seq_lens[b])
        got_k = to_f64(dev["k_cache"][b, L - 1])
        assert np.all(np.abs(got_k - k_slot) <= 2.0 ** -8 * np.abs(k_slot) + 1e-6)
        assert np.array_equal(to_f64(dev["v_cache"][b, L - 1]), v_slot)


def edge_lens(S):
    """Lengths around a split-KV partition of S keys: empty, tiny, both sides of one and two
    splits, a quarter split (one wave's share), and a ragged multi-split length."""
    return [0, 1, 2, 31, 33, S // 4 - 1, S // 4 + 1, S - 1, S, S + 1, 2 * S, 2 * S + 37, 3 * S - 5]


@pytest.mark.parametrize("max_seq", [3100, 24576])
@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("H,G,d", [(32, 8, 128), (12, 4, 128), (8, 8, 64), (16, 1, 128),
                                   (6, 2, 64), (40, 1, 128)])
def test_decode_edge_lengths(dtype, H, G, d, max_seq):
    # the split length follows the shape (1024, 512 and 256 all occur over these cases); the
    # lengths sit on that split's edges. At max_seq 24576 the bf16 caches of the G = 8 and
    # G = 4 shapes exceed 512 MiB, so those cases take the pass that streams V non-temporally.
    import attention_head_qk_amd as gqa
    B = 13
    S = gqa.decode_split_keys(B, H, G, max_seq)
    lens = edge_lens(S)
    assert len(lens) == B and max(lens) <= max_seq
    case = W.make_decode("edge", 61 + H + G + d, B=B, max_seq=max_seq, H=H, G=G, d=d,
                         dtype=dtype, seq_lens=lens)
    say("decode edges", dtype, H, G, d, "max_seq", max_seq, "split", S)
    dev = device_decode_inputs(case, fill_invalid=float("nan"))
    out = to_f64(run_decode(case, dev))
    for b, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(out[b], np.zeros((H, d))), "empty sequence must give zeros"
            continue
        want, _, _ = oracle_decode_seq(case, b)
        check(out[b], want, dtype, f"L={L}")


def test_decode_without_append_and_explicit_positions():
    case = W.make_decode("noappend", 71, B=5, max_seq=2048, H=16, G=4, d=128,
                         seq_lens=[700, 1, 2048, 513, 64])
    dev = device_decode_inputs(case)
    say("decode no append / explicit positions")
    before = dev["k_cache"].clone()
    out = to_f64(run_decode(case, dev, append=False))
    assert torch.equal(before, dev["k_cache"]), "no append: the cache must stay untouched"
    for b in range(case.B):
        want, _, _ = oracle_decode_seq(case, b, append=False)
        check(out[b], want, W.BF16, f"b={b}")
    pos = np.array([5, 0, 100000, 3, 63], dtype=np.int32)
    out = to_f64(run_decode(case, dev, append=True, positions=i32(pos)))
    for b in range(case.B):
        want, _, _ = oracle_decode_seq(case, b, position=int(pos[b]))
        check(out[b], want, W.BF16, f"b={b} pos={pos[b]}")


def test_decode_equals_last_prefill_row():
    import attention_head_qk_amd as gqa
    from _gpu import device_prefill_inputs
    L, H, G, d = 1300, 32, 8, 128
    pcase = W.make_prefill("dp", 81, lengths=[L], H=H, G=G, d=d)
    dev = device_prefill_inputs(pcase)
    say("decode vs prefill last row")
    k_out = torch.empty_like(dev["k"])
    full = run_prefill_helper(pcase, dev, k_out)
    kc = torch.zeros((1, 2048, G, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kc[0, :L - 1] = k_out[:L - 1]
    vc[0, :L - 1] = dev["v"][:L - 1]
    out = gqa.decode(dev["q"][L - 1:L], kc, vc, i32([L]), k_new=dev["k"][L - 1:L],
                     v_new=dev["v"][L - 1:L], q_norm_w=dev["q_norm_w"], k_norm_w=dev["k_norm_w"])
    diff = (out[0].float() - full[L - 1].float()).abs().max().item()
    assert diff <= 2e-2
    assert torch.equal(kc[0, L - 1], k_out[L - 1])


def run_prefill_helper(case, dev, k_out):
    from _gpu import run_prefill
    return run_prefill(case, dev=dev, k_out=k_out)


def test_decode_deterministic():
    case = W.make_decode("det", 91, B=6, max_seq=5000, H=32, G=8, d=128,
                         seq_lens=[4999, 10, 2500, 513, 1, 4096])
    dev = device_decode_inputs(case)
    say("decode determinism")
    a = run_decode(case, dev)
    b = run_decode(case, dev)
    assert torch.equal(a, b)
