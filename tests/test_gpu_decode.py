"""GPU parity of gqa_decode (prologue + KV append + split-KV pass + combine) against the
fp64 oracle, on the 64-sequence workload and on edge cases of the split partition."""
import numpy as np
import pytest
import torch

import workloads as W

from _gpu import (check, device_decode_inputs, i32, oracle_decode_seq, run_decode, say,
                  to_f64)

pytestmark = pytest.mark.gpu


def test_decode_64_sequences_all():
    # every sequence of the 64-sequence workload, and every appended K/V row
    import _oracle_pool as OP
    case = W.decode_64()
    say("decode 64 seqs, cache", case.max_seq, "lens", int(case.seq_lens.min()), int(case.seq_lens.max()))
    dev = device_decode_inputs(case)
    out = to_f64(run_decode(case, dev))
    want, k_slots, v_slots = OP.decode_all(case)
    stats = check(out, want, W.BF16, case.name)
    say(case.name, stats)
    for b in range(case.B):
        L = int(case.seq_lens[b])
        got_k = to_f64(dev["k_cache"][b, L - 1])
        assert np.all(np.abs(got_k - k_slots[b]) <= 2.0 ** -8 * np.abs(k_slots[b]) + 1e-6), b
        assert np.array_equal(to_f64(dev["v_cache"][b, L - 1]), v_slots[b]), b


def edge_lens(S):
    """Lengths around a split-KV partition of S keys: empty, tiny, both sides of one and two
    splits, a quarter split (one wave's share), and a ragged multi-split length."""
    return [0, 1, 2, 31, 33, S // 4 - 1, S // 4 + 1, S - 1, S, S + 1, 2 * S, 2 * S + 37, 3 * S - 5]


@pytest.mark.parametrize("max_seq", [3100, 24576])
@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("H,G,d", [(32, 8, 128), (12, 4, 128), (8, 8, 64), (16, 1, 128),
                                   (6, 2, 64), (40, 1, 128), (64, 8, 128), (10, 2, 128),
                                   (16, 1, 64), (24, 2, 64), (64, 4, 128), (8, 8, 128)])
def test_decode_edge_lengths(dtype, H, G, d, max_seq):
    # the split length follows the shape (1024, 512 and 256 all occur over these cases); the
    # lengths sit on that split's edges. At max_seq 24576 the bf16 caches of the G = 8 and
    # G = 4 shapes exceed 512 MiB, so those cases take the pass that streams V non-temporally.
    # Group sizes: h = 1, 3 and 4 (one head set of the whole-row pass at d = 128), 5..8 (two sets),
    # 16 at G = 4 (four sets when streamed, else the tiled pass), 16 at G = 1 (tiled), 40
    # (tiles of 32 heads); at d = 64: 1, 3 (one set), 12 and 16 (two sets).
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


def _random_decode_shapes(n, seed):
    """n seeded draws of (B, max_seq, lengths, H, G, d, dtype, append): 1-16 sequences, a
    cache of 1-6000 rows with lengths uniform in [0, max_seq], G in {1, 2, 4, 8}, h in
    {1, 2, 3, 4, 6, 8, 12, 16, 32, 40} (H <= 128), d in {64, 128}, bf16 3 times in 4, the
    K/V append 4 times in 5."""
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        G = int(rng.choice([1, 2, 4, 8]))
        h = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16, 32, 40]))
        if G * h > 128:
            continue
        B = int(rng.integers(1, 17))
        max_seq = int(rng.integers(1, 6001))
        lens = [int(x) for x in rng.integers(0, max_seq + 1, size=B)]
        shapes.append((B, max_seq, lens, G * h, G, int(rng.choice([64, 128])),
                       W.BF16 if rng.random() < 0.75 else W.F32, bool(rng.random() < 0.8)))
    return shapes


@pytest.mark.parametrize("B,max_seq,lens,H,G,d,dtype,append", _random_decode_shapes(18, 808))
def test_decode_random_shapes(B, max_seq, lens, H, G, d, dtype, append):
    # seeded shapes beyond the edge-length grid: every sequence against the oracle
    case = W.make_decode("rand", 91 + H + G + d + B, B=B, max_seq=max_seq, H=H, G=G, d=d,
                         dtype=dtype, seq_lens=lens)
    say("decode random", B, max_seq, H, G, d, dtype, append)
    dev = device_decode_inputs(case, fill_invalid=float("nan"))
    out = to_f64(run_decode(case, dev, append=append))
    for b, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(out[b], np.zeros((H, d))), "empty sequence must give zeros"
            continue
        want, _, _ = oracle_decode_seq(case, b, append=append)
        check(out[b], want, dtype, f"b={b} L={L}")


def test_decode_at_the_split_limit():
    # The largest decode the combine pass takes at G = 1: 1024-key splits, at most 4096 of
    # them per sequence, so a 4194304-row cache (1 GiB of K, 1 GiB of V at d = 128); one
    # sequence fills it (the newest key appended at the last slot), the next stops one short.
    import attention_head_qk_amd as gqa
    B, max_seq, H, G, d = 2, 4194304, 8, 1, 128
    assert gqa.decode_split_keys(B, H, G, max_seq) * 4096 == max_seq
    lens = [max_seq, max_seq - 1]
    case = W.make_decode("splitlimit", 97, B=B, max_seq=max_seq, H=H, G=G, d=d, seq_lens=lens)
    say("decode at the split limit", max_seq)
    dev = device_decode_inputs(case)
    out = to_f64(run_decode(case, dev))
    del dev
    torch.cuda.empty_cache()
    for b, L in enumerate(lens):
        want, _, _ = oracle_decode_seq(case, b)
        check(out[b], want, W.BF16, f"b={b} L={L}")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_decode_batch_at_the_grid_limit(dtype):
    # 65535 sequences, the most a decode takes (sequences index a grid dimension), with
    # caches of 0-8 rows
    B, max_seq = 65535, 8
    lens = np.random.default_rng(5).integers(0, max_seq + 1, size=B)
    case = W.make_decode("gridlimit", 98, B=B, max_seq=max_seq, H=4, G=2, d=64, dtype=dtype,
                         seq_lens=lens)
    say("decode at the grid limit", dtype, B)
    dev = device_decode_inputs(case)
    out = to_f64(run_decode(case, dev))
    from oracle import gqa_oracle as O
    q, kn, vn = case.f64("q"), case.f64("k_new"), case.f64("v_new")
    gq, gk = case.f64("q_norm_w"), case.f64("k_norm_w")
    want = np.zeros_like(out)
    for b, L in enumerate(lens):
        if L:
            k, v = case.cache_rows(b)
            want[b] = O.decode_one(q[b], W.to_f64(k, dtype), W.to_f64(v, dtype), int(L), gq, gk,
                                   case.eps, case.theta, k_new=kn[b], v_new=vn[b])[0]
    assert np.array_equal(out[lens == 0], want[lens == 0])  # empty sequences give zeros
    check(out, want, dtype, case.name)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_decode_most_heads(dtype):
    # H = 4096 query heads on one KV head (h = 4096, the most heads taken)
    lens = [1, 300, 2048]
    case = W.make_decode("mostheads", 99, B=3, max_seq=2048, H=4096, G=1, d=64, dtype=dtype,
                         seq_lens=lens)
    say("decode most heads", dtype)
    out = to_f64(run_decode(case, device_decode_inputs(case)))
    for b, L in enumerate(lens):
        want, _, _ = oracle_decode_seq(case, b)
        check(out[b], want, dtype, f"b={b} L={L}")


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


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_decode_independent_of_split_length(dtype):
    # The same four sequences in caches of 4096 and 32768 rows, and among 60 empty ones: the
    # host picks 256-, 512- and 1024-key splits. The cross-split merge regroups the softmax
    # exactly (D1-2), so the three results differ only by rounding: in fp32 by a few ulps; in
    # bf16 also through the probabilities' rounding to bf16 against a running reference that
    # depends on where the splits fall.
    import dataclasses
    import attention_head_qk_amd as gqa
    lens = [4000, 1, 2049, 777]
    base = W.make_decode("splitinv", 97, B=4, max_seq=4096, H=32, G=8, d=128, dtype=dtype,
                         seq_lens=lens)

    def padded(B, max_seq):
        pad = lambda x: np.concatenate([x, np.zeros((B - 4,) + x.shape[1:], x.dtype)])
        return dataclasses.replace(base, max_seq=max_seq, q=pad(base.q), k_new=pad(base.k_new),
                                   v_new=pad(base.v_new),
                                   seq_lens=np.array(lens + [0] * (B - 4), dtype=np.int32))

    outs, splits = [], []
    for B, max_seq in [(4, 4096), (4, 32768), (64, 32768)]:
        case = padded(B, max_seq)
        splits.append(gqa.decode_split_keys(B, case.H, case.G, max_seq))
        say("decode split invariance", dtype, "B", B, "max_seq", max_seq, "split", splits[-1])
        outs.append(to_f64(run_decode(case, device_decode_inputs(case)))[:4])
    assert sorted(splits) == [256, 512, 1024], splits
    for b in range(4):
        want, _, _ = oracle_decode_seq(base, b)
        check(outs[0][b], want, dtype, f"b={b}")
    for o in outs[1:]:
        if dtype == W.F32:
            assert np.abs(o - outs[0]).max() <= 2e-6
        else:
            assert np.all(np.abs(o - outs[0]) <= 2.0 ** -6 * np.abs(outs[0]) + 2.0 ** -9)
