"""GPU parity of gqa_prefill_cached (new tokens of sequences that already hold a KV cache:
chunked / multi-turn prefill) against the fp64 oracle, on small ragged shapes in full and on
the 4 x 2048-token chunk workload at sampled rows; plus what must hold between entry points
(a chunked prefill equals the one-shot prefill, one new token equals decode)."""
import numpy as np
import pytest
import torch

import workloads as W

from _gpu import (BF16_MAX_ABS, check, device_cached_inputs, device_prefill_inputs, i32,
                  oracle_prefill_cached_seq, run_prefill, run_prefill_cached, say, to_f64)

pytestmark = pytest.mark.gpu


def _check_cache(dev, case, b, kc_want, vc_want, what):
    """Rows 0 .. past + T_b - 1 of sequence b's caches against the oracle: the cached prefix
    unchanged, the appended K within bf16 rounding of the oracle's, the appended V exact."""
    past = int(case.cache_lens[b])
    L = kc_want.shape[0]
    k_rows, v_rows = case.cache_rows(b)
    got_k = to_f64(dev["k_cache"][b, :L])
    got_v = to_f64(dev["v_cache"][b, :L])
    assert np.array_equal(got_k[:past], W.to_f64(k_rows, W.BF16)), what
    assert np.array_equal(got_v[:past], W.to_f64(v_rows, W.BF16)), what
    kt = kc_want[past:]
    assert np.all(np.abs(got_k[past:] - kt) <= 2.0 ** -8 * np.abs(kt) + 1e-6), what
    assert np.array_equal(got_v[past:], vc_want[past:]), what


SHAPES = [
    # (new lengths, cache lengths, max_seq, H, G, d, causal)
    ([100, 100, 100], [0, 37, 500], 1024, 16, 8, 128, True),   # dense batch, an empty cache
    ([64, 1, 130, 0], [10, 0, 2000, 5], 2200, 32, 8, 128, True),  # packed, ragged, empty chunk
    ([190], [333], 600, 16, 4, 64, True),                       # d = 64
    ([129], [64], 200, 8, 8, 128, True),                         # h = 1, chunk on a tile edge
    ([50], [77], 130, 64, 1, 128, True),                         # MQA, h = 64
    ([65, 3], [191, 253], 256, 12, 4, 128, True),                # chunks end at max_seq
    ([70, 30], [100, 0], 256, 8, 2, 128, False),                 # no causal mask
]


def _random_cached_shapes(n, seed):
    """n seeded draws of (lengths, cache_lens, max_seq, H, G, d, causal): 1-4 sequences with
    chunks of 0-300 new tokens after caches of 0-700 rows (packed, or dense when the chunk
    lengths agree), max_seq 0-100 rows above the longest, G in {1, 2, 4, 8}, h in
    {1, 2, 3, 4, 8, 16} (H <= 64), d in {64, 128}, causal 4 times in 5."""
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        G = int(rng.choice([1, 2, 4, 8]))
        h = int(rng.choice([1, 2, 3, 4, 8, 16]))
        if G * h > 64:
            continue
        B = int(rng.integers(1, 5))
        lengths = [int(x) for x in rng.integers(0, 301, size=B)]
        if rng.random() < 0.25:
            lengths = [lengths[0]] * B
        if max(lengths) == 0:
            lengths[0] = 1
        cache_lens = [int(x) for x in rng.integers(0, 701, size=B)]
        max_seq = max(c + t for c, t in zip(cache_lens, lengths)) + int(rng.integers(0, 101))
        shapes.append((lengths, cache_lens, max_seq, G * h, G, int(rng.choice([64, 128])),
                       bool(rng.random() < 0.8)))
    return shapes


@pytest.mark.parametrize("lengths,cache_lens,max_seq,H,G,d,causal",
                         SHAPES + _random_cached_shapes(10, 404))
def test_small_cached_full(lengths, cache_lens, max_seq, H, G, d, causal):
    # the hand-picked shapes, then seeded random ones
    case = W.make_cached_prefill(f"cached_{lengths}_{cache_lens}", 90 + H + G + d, lengths,
                                 cache_lens, max_seq, H=H, G=G, d=d, causal=causal)
    say("prefill cached", case.name, max_seq, H, G, d, causal)
    # rows past each sequence's chunk hold NaN: the kernel must neither read nor write them
    dev = device_cached_inputs(case, fill_invalid=float("nan"))
    got = to_f64(run_prefill_cached(case, dev))
    for b in range(case.B):
        s, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        want, kc, vc = oracle_prefill_cached_seq(case, b)
        if e > s:
            check(got[s:e], want, W.BF16, f"{case.name} b={b}")
        _check_cache(dev, case, b, kc, vc, f"{case.name} b={b}")
        assert torch.isnan(dev["k_cache"][b, kc.shape[0]:].float()).all()
        assert torch.isnan(dev["v_cache"][b, kc.shape[0]:].float()).all()


def _oracle_rows(case, b, rows):
    """Oracle output rows of a causal cached prefill, one row at a time: under the causal
    mask new token t sees exactly the keys of a chunk that ends at t, so row t is the one new
    token of a cached prefill whose cache holds the prefix and new tokens 0 .. t-1 (the
    oracle's own K rows for those)."""
    from oracle import gqa_oracle as O
    s, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
    past = int(case.cache_lens[b])
    k, v = case.cache_rows(b)
    q, kn, vn = case.f64("q")[s:e], case.f64("k")[s:e], case.f64("v")[s:e]
    pos = case.positions[s:e]
    _, kt_new = O.qk_norm_rope(q, kn, pos, case.f64("q_norm_w"), case.f64("k_norm_w"),
                               case.eps, case.theta)
    kc = np.concatenate([W.to_f64(k, W.BF16), kt_new])[None]
    vc = np.concatenate([W.to_f64(v, W.BF16), vn])[None]
    out = []
    for t in rows:
        o, _, _ = O.prefill_cached(q[t:t + 1], kn[t:t + 1], vn[t:t + 1], kc[:, :past + t + 1],
                                   vc[:, :past + t + 1], [past + t], np.array([0, 1]),
                                   case.f64("q_norm_w"), case.f64("k_norm_w"), case.eps,
                                   case.theta, positions=pos[t:t + 1])
        out.append(o[0])
    return np.stack(out), kt_new


def test_chunked_workload_sampled_rows():
    case = W.prefill_chunked()
    say("prefill cached workload", case.name, case.cache_lens.tolist())
    dev = device_cached_inputs(case)
    got = to_f64(run_prefill_cached(case, dev))
    rng = np.random.default_rng(12)
    T = int(case.lengths[0])
    for b in (int(np.argmin(case.cache_lens)), int(np.argmax(case.cache_lens))):
        rows = sorted({0, 1, 63, 64, 127, 128, T - 2, T - 1} |
                      {int(x) for x in rng.integers(0, T, size=12)})
        want, kt_new = _oracle_rows(case, b, rows)
        s = int(case.cu_seqlens[b])
        check(got[s + np.array(rows)], want, W.BF16, f"b={b} past={case.cache_lens[b]}")
        past = int(case.cache_lens[b])
        got_k = to_f64(dev["k_cache"][b, past:past + T])
        assert np.all(np.abs(got_k - kt_new) <= 2.0 ** -8 * np.abs(kt_new) + 1e-6)
        assert np.array_equal(to_f64(dev["v_cache"][b, past:past + T]), case.f64("v")[s:s + T])
        assert not dev["k_cache"][b, past + T:].any() and not dev["v_cache"][b, past + T:].any()


def test_explicit_positions():
    case = W.make_cached_prefill("cached_pos", 95, [80, 41], [300, 7], 512, H=16, G=8)
    dev = device_cached_inputs(case)
    rng = np.random.default_rng(96)
    pos = rng.integers(0, 100000, size=case.N).astype(np.int32)
    dev["positions"] = i32(pos)
    say("prefill cached explicit positions")
    got = to_f64(run_prefill_cached(case, dev))
    for b in range(case.B):
        s, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        want, kc, vc = oracle_prefill_cached_seq(case, b, positions=pos[s:e])
        check(got[s:e], want, W.BF16, f"b={b}")
        _check_cache(dev, case, b, kc, vc, f"b={b}")


def test_chunks_equal_one_prefill():
    # A prefix by gqa_prefill (its K after the prologue kept through k_out) and the rest by
    # gqa_prefill_cached give the one-shot prefill's output bit for bit: the appended K rows
    # are the one-shot prologue's (same positions, same arithmetic), and every query column
    # walks the same key tiles from key 0 in the same order (tiles past its own position are
    # fully masked and add exact zeros).
    import attention_head_qk_amd as gqa
    L, P, H, G, d, S = 1300, 700, 32, 8, 128, 2048
    full = W.make_prefill("chunks", 97, lengths=[L], H=H, G=G, d=d)
    dev = device_prefill_inputs(full)
    say("prefill cached: chunks vs one prefill")
    k_out = torch.empty_like(dev["k"])
    one = run_prefill(full, dev=dev, k_out=k_out)
    kc = torch.zeros((1, S, G, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    common = dict(q_norm_w=dev["q_norm_w"], k_norm_w=dev["k_norm_w"], eps=full.eps,
                  theta=full.theta)
    pre = gqa.prefill(dev["q"][None, :P], dev["k"][None, :P], dev["v"][None, :P], None,
                      k_out=kc[:, :P], **common)
    vc[0, :P] = dev["v"][:P]
    rest = gqa.prefill_cached(dev["q"][None, P:], dev["k"][None, P:], dev["v"][None, P:], kc, vc,
                              i32([P]), **common)
    torch.cuda.synchronize()
    assert torch.equal(kc[0, :L], k_out)
    assert torch.equal(vc[0, :L], dev["v"])
    assert torch.equal(pre[0], one[:P])
    err = (rest[0].float() - one[P:].float()).abs()
    say("chunked vs one-shot: max abs", float(err.max()))
    assert torch.equal(rest[0], one[P:])


def test_one_new_token_equals_decode():
    import attention_head_qk_amd as gqa
    lens = [1, 700, 4097, 64]
    case = W.make_cached_prefill("cached_one", 98, [1] * 4, lens, 4200, H=32, G=8)
    dev = device_cached_inputs(case)
    say("prefill cached: one token vs decode")
    kc0, vc0 = dev["k_cache"].clone(), dev["v_cache"].clone()
    a = run_prefill_cached(case, dev)
    dec = gqa.decode(dev["q"], kc0, vc0, i32(np.asarray(lens) + 1), k_new=dev["k"],
                     v_new=dev["v"], q_norm_w=dev["q_norm_w"], k_norm_w=dev["k_norm_w"],
                     eps=case.eps, theta=case.theta)
    torch.cuda.synchronize()
    assert torch.equal(dev["k_cache"], kc0) and torch.equal(dev["v_cache"], vc0)
    # two kernels, each rounded to bf16 and each held to the oracle below: they may differ by
    # twice the per-element bound
    assert float((a.float() - dec.float()).abs().max()) <= 2 * BF16_MAX_ABS
    got = to_f64(a)
    for b in range(case.B):
        want, _, _ = oracle_prefill_cached_seq(case, b)
        check(got[b:b + 1], want, W.BF16, f"b={b}")


def test_empty_cache_equals_prefill():
    case = W.make_cached_prefill("cached_empty", 99, [150, 150], [0, 0], 256, H=16, G=4)
    dev = device_cached_inputs(case)
    say("prefill cached: empty cache vs prefill")
    a = run_prefill_cached(case, dev)
    b = run_prefill(case.new, dev=dev)
    err = (a.float() - b.float()).abs()
    say("empty cache vs prefill: max abs", float(err.max()), "bit-equal", bool((err == 0).all()))
    assert float(err.max()) <= 1e-2
    got = to_f64(a)
    for s in range(case.B):
        want, _, _ = oracle_prefill_cached_seq(case, s)
        check(got[150 * s:150 * (s + 1)], want, W.BF16, f"b={s}")


def test_nothing_new():
    import attention_head_qk_amd as gqa
    case = W.make_cached_prefill("cached_none", 100, [0, 0], [5, 9], 16, H=8, G=4)
    dev = device_cached_inputs(case)
    kc0 = dev["k_cache"].clone()
    say("prefill cached: no new tokens")
    out = gqa.prefill_cached(dev["q"], dev["k"], dev["v"], dev["k_cache"], dev["v_cache"],
                             dev["cache_lens"], cu_seqlens=dev["cu"], max_seqlen=0,
                             q_norm_w=dev["q_norm_w"], k_norm_w=dev["k_norm_w"])
    torch.cuda.synchronize()
    assert out.numel() == 0 and torch.equal(dev["k_cache"], kc0)
