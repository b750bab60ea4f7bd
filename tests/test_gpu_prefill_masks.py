"""GPU parity of the mask variants of the bf16 prefill (sliding window, 64-key block layout,
both) against the fp64 oracle, element by element on small ragged shapes and at 4096 tokens,
on sampled rows at 32768 tokens; plus the invariants that tie them to the plain kernel
(a window covering the sequence, or a full layout, changes no bit)."""
import numpy as np
import pytest
import torch

import workloads as W

from _gpu import (BF16_MAX_ABS, BF16_MEAN_ABS, check, device_block_mask, device_cached_inputs,
                  device_prefill_inputs, oracle_prefill, oracle_prefill_cached_seq,
                  oracle_prefill_rows, run_prefill, run_prefill_cached, sample_rows, say, to_f64)

pytestmark = pytest.mark.gpu


def _nb(T):
    return max(1, -(-T // 64))


WINDOW_SHAPES = [
    # (lengths, H, G, d, window)
    ([300], 16, 8, 128, 1),          # only the diagonal
    ([300], 16, 8, 128, 37),
    ([300], 16, 8, 128, 64),
    ([300], 16, 8, 128, 100),
    ([300], 8, 8, 128, 100),         # h = 1: a workgroup spans 128 positions
    ([257], 64, 1, 128, 70),         # MQA
    ([190], 16, 4, 64, 70),          # d = 64
    ([1, 63, 64, 65, 0, 129, 200], 32, 8, 128, 50),  # packed, ragged, an empty sequence
]


@pytest.mark.parametrize("lengths,H,G,d,window", WINDOW_SHAPES)
def test_window_full(lengths, H, G, d, window):
    case = W.make_prefill(f"win_{lengths}_{H}_{G}_{d}_{window}", 120 + H + G + d + window,
                          lengths=lengths, H=H, G=G, d=d)
    say("prefill window", case.name)
    got = to_f64(run_prefill(case, window=window))
    check(got, oracle_prefill(case, window=window), W.BF16, case.name)


BLOCK_SHAPES = [
    # (lengths, H, G, d, density, causal)
    ([333], 16, 8, 128, 0.3, True),   # h = 2: one query block per workgroup
    ([257], 8, 8, 128, 0.3, True),    # h = 1: two query blocks per workgroup
    ([150], 64, 1, 128, 0.5, True),   # MQA
    ([100, 1, 200, 64], 16, 4, 128, 0.4, True),
    ([260], 8, 8, 128, 0.0, True),    # diagonal blocks only
    ([190], 16, 4, 64, 0.3, True),    # d = 64
    ([130], 32, 8, 128, 0.4, False),  # no causal mask: later blocks too
]


@pytest.mark.parametrize("lengths,H,G,d,density,causal", BLOCK_SHAPES)
def test_block_mask_full(lengths, H, G, d, density, causal):
    case = W.make_prefill(f"blk_{lengths}_{H}_{G}_{d}_{density}", 140 + H + G + d,
                          lengths=lengths, H=H, G=G, d=d, causal=causal)
    nb = _nb(max(lengths))
    bm = W.make_block_mask(141 + H, nb, density, causal=causal)
    say("prefill block mask", case.name, "kept", int(bm.sum()), "of", nb * nb)
    got = to_f64(run_prefill(case, block_mask=device_block_mask(bm)))
    check(got, oracle_prefill(case, block_mask=bm), W.BF16, case.name)


def _random_mask_shapes(n, seed):
    """n seeded draws of (lengths, H, G, d, window, density, causal): 1-3 sequences of 0-520
    tokens (packed, or dense when the lengths agree), G in {1, 2, 4, 8}, h in
    {1, 2, 3, 4, 8, 16} (H <= 64), d in {64, 128}; a window (1 key, or 8-600 keys across and
    inside key tiles; 2-7 keys have a test of their own below), a 64-key block layout (kept
    share 0-1, causal or not), or both."""
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        G = int(rng.choice([1, 2, 4, 8]))
        h = int(rng.choice([1, 2, 3, 4, 8, 16]))
        if G * h > 64:
            continue
        B = int(rng.integers(1, 4))
        lengths = [int(x) for x in rng.integers(0, 521, size=B)]
        if rng.random() < 0.25:
            lengths = [lengths[0]] * B
        if max(lengths) == 0:
            lengths[0] = 1
        d = int(rng.choice([64, 128]))
        kind = str(rng.choice(["window", "block", "both"]))
        window = int(rng.choice([1, 8, 63, 64, 65, 127, 200, 600])) if kind != "block" else 0
        density = float(rng.choice([0.0, 0.15, 0.5, 1.0])) if kind != "window" else -1.0
        causal = bool(rng.random() < 0.8) if kind == "block" else True
        shapes.append((lengths, G * h, G, d, window, density, causal))
    return shapes


@pytest.mark.parametrize("lengths,H,G,d,window,density,causal", _random_mask_shapes(16, 77))
def test_random_masks_full(lengths, H, G, d, window, density, causal):
    # seeded combinations of shapes and masks beyond the hand-picked lists, every element
    case = W.make_prefill(f"rmask_{lengths}_{H}_{G}_{d}_{window}_{density}", 170 + H + G + d,
                          lengths=lengths, H=H, G=G, d=d, causal=causal)
    masks = {}
    if window:
        masks["window"] = window
    bm = None
    if density >= 0:
        bm = W.make_block_mask(171 + H + d, _nb(max(lengths)), density, causal=causal)
    say("prefill random masks", case.name)
    got = to_f64(run_prefill(case, block_mask=device_block_mask(bm) if bm is not None else None,
                             **masks))
    if bm is not None:
        masks["block_mask"] = bm
    check(got, oracle_prefill(case, **masks), W.BF16, case.name)


@pytest.mark.parametrize("lengths,H,G,d,window", [([394], 64, 4, 64, 2), ([300], 16, 8, 128, 3),
                                                 ([1, 65, 200], 8, 2, 128, 5)])
def test_tiny_windows_full(lengths, H, G, d, window):
    # A window of 2-7 keys makes every output a weighted mean of a few V rows, as large as the
    # rows themselves (|v| up to ~5 for N(0,1) values), and puts it at the mercy of two or
    # three weights. Storing q~ and k~ in bf16 (the bf16 path's operand format) then moves the
    # exact outputs by up to 0.016 on these cases, and one bf16 rounding of the output by up
    # to 2^-8 |out| ~ 0.02, so the absolute bound cannot hold against the fp64 oracle here
    # whatever the kernel does. The element-wise check therefore runs against the oracle's
    # attention on its own q~ and k~ rounded to bf16 (on the CPU), with the output's rounding
    # added to the absolute bound; the mean bound is checked against the plain oracle.
    from oracle import gqa_oracle as O
    case = W.make_prefill(f"tinywin_{lengths}_{H}_{G}_{d}_{window}", 180 + H + G + d + window,
                          lengths=lengths, H=H, G=G, d=d)
    say("prefill tiny window", case.name)
    got = to_f64(run_prefill(case, window=window))
    assert np.all(np.isfinite(got))
    want = oracle_prefill(case, window=window)
    assert np.abs(got - want).mean() <= BF16_MEAN_ABS
    qt, kt = O.qk_norm_rope(case.f64("q"), case.f64("k"), case.positions, case.f64("q_norm_w"),
                            case.f64("k_norm_w"), case.eps, case.theta)
    def as_bf16(x):
        return W.to_f64(W.encode(x.astype(np.float32), W.BF16), W.BF16)
    qb, kb, v = as_bf16(qt), as_bf16(kt), case.f64("v")
    want_b = np.zeros_like(want)
    for b in range(case.B):
        s, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        if e > s:
            want_b[s:e] = O.attend(qb[s:e], kb[s:e], v[s:e], True, window=window)
    excess = np.abs(got - want_b) - 2.0 ** -8 * np.abs(want_b)
    assert excess.max() <= BF16_MAX_ABS, excess.max()


@pytest.mark.parametrize("lengths,H,G", [([400], 16, 4), ([300], 8, 8)])
def test_window_and_block_mask_full(lengths, H, G):
    case = W.make_prefill(f"winblk_{lengths}_{H}_{G}", 160 + H + G, lengths=lengths, H=H, G=G)
    bm = W.make_block_mask(161, _nb(max(lengths)), 0.4)
    say("prefill window + block mask", case.name)
    got = to_f64(run_prefill(case, window=150, block_mask=device_block_mask(bm)))
    check(got, oracle_prefill(case, window=150, block_mask=bm), W.BF16, case.name)


def test_window_at_maximum_length_sampled_rows():
    # The longest sequence the bf16 kernel takes at G = 1, d = 128: it addresses a group's K/V
    # rows with 32-bit byte offsets, so T * G * d * 2 < 2^31, T = 8388607 (h = 2: 16.8 M
    # columns). A 512-key window keeps the work linear. The inputs repeat one seeded
    # 65536-token block (RoPE positions still run 0 .. T - 1, so no two windows see the same
    # rotated keys); each sampled row is checked against the oracle on the 512 keys it sees,
    # passed as a sequence of its own at their true positions.
    import dataclasses
    T, P, window = 8388607, 1 << 16, 512
    base = W.make_prefill("maxlen_block", 191, lengths=[P], H=2, G=1, d=128)
    reps = -(-T // P)

    def tile(a):
        return np.ascontiguousarray(np.tile(a, (reps, 1, 1))[:T])

    case = dataclasses.replace(base, name="maxlen_window", lengths=np.array([T]),
                               q=tile(base.q), k=tile(base.k), v=tile(base.v),
                               positions=np.arange(T, dtype=np.int32),
                               cu_seqlens=np.array([0, T], dtype=np.int32))
    say("prefill window 512 at the maximum length", T)
    rows = [0, 511, 512, 4096, 1 << 22, (1 << 22) + 63, (1 << 22) + 64, (1 << 23) - 1000,
            T - 65, T - 64, T - 63, T - 2, T - 1]
    out = run_prefill(case, window=window)
    got = to_f64(out[rows])
    del out
    torch.cuda.empty_cache()
    for r, g in zip(rows, got):
        lo = max(0, r - window + 1)
        n = r + 1 - lo
        sub = dataclasses.replace(case, name=f"row {r}", lengths=np.array([n]), q=case.q[lo:r + 1],
                                  k=case.k[lo:r + 1], v=case.v[lo:r + 1],
                                  positions=np.arange(lo, r + 1, dtype=np.int32),
                                  cu_seqlens=np.array([0, n], dtype=np.int32))
        check(g[None], oracle_prefill(sub, window=window)[-1:], W.BF16, f"row {r}")


def test_window_4k_full():
    case = W.prefill_4k()
    say("prefill window 512 at T=4096")
    got = to_f64(run_prefill(case, window=512))
    check(got, oracle_prefill(case, window=512), W.BF16, case.name)


@pytest.mark.parametrize("kind", ["window", "blocks"])
def test_long_32k_sampled_rows(kind):
    # at least 512 query rows with every head (see the plain kernel's long test)
    import _oracle_pool as OP
    case = W.prefill_long(4)
    rows = OP.sample_rows(case, 512, seed=7)
    assert len(rows) >= 512
    if kind == "window":
        masks = dict(window=512)
        dev_masks = dict(window=512)
    else:
        bm = W.make_block_mask(171, _nb(case.T_max), 0.1)
        masks = dict(block_mask=bm)
        dev_masks = dict(block_mask=device_block_mask(bm))
    say("prefill long T=32768 H=64 G=4", kind)
    got = to_f64(run_prefill(case, **dev_masks))
    check(got[rows], oracle_prefill_rows(case, rows, **masks), W.BF16, case.name + " " + kind)


def test_cached_prefill_with_masks():
    case = W.make_cached_prefill("cached_masks", 180, [100, 37], [150, 64], 320, H=16, G=8)
    bm = W.make_block_mask(181, _nb(case.max_seq), 0.4)
    dev = device_cached_inputs(case)
    say("prefill cached with window + block mask")
    got = to_f64(run_prefill_cached(case, dev, window=90, block_mask=device_block_mask(bm)))
    for b in range(case.B):
        s, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        want, _, _ = oracle_prefill_cached_seq(case, b, window=90, block_mask=bm)
        check(got[s:e], want, W.BF16, f"b={b}")


def test_wide_masks_change_no_bit():
    # a window of at least the sequence and a layout with every block kept visit the same
    # tiles in the same order: the masked variants agree bit for bit with each other, and
    # with the plain kernel up to the order of its score sums (the plain kernel runs its
    # score product one tile ahead in two accumulator chains, the masked ones in four)
    case = W.make_prefill("wide", 190, lengths=[700], H=16, G=8)
    dev = device_prefill_inputs(case)
    say("prefill wide masks vs plain")
    plain = run_prefill(case, dev=dev)
    full = np.ones((_nb(700), _nb(700)), dtype=bool)
    win = run_prefill(case, dev=dev, window=700)
    assert torch.equal(run_prefill(case, dev=dev, window=100000), win)
    assert torch.equal(run_prefill(case, dev=dev, block_mask=device_block_mask(full)), win)
    err = (win.float() - plain.float()).abs()
    assert float(err.max()) <= 2e-2 and float(err.mean()) <= 1e-3


@pytest.mark.parametrize("sign", ["neg", "mixed"])
def test_window_extreme_scores(sign):
    # equal scores of +-200 in log2 units (see the plain kernel's extreme test): the exact
    # path must engage also when some columns of a wave have seen no key yet
    case = W.make_prefill("win_extreme_" + sign, 191, lengths=[300], H=8, G=8,
                          positions=np.zeros(300, np.int32))
    rng = np.random.default_rng(192)
    x = rng.standard_normal(case.d).astype(np.float32)
    sgn = {"neg": -np.ones(case.H), "mixed": np.where(np.arange(case.H) % 2 == 0, 1.0, -1.0)}[sign]
    q = np.broadcast_to(x[None, None, :] * sgn.astype(np.float32)[None, :, None],
                        (case.N, case.H, case.d))
    k = np.broadcast_to(x[None, None, :], (case.N, case.G, case.d))
    case.q = W.encode(np.ascontiguousarray(q), W.BF16)
    case.k = W.encode(np.ascontiguousarray(k), W.BF16)
    g = np.full(case.d, 3.5, np.float32)
    case.q_norm_w = W.encode(g, W.BF16)
    case.k_norm_w = W.encode(g, W.BF16)
    say("prefill window extreme scores", sign)
    got = to_f64(run_prefill(case, window=100))
    want = oracle_prefill(case, window=100)
    v = case.f64("v")
    # equal scores: each row is the mean of V over its window (the closed form)
    for t in (0, 50, 99, 100, 299):
        lo = max(0, t - 99)
        assert np.allclose(want[t], np.repeat(v[lo:t + 1].mean(axis=0), 1, axis=0), atol=1e-9)
    check(got, want, W.BF16, "window extreme " + sign)
