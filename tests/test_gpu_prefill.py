"""GPU parity of gqa_prefill (prologue + attention) against the fp64 oracle, element by
element, on the seeded workloads and on ragged / degenerate shapes; plus the invariants
that hold at any size (determinism, causality, packed = separate)."""
import numpy as np
import pytest
import torch

import workloads as W

from _gpu import (check, device_prefill_inputs, oracle_prefill, oracle_prefill_rows,
                  run_prefill, sample_rows, say, to_f64)

pytestmark = pytest.mark.gpu


def test_tiny_f32_full():
    case = W.tiny_f32()
    say("prefill tiny_f32 full")
    got = to_f64(run_prefill(case))
    check(got, oracle_prefill(case), W.F32, case.name)


def test_bf16_4k_full():
    case = W.prefill_4k()
    say("prefill bf16 T=4096 H=16 G=8 full")
    got = to_f64(run_prefill(case))
    stats = check(got, oracle_prefill(case), W.BF16, case.name)
    say(case.name, stats)


def test_varlen_packed_full():
    # every element of the 8-sequence varlen workload (the oracle per (sequence, head) on a
    # thread pool)
    import _oracle_pool as OP
    case = W.prefill_varlen()
    say("prefill varlen packed, full tensor", case.lengths.tolist())
    got = to_f64(run_prefill(case))
    stats = check(got, OP.prefill_full(case), W.BF16, case.name)
    say(case.name, stats)


@pytest.mark.parametrize("G", [4, 1])
def test_long_32k_sampled_rows(G):
    # at least 512 query rows with every head: rows 0, 1, the last rows, both sides of key-tile
    # and column-block boundaries, the rest seeded uniform
    import _oracle_pool as OP
    case = W.prefill_long(G)
    say(f"prefill long T=32768 H=64 G={G}")
    got = to_f64(run_prefill(case))
    rows = OP.sample_rows(case, 512, seed=G)
    assert len(rows) >= 512 and rows[0] == 0 and rows[-1] == case.N - 1
    stats = check(got[rows], oracle_prefill_rows(case, rows), W.BF16, case.name)
    say(case.name, len(rows), "rows", stats)


@pytest.mark.parametrize("T,H,G", [(8192, 32, 2), (6000, 48, 3), (3072, 32, 4)])
def test_claimed_ranks_sampled_rows(T, H, G):
    # grids of more than 2.5 rounds whose groups each span several XCDs (G < 8): the
    # workgroups take their ranks from the per-group counters instead of their block ids
    # (T = 3072, H = 32, G = 4: 768 workgroups, just past the heavy/light pairing)
    import _oracle_pool as OP
    case = W.make_prefill(f"claims_T{T}_H{H}_G{G}", 131 + G, lengths=[T], H=H, G=G, d=128)
    say("prefill with claimed ranks", T, H, G)
    got = to_f64(run_prefill(case))
    rows = OP.sample_rows(case, 256, seed=G)
    stats = check(got[rows], oracle_prefill_rows(case, rows), W.BF16, case.name)
    say(case.name, len(rows), "rows", stats)


SHAPES = [
    # (lengths, H, G, d, causal)
    ([1], 4, 2, 128, True),
    ([2], 2, 2, 128, True),
    ([63], 16, 8, 128, True),
    ([64], 16, 8, 128, True),
    ([65], 16, 8, 128, True),
    ([129], 12, 4, 128, True),      # h = 3: column blocks straddle positions
    ([200], 40, 8, 128, True),      # h = 5
    ([300], 8, 8, 128, True),       # h = 1 (MHA)
    ([150], 64, 1, 128, True),      # MQA, h = 64
    ([77], 128, 1, 128, True),      # h = 128: one position per column block
    ([97], 256, 1, 128, True),      # h = 256 > columns per block
    ([5], 4096, 1, 64, True),       # H = 4096, the most heads taken: h = 4096
    ([190], 16, 8, 64, True),       # d = 64
    ([130], 32, 8, 128, False),     # no causal mask
    ([1, 63, 64, 65, 0, 129, 7], 32, 8, 128, True),  # packed, ragged, an empty sequence
    ([40, 0, 0, 90], 16, 4, 64, False),
]


def _random_shapes(n, seed):
    """n seeded draws of (lengths, H, G, d, causal): 1-4 sequences of 0-400 tokens (packed, or
    dense when the lengths agree), G in {1, 2, 4, 8}, h in {1, 2, 3, 4, 5, 8, 16} (H <= 64),
    d in {64, 128}, causal 4 times in 5."""
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        G = int(rng.choice([1, 2, 4, 8]))
        h = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
        if G * h > 64:
            continue
        B = int(rng.integers(1, 5))
        lengths = [int(x) for x in rng.integers(0, 401, size=B)]
        if rng.random() < 0.25:
            lengths = [lengths[0]] * B
        if max(lengths) == 0:
            lengths[0] = 1
        shapes.append((lengths, G * h, G, int(rng.choice([64, 128])), bool(rng.random() < 0.8)))
    return shapes


@pytest.mark.parametrize("lengths,H,G,d,causal", _random_shapes(16, 2024))
def test_random_shapes_full(lengths, H, G, d, causal):
    # seeded combinations of the shape parameters beyond the hand-picked list, every element
    case = W.make_prefill(f"random_{lengths}_{H}_{G}_{d}_{causal}", 17 + H + G + d + len(lengths),
                          lengths=lengths, H=H, G=G, d=d, causal=causal)
    say("prefill", case.name)
    got = to_f64(run_prefill(case))
    check(got, oracle_prefill(case), W.BF16, case.name)


@pytest.mark.parametrize("lengths,H,G,d,causal", SHAPES)
def test_small_shapes_full(lengths, H, G, d, causal):
    case = W.make_prefill(f"small_{lengths}_{H}_{G}_{d}_{causal}", 11 + H + G + d,
                          lengths=lengths, H=H, G=G, d=d, causal=causal)
    say("prefill", case.name)
    got = to_f64(run_prefill(case))
    check(got, oracle_prefill(case), W.BF16, case.name)


@pytest.mark.parametrize("lengths,H,G,d", [
    ([1500, 1500], 8, 2, 128),  # dense batch of two, ragged last tile
    ([1100], 4, 4, 64),         # d = 64, h = 1
    ([2000], 8, 1, 128),        # h = 8, 125 column blocks of one group
])
def test_dense_batches_full(lengths, H, G, d):
    # mid-size dense causal grids (a few hundred blocks or fewer), every output element
    case = W.make_prefill(f"dense_{lengths}_{H}_{G}_{d}", 51 + H + G + d, lengths=lengths,
                          H=H, G=G, d=d)
    assert case.dense
    say("prefill", case.name)
    got = to_f64(run_prefill(case))
    check(got, oracle_prefill(case), W.BF16, case.name)


# more dense causal grids of about one round of workgroups, every output element
ONE_ROUND = [
    ([1024], 16, 8, 128),
    ([1000], 8, 8, 128),            # h = 1: a column block spans two key tiles of positions
    ([2048], 32, 4, 128),           # h = 8, G = 4
    ([3000], 32, 8, 64),            # d = 64, h = 4, ragged last tile
    ([700, 700, 700], 16, 8, 128),  # a dense batch of three
]


@pytest.mark.parametrize("lengths,H,G,d", ONE_ROUND)
def test_one_round_grids_full(lengths, H, G, d):
    case = W.make_prefill(f"round_{lengths}_{H}_{G}_{d}", 61 + H + G + d, lengths=lengths,
                          H=H, G=G, d=d)
    assert case.dense
    say("prefill", case.name)
    got = to_f64(run_prefill(case))
    check(got, oracle_prefill(case), W.BF16, case.name)


@pytest.mark.parametrize("lengths,H,G,d,causal", [([150], 16, 8, 64, True), ([70, 0, 33], 12, 4, 128, True),
                                                  ([100], 8, 2, 128, False)])
def test_small_shapes_f32(lengths, H, G, d, causal):
    case = W.make_prefill("f32_small", 5, lengths=lengths, H=H, G=G, d=d, causal=causal,
                          dtype=W.F32)
    say("prefill f32", lengths, H, G, d, causal)
    check(to_f64(run_prefill(case)), oracle_prefill(case), W.F32, case.name)


@pytest.mark.parametrize("lengths,H,G,d,causal", _random_shapes(8, 4242))
def test_random_shapes_f32(lengths, H, G, d, causal):
    # the fp32 path on seeded shapes, every element within the fp32 bound
    case = W.make_prefill("f32_random", 7 + H + G + d, lengths=lengths, H=H, G=G, d=d,
                          causal=causal, dtype=W.F32)
    say("prefill f32 random", lengths, H, G, d, causal)
    check(to_f64(run_prefill(case)), oracle_prefill(case), W.F32, case.name)


@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
def test_batch_at_the_grid_limit(dtype):
    # 65535 one- or two-token sequences: the fp32 kernel puts the sequence on a grid dimension
    # of at most 65535 entries (the largest batch it takes), the bf16 one numbers B * G * n_blk
    # workgroups along one dimension; every element against the oracle
    B = 65535
    lengths = [2] * B if dtype == W.BF16 else [1] * B
    case = W.make_prefill(f"gridlimit_{dtype}", 23, lengths=lengths, H=4, G=2, d=64, dtype=dtype)
    say("prefill at the grid limit", dtype, B)
    check(to_f64(run_prefill(case)), oracle_prefill(case), dtype, case.name)


def test_peaky_softmax():
    # gamma x 8 drives every row towards one-hot (Qwen3 series 1, D1-4 Q8); scores reach
    # ~1e3 in magnitude. The bf16 rounding of q~ and k~ moves such a score by about |s| 2^-8
    # (a few nats), so only rows whose oracle weight sits overwhelmingly on one key
    # (top weight > 1 - 1e-6, i.e. a gap of > 13.8 nats) have a rounding-stable answer:
    # there the output must be that key's V row. Every output must be finite and inside the
    # range of V (it is a convex combination of V rows).
    from oracle import gqa_oracle as O
    case = W.make_prefill("peaky", 21, lengths=[257], H=8, G=2, d=128)
    case.q_norm_w = W.encode(W.bf16_bits_to_f32(case.q_norm_w) * 8, W.BF16)
    case.k_norm_w = W.encode(W.bf16_bits_to_f32(case.k_norm_w) * 8, W.BF16)
    say("prefill peaky")
    got = to_f64(run_prefill(case))
    assert np.all(np.isfinite(got))
    v = case.f64("v")
    assert np.abs(got).max() <= np.abs(v).max() + 1e-2
    qt, kt = O.qk_norm_rope(case.f64("q"), case.f64("k"), case.positions, case.f64("q_norm_w"),
                            case.f64("k_norm_w"), case.eps, case.theta)
    h = case.H // case.G
    n_stable = 0
    for i in range(case.H):
        P = O.attention_weights(qt[:, i], kt[:, i // h], True)
        stable = P.max(axis=1) > 1 - 1e-6
        n_stable += int(stable.sum())
        top = np.argmax(P, axis=1)
        err = np.abs(got[stable, i] - v[top[stable], i // h])
        assert err.max(initial=0.0) <= 2e-2, (i, err.max())
    assert n_stable > case.H * 257 // 2


@pytest.mark.parametrize("sign", ["neg", "pos", "mixed"])
def test_extreme_uniform_scores(sign):
    # Every key row is the same vector x and every query row +-x, all at RoPE position 0, with
    # gamma = 3.5: every score of a (query head, key) pair is the same value, about +-200 in
    # log2 units (|s| = gamma^2 sqrt(d) after the RMSNorm). 2^-200 underflows and 2^200
    # overflows fp32, so the kernel must move its softmax reference (the exact path) to
    # get anything finite; the exact answer, whatever the rounding, is the running mean of V
    # (equal scores give uniform weights, D1-2). "mixed" alternates the sign by query head,
    # so columns of one wave need references 400 log2 units apart.
    case = W.make_prefill("extreme_" + sign, 31, lengths=[300], H=8, G=2, d=128,
                          positions=np.zeros(300, np.int32))
    rng = np.random.default_rng(32)
    x = rng.standard_normal(case.d).astype(np.float32)
    sgn = {"neg": -np.ones(case.H), "pos": np.ones(case.H),
           "mixed": np.where(np.arange(case.H) % 2 == 0, 1.0, -1.0)}[sign].astype(np.float32)
    q = np.broadcast_to(x[None, None, :] * sgn[None, :, None], (case.N, case.H, case.d))
    k = np.broadcast_to(x[None, None, :], (case.N, case.G, case.d))
    case.q = W.encode(np.ascontiguousarray(q), W.BF16)
    case.k = W.encode(np.ascontiguousarray(k), W.BF16)
    g = np.full(case.d, 3.5, np.float32)
    case.q_norm_w = W.encode(g, W.BF16)
    case.k_norm_w = W.encode(g, W.BF16)
    say("prefill extreme uniform scores", sign)
    got = to_f64(run_prefill(case))
    want = oracle_prefill(case)
    v = case.f64("v")
    h = case.H // case.G
    mean = np.cumsum(v, axis=0) / np.arange(1, case.N + 1)[:, None, None]
    assert np.allclose(want, np.repeat(mean, h, axis=1), atol=1e-9)  # the closed form
    check(got, want, W.BF16, "extreme " + sign)


def test_default_positions_and_k_out():
    import attention_head_qk_amd as gqa
    case = W.make_prefill("kout", 8, lengths=[70, 33], H=8, G=4, d=128)
    dev = device_prefill_inputs(case)
    say("prefill positions=None + k_out")
    k_out = torch.empty_like(dev["k"])
    a = run_prefill(case, dev=dev, pass_positions=False, k_out=k_out)
    b = run_prefill(case, dev=dev)
    assert torch.equal(a, b)
    from oracle import gqa_oracle as O
    _, kt = O.qk_norm_rope(case.f64("q"), case.f64("k"), case.positions, case.f64("q_norm_w"),
                           case.f64("k_norm_w"), case.eps, case.theta)
    err = np.abs(to_f64(k_out) - kt)
    assert np.all(err <= 2.0 ** -8 * np.abs(kt) + 1e-6)


@pytest.mark.parametrize("lengths,H,G,d", [
    ([4096], 16, 8, 128),
    ([3100], 24, 8, 128),        # 584 workgroups: past the pairing, zigzag order only
    ([4000], 8, 2, 128),         # 125 blocks per group: the middle block has no partner
    ([3072], 16, 8, 64),         # d = 64
    ([3072, 3072], 8, 4, 128),   # a dense batch of two: pairs within each sequence
    ([4000], 8, 8, 128),         # h = 1: a column block spans 128 positions, two key tiles
])
def test_paired_schedule(lengths, H, G, d):
    # one-round grids whose heavy blocks share their key tiles with their light partners
    # (fixed cut, partial states merged by whichever part ends last): every element against
    # the oracle, and bit-identical on a second run
    case = W.make_prefill(f"paired_{lengths}_H{H}_G{G}_d{d}", 141 + H + G + d, lengths=lengths,
                          H=H, G=G, d=d)
    assert case.dense
    dev = device_prefill_inputs(case)
    say("prefill paired schedule", lengths, H, G, d)
    first = run_prefill(case, dev=dev)
    second = run_prefill(case, dev=dev)
    assert torch.equal(first, second)
    check(to_f64(first), oracle_prefill(case), W.BF16, case.name)


def test_deterministic_and_causal():
    case = W.make_prefill("inv", 31, lengths=[333], H=16, G=4, d=128)
    dev = device_prefill_inputs(case)
    say("prefill determinism + causality")
    a = run_prefill(case, dev=dev)
    b = run_prefill(case, dev=dev)
    assert torch.equal(a, b)
    # changing tokens from row 200 on leaves rows < 200 bit-identical
    for name in ("q", "k", "v"):
        dev[name][200:] = -dev[name][200:] * 1.5
    c = run_prefill(case, dev=dev)
    assert torch.equal(a[:200], c[:200])
    assert not torch.equal(a[200:], c[200:])


def test_packed_equals_separate_calls():
    lengths = [100, 1, 64, 250]
    case = W.make_prefill("pack", 41, lengths=lengths, H=16, G=8, d=128)
    dev = device_prefill_inputs(case)
    say("prefill packed vs separate")
    packed = run_prefill(case, dev=dev, packed=True)
    import attention_head_qk_amd as gqa
    for b, t in enumerate(lengths):
        s = int(case.cu_seqlens[b])
        one = gqa.prefill(dev["q"][s:s + t][None], dev["k"][s:s + t][None],
                          dev["v"][s:s + t][None], None, q_norm_w=dev["q_norm_w"],
                          k_norm_w=dev["k_norm_w"], eps=case.eps, theta=case.theta)
        assert torch.equal(one[0], packed[s:s + t])


def test_shifted_positions_change_little():
    # RoPE makes scores depend on position differences only: shifting every position by a
    # constant changes outputs only by rounding (bf16 q~, k~ are re-rounded).
    case = W.make_prefill("shift", 51, lengths=[180], H=8, G=4, d=128)
    dev = device_prefill_inputs(case)
    say("prefill shifted positions")
    a = to_f64(run_prefill(case, dev=dev))
    dev["positions"] += 1000
    b = to_f64(run_prefill(case, dev=dev))
    assert np.abs(a - b).max() <= 2e-2
