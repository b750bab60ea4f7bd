"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test names the passage it rests on. The pages print no numeric attention example, so
the pins are closed forms for small hand inputs, the properties the pages state, brute force
on tiny inputs and a library special case (torch's scaled_dot_product_attention in float64
on the CPU, which the oracle itself never imports).
"""
import cmath
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import brute
from oracle import gqa_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ============================================================================ RMSNorm (D2-1)
def test_rmsnorm_unit_rms_before_weight():
    # Qwen3 series 1, D2-1: with gamma = 1 and eps = 0 the output has RMS exactly 1.
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 3, 64)) * rng.uniform(0.1, 10, size=(5, 3, 1))
    y = O.rms_norm(x, np.ones(64), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-13)


def test_rmsnorm_eps_inside_root():
    # eps sits under the square root: RMS(x_hat) = sqrt(ms / (ms + eps)).
    x = np.array([[1.0, -2.0, 3.0, 0.5]])
    eps = 0.75
    ms = np.mean(x * x)
    y = O.rms_norm(x, np.ones(4), eps)
    assert math.isclose(float(np.sqrt(np.mean(y * y))), math.sqrt(ms / (ms + eps)), rel_tol=1e-14)


def test_rmsnorm_hand_value_and_weight_after_normalising():
    g = _gold("rmsnorm_rope_dot.json")
    q = np.array([g["q"]])
    # (3, 4): mean square 12.5 -> (3, 4) / sqrt(12.5)
    y = O.rms_norm(q, np.ones(2), 0.0)[0]
    assert np.allclose(y, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], atol=1e-15)
    assert math.isclose(y[0], 0.848528137423857, rel_tol=1e-13)
    # gamma multiplies the normalised vector element-wise (not the input before the norm)
    gw = np.array(g["gamma_weighted"])
    yw = O.rms_norm(q, gw, 0.0)[0]
    assert np.allclose(yw, [2 * 3 / math.sqrt(12.5), 0.5 * 4 / math.sqrt(12.5)], atol=1e-15)


def test_rmsnorm_scale_invariant_and_none_skips():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 2, 8))
    gam = rng.uniform(0.5, 1.5, 8)
    assert np.allclose(O.rms_norm(7.5 * x, gam, 0.0), O.rms_norm(x, gam, 0.0), atol=1e-14)
    assert np.array_equal(O.rms_norm(x, None, 1e-6), x)


# ============================================================================ RoPE (D2-2, 3.1.2, 3.4.1)
def test_rope_d2_is_complex_rotation():
    # With d = 2 the single frequency is theta^0 = 1: R(p) rotates counter-clockwise by p
    # radians, i.e. multiplies x0 + i x1 by e^{ip} (Qwen3 architecture 3.1.2 complex product).
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 1, 2))
    pos = np.array([0, 1, 2, 5, 100, 4095])
    y = O.rope(x, pos, 1e6)
    for t in range(6):
        z = complex(x[t, 0, 0], x[t, 0, 1]) * cmath.exp(1j * pos[t])
        assert abs(complex(y[t, 0, 0], y[t, 0, 1]) - z) < 1e-13


def test_rope_pairs_and_frequencies_d4():
    # d = 4, theta = 100: pair (0,1) turns by p, pair (2,3) by p * 100^(-2/4) = p / 10.
    x = np.array([[[0.3, -1.2, 2.0, 0.7]]])
    p = 3
    y = O.rope(x, np.array([p]), 100.0)[0, 0]
    z0 = complex(0.3, -1.2) * cmath.exp(1j * p)
    z1 = complex(2.0, 0.7) * cmath.exp(1j * p / 10)
    assert np.allclose(y, [z0.real, z0.imag, z1.real, z1.imag], atol=1e-14)


def test_rope_inv_freq_base_1e6():
    w = O.rope_inv_freq(128, 1e6)
    assert w[0] == 1.0
    assert math.isclose(w[1], 1e6 ** (-2 / 128), rel_tol=1e-15)
    assert math.isclose(w[63], 1e6 ** (-126 / 128), rel_tol=1e-14)
    assert np.all(np.diff(w) < 0)


def test_rope_norm_preserving_transpose_identity():
    # Qwen3 series 1, D2-2: rotation keeps the length; R(p)^T = R(-p); R(0) = I.
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 3, 128))
    pos = rng.integers(0, 32768, 7)
    y = O.rope(x, pos, 1e6)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    assert np.allclose(O.rope(y, -pos, 1e6), x, atol=1e-12)
    assert np.array_equal(O.rope(x, np.zeros(7, int), 1e6), x)


def test_rope_relative_position():
    # <R(m)a, R(n)b> depends only on m - n (Qwen3 study log RoPE intro; D2-2).
    rng = np.random.default_rng(4)
    a = rng.standard_normal((1, 1, 64))
    b = rng.standard_normal((1, 1, 64))
    ref = None
    for m, n in [(7, 3), (11, 7), (1007, 1003), (32767, 32763)]:
        s = float(np.sum(O.rope(a, np.array([m]), 1e6) * O.rope(b, np.array([n]), 1e6)))
        ref = s if ref is None else ref
        assert math.isclose(s, ref, rel_tol=1e-9, abs_tol=1e-9)


def test_rope_matches_block_diagonal_matrix():
    # the explicit matrix R(pos) of D2-2 (brute force) against the vectorised rotation
    rng = np.random.default_rng(5)
    for d in (2, 4, 8, 16):
        x = rng.standard_normal(d)
        for pos in (0, 1, 9, 1234):
            ref = brute.matvec(brute.rope_matrix(pos, d, 1e4), list(x))
            got = O.rope(x[None, None, :], np.array([pos]), 1e4)[0, 0]
            assert np.allclose(got, ref, atol=1e-12)


def test_norm_then_rope_hand_value():
    # D2-2 task: RMSNorm a 2-d query, rotate, dot with a key. q=(3,4) at position 1,
    # k=(1,0) at position 0, eps=0, gamma=1: q_hat=(3,4)/sqrt(12.5), k_hat=(sqrt2, 0);
    # dot = sqrt(2)/sqrt(12.5) * (3 cos 1 - 4 sin 1) = 0.4 * (3 cos 1 - 4 sin 1).
    g = _gold("rmsnorm_rope_dot.json")
    q = np.array([[g["q"]]])
    k = np.array([[g["k"]]])
    want = 0.4 * (3 * math.cos(1) - 4 * math.sin(1))
    for qp, kp in [(g["q_pos"], g["k_pos"]), tuple(g["shifted_positions"])]:
        qt, _ = O.qk_norm_rope(q, k, np.array([qp]), np.ones(2), np.ones(2), g["eps"], g["theta"])
        _, kt = O.qk_norm_rope(q, k, np.array([kp]), np.ones(2), np.ones(2), g["eps"], g["theta"])
        assert math.isclose(float(qt[0, 0] @ kt[0, 0]), want, rel_tol=1e-12)
    assert math.isclose(want, -0.697990808651, rel_tol=1e-10)
    # with gamma = (2, 0.5): normalise, weight, then rotate (norm before RoPE, forward
    # steps (4) then (5) of the nano-vllm page). Rotating first gives a different vector.
    gw = np.array(g["gamma_weighted"])
    qt, _ = O.qk_norm_rope(q, k, np.array([1]), gw, gw, 0.0, g["theta"])
    z = complex(6 / math.sqrt(12.5), 2 / math.sqrt(12.5)) * cmath.exp(1j)
    assert np.allclose(qt[0, 0], [z.real, z.imag], atol=1e-14)
    zr = complex(3, 4) * cmath.exp(1j) / math.sqrt(12.5)
    assert not np.allclose(qt[0, 0], [2 * zr.real, 0.5 * zr.imag], atol=1e-3)


# ============================================================================ attention core
def test_hand_example_3_tokens_d2():
    g = _gold("hand_3tok_d2.json")
    Q = np.array(g["Q"])[:, None, :]
    K = np.array(g["K"])[:, None, :]
    V = np.array(g["V"])[:, None, :]
    out = O.attend(Q, K, V, causal=True)[:, 0, :]
    a = 1 / math.sqrt(2)
    # row 0 sees only key 0
    w1 = [1 / (1 + math.exp(a)), math.exp(a) / (1 + math.exp(a))]  # scores [0, a]
    z2 = 2 + math.exp(a)  # scores [a, a, 2a] ~ [1, 1, e^a]
    w2 = [1 / z2, 1 / z2, math.exp(a) / z2]
    Vl = g["V"]
    want = [Vl[0],
            [w1[0] * Vl[0][c] + w1[1] * Vl[1][c] for c in range(2)],
            [sum(w2[j] * Vl[j][c] for j in range(3)) for c in range(2)]]
    assert np.allclose(out, want, atol=1e-14)
    assert math.isclose(out[1, 0], 2.339523098653, rel_tol=1e-11)
    assert math.isclose(out[2, 0], 3.510469530454, rel_tol=1e-11)
    P = O.attention_weights(Q[:, 0], K[:, 0], True)
    assert np.allclose(P[2], w2, atol=1e-15)
    assert P[0, 1] == 0.0 and P[0, 2] == 0.0 and P[1, 2] == 0.0


def test_mini_gqa_two_heads_one_kv():
    g = _gold("mini_gqa_2q1kv.json")
    q, k, v = (np.array(g[n]) for n in ("q", "k", "v"))
    out = O.attend(q, k, v, causal=True)
    a = 1 / math.sqrt(2)
    assert np.allclose(out[0, 0], [1, 0]) and np.allclose(out[0, 1], [1, 0])
    # token 1, head 0: q=(0,1): scores [0, a]
    w = [1 / (1 + math.exp(a)), math.exp(a) / (1 + math.exp(a))]
    assert np.allclose(out[1, 0], w, atol=1e-15)
    # token 1, head 1: q=(-1,1): scores [-a, a] -> [1, e^{2a}] / (1 + e^{2a})
    w = [1 / (1 + math.exp(math.sqrt(2))), math.exp(math.sqrt(2)) / (1 + math.exp(math.sqrt(2)))]
    assert np.allclose(out[1, 1], w, atol=1e-15)
    assert math.isclose(out[1, 1, 0], 0.195570317493, rel_tol=1e-10)


def test_softmax_rows_sum_to_one_and_masked_zero():
    # Qwen3 series 1, D1-4 (each row sums to 1) and D1-5 (masked weights are 0).
    rng = np.random.default_rng(6)
    q = rng.standard_normal((37, 16)) * 3
    k = rng.standard_normal((37, 16)) * 3
    P = O.attention_weights(q, k, True)
    assert np.allclose(P.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(P[np.triu_indices(37, 1)] == 0.0)
    assert np.all(P[np.tril_indices(37)] > 0.0)


def test_softmax_shift_invariance_and_stability():
    # D1-2: subtracting the row maximum avoids overflow and changes nothing else.
    rng = np.random.default_rng(7)
    S = rng.standard_normal((4, 9))
    assert np.allclose(O.softmax_rows(S + 1234.5), O.softmax_rows(S), atol=1e-15)
    big = O.softmax_rows(S * 1e4)
    assert np.all(np.isfinite(big)) and np.allclose(big.sum(1), 1.0)


def test_first_row_equals_v0_and_equal_keys_give_prefix_means():
    rng = np.random.default_rng(8)
    T, H, G, d = 19, 4, 2, 8
    q = rng.standard_normal((T, H, d))
    k = np.tile(rng.standard_normal((1, G, d)), (T, 1, 1))
    v = rng.standard_normal((T, G, d))
    out = O.attend(q, k, v, causal=True)
    h = H // G
    for i in range(H):
        assert np.array_equal(out[0, i], v[0, i // h])
        prefix_mean = np.cumsum(v[:, i // h], axis=0) / np.arange(1, T + 1)[:, None]
        assert np.allclose(out[:, i], prefix_mean, atol=1e-14)


def _torch_sdpa(q, k, v, causal):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    Qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    Kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    Vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    o = F.scaled_dot_product_attention(Qt, Kt, Vt, is_causal=causal)
    return o[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("H,G", [(8, 8), (8, 1), (8, 2), (16, 8), (6, 3)])
@pytest.mark.parametrize("causal", [True, False])
def test_gqa_equals_mha_with_repeat_interleaved_kv(H, G, causal):
    # Qwen3 architecture 3.1.2: GQA is MHA after repeating each K/V head h times.
    # G = H is per-head MHA, G = 1 is MQA (nano-vllm "Qwen3" page, MHA/MQA/GQA).
    rng = np.random.default_rng(9 + H + G)
    T, d = 23, 16
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, G, d))
    v = rng.standard_normal((T, G, d))
    h = H // G
    want = _torch_sdpa(q, np.repeat(k, h, axis=1), np.repeat(v, h, axis=1), causal)
    got = O.attend(q, k, v, causal)
    assert np.allclose(got, want, atol=1e-13)
    if G == H:  # independent single-head attention per head
        for i in range(H):
            one = O.attend(q[:, i:i + 1], k[:, i:i + 1], v[:, i:i + 1], causal)
            assert np.allclose(got[:, i:i + 1], one, atol=1e-15)
    if G == 1:  # every head against the single shared K/V head
        for i in range(H):
            one = O.attend(q[:, i:i + 1], k, v, causal)
            assert np.allclose(got[:, i:i + 1], one, atol=1e-15)


def test_head_to_group_is_floor_not_modulo():
    # With distinct groups, query head i must use KV head floor(i / h): head 1 of H=4, G=2
    # belongs to group 0. The modulo mapping would pair it with group 1.
    rng = np.random.default_rng(10)
    T, d = 5, 4
    q = rng.standard_normal((T, 4, d))
    k = rng.standard_normal((T, 2, d))
    v = rng.standard_normal((T, 2, d))
    out = O.attend(q, k, v, True)
    one = O.attend(q[:, 1:2], k[:, 0:1], v[:, 0:1], True)
    assert np.allclose(out[:, 1:2], one, atol=1e-15)
    wrong = O.attend(q[:, 1:2], k[:, 1:2], v[:, 1:2], True)
    assert not np.allclose(out[:, 1:2], wrong, atol=1e-3)


# ============================================================================ whole path vs brute force
def _tiny_shapes():
    for H in range(1, 9):
        for G in range(1, H + 1):
            if H % G == 0:
                yield H, G


@pytest.mark.parametrize("H,G", list(_tiny_shapes()))
def test_prefill_matches_brute_force(H, G):
    rng = np.random.default_rng(100 * H + G)
    for d, T, causal in [(2, 3, True), (4, 6, False), (8, 5, True)]:
        q = rng.standard_normal((T, H, d))
        k = rng.standard_normal((T, G, d))
        v = rng.standard_normal((T, G, d))
        gq = rng.uniform(0.5, 1.5, d)
        gk = rng.uniform(0.5, 1.5, d)
        pos = rng.integers(0, 50, T)
        eps, theta = 1e-3, 1e4
        want = brute.gqa_prefill(q.tolist(), k.tolist(), v.tolist(), pos.tolist(), gq.tolist(),
                                 gk.tolist(), eps, theta, causal)
        got = O.prefill(q, k, v, pos, np.array([0, T]), gq, gk, eps, theta, causal)
        assert np.allclose(got, np.array(want), atol=1e-12, rtol=0)


def test_value_is_not_normalised_or_rotated():
    # Qwen3 series 1, D2-2: V gets neither QK-Norm nor RoPE. With equal keys the output is
    # a prefix mean of the raw V rows, whatever gamma and positions are.
    rng = np.random.default_rng(11)
    T, H, G, d = 7, 4, 2, 8
    q = rng.standard_normal((T, H, d))
    k = np.tile(rng.standard_normal((1, G, d)), (T, 1, 1))
    v = rng.standard_normal((T, G, d)) * 5
    out = O.prefill(q, k, v, np.zeros(T, int), np.array([0, T]), rng.uniform(0.5, 1.5, d),
                    rng.uniform(0.5, 1.5, d), 1e-6, 1e6, True)
    prefix_mean = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None, None]
    assert np.allclose(out[:, ::2], prefix_mean, atol=1e-13)


# ============================================================================ packing, rows, decode
def _case(rng, lengths, H=4, G=2, d=8):
    N = int(sum(lengths))
    q = rng.standard_normal((N, H, d))
    k = rng.standard_normal((N, G, d))
    v = rng.standard_normal((N, G, d))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    pos = np.concatenate([np.arange(t) for t in lengths]) if N else np.zeros(0, int)
    return q, k, v, cu, pos, rng.uniform(0.5, 1.5, d), rng.uniform(0.5, 1.5, d)


def test_packed_equals_separate_sequences():
    rng = np.random.default_rng(12)
    lengths = [5, 0, 9, 1, 3]
    q, k, v, cu, pos, gq, gk = _case(rng, lengths)
    out = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6)
    for b, t in enumerate(lengths):
        s = cu[b]
        if t == 0:
            continue
        one = brute.gqa_prefill(q[s:s + t].tolist(), k[s:s + t].tolist(), v[s:s + t].tolist(),
                                list(range(t)), gq.tolist(), gk.tolist(), 1e-6, 1e6, True)
        assert np.allclose(out[s:s + t], np.array(one), atol=1e-12)


def test_prefill_rows_equal_full_prefill():
    rng = np.random.default_rng(13)
    q, k, v, cu, pos, gq, gk = _case(rng, [6, 11, 4], H=6, G=3)
    full = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6)
    rows = [0, 5, 6, 7, 12, 16, 17, 20]
    got = O.prefill_rows(q, k, v, pos, cu, rows, gq, gk, 1e-6, 1e6)
    assert np.allclose(got, full[rows], atol=1e-13)


def test_causality_future_tokens_do_not_matter():
    rng = np.random.default_rng(14)
    q, k, v, cu, pos, gq, gk = _case(rng, [12])
    out = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[8:] += 3.0
    k2[8:] -= 2.0
    v2[8:] *= 7.0
    out2 = O.prefill(q2, k2, v2, pos, cu, gq, gk, 1e-6, 1e6)
    assert np.array_equal(out[:8], out2[:8])


def test_decode_equals_last_prefill_row():
    # Qwen3 series 1, D2-3: decode feeds one token that attends to every cached row, its own
    # K/V written first. The same tokens through prefill give the same last row.
    rng = np.random.default_rng(15)
    L, H, G, d = 13, 8, 2, 16
    q, k, v, cu, pos, gq, gk = _case(rng, [L], H=H, G=G, d=d)
    full = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6)
    _, kt = O.qk_norm_rope(q, k, pos, gq, gk, 1e-6, 1e6)
    k_cache = np.zeros((L + 3, G, d))
    v_cache = np.zeros((L + 3, G, d))
    k_cache[:L - 1] = kt[:L - 1]
    v_cache[:L - 1] = v[:L - 1]
    out, ks, vs = O.decode_one(q[L - 1], k_cache, v_cache, L, gq, gk, 1e-6, 1e6,
                               k_new=k[L - 1], v_new=v[L - 1])
    assert np.allclose(out, full[L - 1], atol=1e-13)
    assert np.allclose(ks, kt[L - 1], atol=1e-14) and np.array_equal(vs, v[L - 1])
    # without an append the cache slot is used as it stands
    k_cache[L - 1] = kt[L - 1]
    v_cache[L - 1] = v[L - 1]
    out2, _, _ = O.decode_one(q[L - 1], k_cache, v_cache, L, gq, gk, 1e-6, 1e6)
    assert np.allclose(out2, full[L - 1], atol=1e-13)


def test_decode_empty_sequence_is_zero():
    out, _, _ = O.decode_one(np.ones((4, 8)), np.ones((3, 2, 8)), np.ones((3, 2, 8)), 0,
                             None, None, 1e-6, 1e6)
    assert np.array_equal(out, np.zeros((4, 8)))


def test_peaky_softmax_stays_finite():
    # Qwen3 series 1, D1-4 Q8: scaling Q up drives each row towards one-hot.
    rng = np.random.default_rng(16)
    q, k, v, cu, pos, gq, gk = _case(rng, [30], H=2, G=1, d=16)
    out = O.prefill(q, k, v, pos, cu, gq * 40, gk * 40, 1e-6, 1e6)
    assert np.all(np.isfinite(out))
    qt, kt = O.qk_norm_rope(q, k, pos, gq * 40, gk * 40, 1e-6, 1e6)
    for r in (5, 17, 29):
        P = O.attention_weights(qt[:r + 1, 0], kt[:r + 1, 0], True)[-1]
        assert P.max() > 0.999
        assert np.allclose(out[r, 0], v[int(np.argmax(P)), 0], atol=1e-2)


# ============================================================================ cached prefill
def _cache_from_prefix(q, k, v, pos, gq, gk, past, max_seq):
    """Cache rows of a prefix: K after the prologue (as a layer stores it), raw V."""
    _, kt = O.qk_norm_rope(q[:past], k[:past], pos[:past], gq, gk, 1e-6, 1e6)
    G, d = k.shape[1], k.shape[2]
    kc = np.zeros((1, max_seq, G, d))
    vc = np.zeros((1, max_seq, G, d))
    kc[0, :past] = kt
    vc[0, :past] = v[:past]
    return kc, vc


@pytest.mark.parametrize("past,T", [(0, 9), (5, 1), (7, 6), (20, 13)])
def test_cached_prefill_equals_full_prefill(past, T):
    # Qwen3 series 1, D2-3: chunked prefill over a cache gives the same attention as one
    # prefill over the whole sequence (the cache holds what the earlier tokens produced).
    rng = np.random.default_rng(200 + past + T)
    L, H, G, d = past + T, 6, 2, 8
    q, k, v, cu, pos, gq, gk = _case(rng, [L], H=H, G=G, d=d)
    pos = np.arange(L)
    full = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6)
    kc, vc = _cache_from_prefix(q, k, v, pos, gq, gk, past, L + 4)
    out, kc2, vc2 = O.prefill_cached(q[past:], k[past:], v[past:], kc, vc, [past],
                                     np.array([0, T]), gq, gk, 1e-6, 1e6)
    assert np.allclose(out, full[past:], atol=1e-12, rtol=0)
    _, kt = O.qk_norm_rope(q, k, pos, gq, gk, 1e-6, 1e6)
    assert np.allclose(kc2[0, :L], kt, atol=1e-13) and np.array_equal(vc2[0, :L], v)
    assert np.array_equal(kc2[0, L:], kc[0, L:])  # rows past the chunk untouched


def test_cached_prefill_one_token_is_decode():
    rng = np.random.default_rng(210)
    L, H, G, d = 11, 4, 2, 8
    q, k, v, cu, pos, gq, gk = _case(rng, [L], H=H, G=G, d=d)
    pos = np.arange(L)
    kc, vc = _cache_from_prefix(q, k, v, pos, gq, gk, L - 1, L + 2)
    out, _, _ = O.prefill_cached(q[L - 1:], k[L - 1:], v[L - 1:], kc, vc, [L - 1],
                                 np.array([0, 1]), gq, gk, 1e-6, 1e6)
    dec, _, _ = O.decode_one(q[L - 1], kc[0], vc[0], L, gq, gk, 1e-6, 1e6, k_new=k[L - 1],
                             v_new=v[L - 1])
    assert np.allclose(out[0], dec, atol=1e-13)


def test_cached_prefill_matches_brute_force_and_packs():
    rng = np.random.default_rng(220)
    H, G, d = 4, 2, 4
    pasts, lens = [3, 0, 6], [2, 4, 0]
    N, max_seq = sum(lens), 12
    q = rng.standard_normal((N, H, d))
    k = rng.standard_normal((N, G, d))
    v = rng.standard_normal((N, G, d))
    kc = rng.standard_normal((3, max_seq, G, d))  # any cache contents
    vc = rng.standard_normal((3, max_seq, G, d))
    gq = rng.uniform(0.5, 1.5, d)
    gk = rng.uniform(0.5, 1.5, d)
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, kc2, _ = O.prefill_cached(q, k, v, kc, vc, pasts, cu, gq, gk, 1e-3, 1e4)
    for b in range(3):
        s, e = cu[b], cu[b + 1]
        if e == s:
            assert np.array_equal(kc2[b], kc[b])
            continue
        want = brute.gqa_prefill_cached(q[s:e].tolist(), k[s:e].tolist(), v[s:e].tolist(),
                                        kc[b].tolist(), vc[b].tolist(), pasts[b], gq.tolist(),
                                        gk.tolist(), 1e-3, 1e4)
        assert np.allclose(out[s:e], np.array(want), atol=1e-12, rtol=0)


def test_cached_prefill_without_cache_is_prefill():
    rng = np.random.default_rng(230)
    q, k, v, cu, pos, gq, gk = _case(rng, [7, 12], H=4, G=4, d=8)
    pos = np.concatenate([np.arange(7), np.arange(12)])
    want = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6)
    kc = np.zeros((2, 16, 4, 8))
    out, _, _ = O.prefill_cached(q, k, v, kc, kc, [0, 0], cu, gq, gk, 1e-6, 1e6)
    assert np.allclose(out, want, atol=1e-13)



def test_decode_steps_equal_a_cached_chunk_and_brute_force():
    # S decode steps with known inputs see exactly what a causal chunk of S new tokens sees
    # (step s = new token s at slot past + s); checked against prefill_cached and against the
    # pure-Python brute force, outputs and appended cache rows.
    rng = np.random.default_rng(240)
    S, B, H, G, d, max_seq = 5, 3, 6, 2, 8, 16
    pasts = [0, 4, 9]
    q = rng.standard_normal((S, B, H, d))
    k = rng.standard_normal((S, B, G, d))
    v = rng.standard_normal((S, B, G, d))
    kc = rng.standard_normal((B, max_seq, G, d))
    vc = rng.standard_normal((B, max_seq, G, d))
    gq, gk = rng.uniform(0.5, 1.5, d), rng.uniform(0.5, 1.5, d)
    out, kc2, vc2 = O.decode_steps(q, k, v, kc, vc, pasts, gq, gk, 1e-6, 1e6)
    # the chunk view: sequence-major packing of the same tokens
    qp = q.transpose(1, 0, 2, 3).reshape(B * S, H, d)
    kp = k.transpose(1, 0, 2, 3).reshape(B * S, G, d)
    vp = v.transpose(1, 0, 2, 3).reshape(B * S, G, d)
    cu = np.arange(B + 1) * S
    ch, kc3, vc3 = O.prefill_cached(qp, kp, vp, kc, vc, pasts, cu, gq, gk, 1e-6, 1e6)
    assert np.allclose(out.transpose(1, 0, 2, 3).reshape(B * S, H, d), ch, atol=1e-12, rtol=0)
    assert np.allclose(kc2, kc3, atol=1e-14) and np.array_equal(vc2, vc3)
    for b in range(B):
        want = brute.gqa_prefill_cached(q[:, b].tolist(), k[:, b].tolist(), v[:, b].tolist(),
                                        kc[b].tolist(), vc[b].tolist(), pasts[b], gq.tolist(),
                                        gk.tolist(), 1e-6, 1e6)
        assert np.allclose(out[:, b], np.array(want), atol=1e-12, rtol=0)
        assert np.array_equal(kc2[b, pasts[b] + S:], kc[b, pasts[b] + S:])  # untouched


def test_decode_steps_first_token_sees_itself():
    # An empty sequence's first step has one key, its own: every head returns its V row.
    rng = np.random.default_rng(250)
    S, B, H, G, d = 2, 2, 4, 2, 8
    q = rng.standard_normal((S, B, H, d))
    k = rng.standard_normal((S, B, G, d))
    v = rng.standard_normal((S, B, G, d))
    kc = np.zeros((B, 4, G, d))
    out, _, vc2 = O.decode_steps(q, k, v, kc, kc.copy(), [0, 0], None, None, 1e-6, 1e6)
    for b in range(B):
        for i in range(H):
            assert np.allclose(out[0, b, i], v[0, b, i // 2], atol=1e-15)
    assert np.array_equal(vc2[:, :2], v.transpose(1, 0, 2, 3))


# ----------------------------------------------------------------------------- mask variants
def _mask_case(rng, T, H=4, G=2, d=8):
    q, k, v, cu, pos, gq, gk = _case(rng, [T], H=H, G=G, d=d)
    return q, k, v, cu, np.arange(T), gq, gk


@pytest.mark.parametrize("W", [12, 13, 40])
def test_window_at_least_the_sequence_is_plain_causal(W):
    rng = np.random.default_rng(300 + W)
    q, k, v, cu, pos, gq, gk = _mask_case(rng, 12)
    a = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6, window=W)
    b = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6)
    assert np.array_equal(a, b)


def test_window_one_returns_own_value():
    # one visible key (itself): weight 1 on the token's own V row, for every head
    rng = np.random.default_rng(310)
    q, k, v, cu, pos, gq, gk = _mask_case(rng, 9, H=6, G=3)
    out = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6, window=1)
    assert np.allclose(out, np.repeat(v, 2, axis=1), atol=1e-15)


@pytest.mark.parametrize("W", [2, 3, 5])
def test_window_is_prefill_of_the_window_slice(W):
    # row t sees exactly tokens t-W+1..t: the last row of a plain causal prefill of that
    # slice (positions kept), and the brute force with an explicit window test
    rng = np.random.default_rng(320 + W)
    T = 11
    q, k, v, cu, pos, gq, gk = _mask_case(rng, T)
    out = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6, window=W)
    for t in range(T):
        lo = max(0, t - W + 1)
        part = O.prefill(q[lo:t + 1], k[lo:t + 1], v[lo:t + 1], pos[lo:t + 1],
                         np.array([0, t + 1 - lo]), gq, gk, 1e-6, 1e6)
        assert np.allclose(out[t], part[-1], atol=1e-12, rtol=0)
    want = brute.gqa_prefill(q.tolist(), k.tolist(), v.tolist(), list(range(T)), gq.tolist(),
                             gk.tolist(), 1e-6, 1e6, visible=lambda r, c: r - W < c <= r)
    assert np.allclose(out, np.array(want), atol=1e-12, rtol=0)


def test_block_mask_all_set_is_plain_causal():
    rng = np.random.default_rng(330)
    q, k, v, cu, pos, gq, gk = _mask_case(rng, 14)
    bm = np.ones((4, 4), bool)
    a = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6, block_mask=bm, block=4)
    b = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6)
    assert np.array_equal(a, b)


def test_block_mask_empty_is_blockwise_causal():
    # nothing set: only the diagonal blocks remain (always kept), so attention restarts at
    # every block boundary: a packed prefill whose sequences are the blocks, positions kept
    rng = np.random.default_rng(340)
    T, blk = 14, 4
    q, k, v, cu, pos, gq, gk = _mask_case(rng, T)
    out = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6, block_mask=np.zeros((4, 4), bool),
                    block=blk)
    cut = np.array([0, 4, 8, 12, 14])
    want = O.prefill(q, k, v, pos, cut, gq, gk, 1e-6, 1e6)
    assert np.allclose(out, want, atol=1e-13, rtol=0)


def test_block_mask_and_window_match_brute_force():
    rng = np.random.default_rng(350)
    T, blk, W = 13, 3, 7
    q, k, v, cu, pos, gq, gk = _mask_case(rng, T)
    nb = -(-T // blk)
    bm = rng.random((nb, nb)) < 0.4
    for causal, win in ((True, 0), (True, W), (False, 0)):
        out = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6, causal=causal, window=win,
                        block_mask=bm, block=blk)

        def vis(r, c, causal=causal, win=win):
            if causal and c > r:
                return False
            if win and c <= r - win:
                return False
            return bool(bm[r // blk][c // blk]) or r // blk == c // blk

        want = brute.gqa_prefill(q.tolist(), k.tolist(), v.tolist(), list(range(T)),
                                 gq.tolist(), gk.tolist(), 1e-6, 1e6, visible=vis)
        assert np.allclose(out, np.array(want), atol=1e-12, rtol=0), (causal, win)
        rows = [0, 2, 3, 7, 12]
        got = O.prefill_rows(q, k, v, pos, cu, rows, gq, gk, 1e-6, 1e6, causal=causal,
                             window=win, block_mask=bm, block=blk)
        assert np.allclose(got, out[rows], atol=1e-13, rtol=0)


def test_masks_in_cached_prefill_count_cache_rows():
    # the same masks over a cached prefix + chunk equal the one-shot masked prefill's rows
    rng = np.random.default_rng(360)
    T, past, blk, W = 15, 6, 4, 5
    q, k, v, cu, pos, gq, gk = _mask_case(rng, T)
    bm = rng.random((4, 4)) < 0.5
    full = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6, window=W, block_mask=bm, block=blk)
    kc, vc = _cache_from_prefix(q, k, v, pos, gq, gk, past, T + 2)
    out, _, _ = O.prefill_cached(q[past:], k[past:], v[past:], kc, vc, [past],
                                 np.array([0, T - past]), gq, gk, 1e-6, 1e6, window=W,
                                 block_mask=bm, block=blk)
    assert np.allclose(out, full[past:], atol=1e-12, rtol=0)


# ----------------------------------------------------------------------------- RoPE frequency variants
def test_frequency_table_of_the_base_is_the_base_path():
    rng = np.random.default_rng(400)
    q, k, v, cu, pos, gq, gk = _case(rng, [9], H=4, G=2, d=8)
    a = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, 1e6)
    b = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, O.rope_inv_freq(8, 1e6))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("alpha", [2.0, 4.0, 3.5])
def test_linear_interpolation_divides_positions(alpha):
    # summary §4.2: the position index divided by alpha; as a table, every frequency / alpha
    rng = np.random.default_rng(410)
    q, k, v, cu, pos, gq, gk = _case(rng, [11], H=4, G=2, d=8)
    pos = np.arange(11) * 3 + 5
    a = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, O.inv_freq_linear(8, 1e4, alpha))
    b = O.prefill(q, k, v, pos / alpha, cu, gq, gk, 1e-6, 1e4)
    assert np.allclose(a, b, atol=1e-12, rtol=0)


def test_yarn_page_formula_hand_values():
    # d = 8, theta = 1e4: omega = (1, 0.1, 0.01, 0.001); train 2048 -> infer 8192, scale 1:
    # s = log2(4) = 2, factors 1 - 2 * (0, 2, 4, 6) / 8 = (1, 0.5, 0, -0.5)
    w = O.inv_freq_yarn_page(8, 1e4, 2048, 8192)
    assert np.allclose(w, [1.0, 0.05, 0.0, -0.0005], atol=1e-15, rtol=1e-12)
    w = O.inv_freq_yarn_page(8, 1e4, 2048, 4096, scale=0.5)  # s = 0.5
    assert np.allclose(w, [1.0, 0.1 * 0.875, 0.01 * 0.75, 0.001 * 0.625], rtol=1e-12)
    assert np.array_equal(O.inv_freq_yarn_page(8, 1e4, 4096, 4096), O.rope_inv_freq(8, 1e4))


def test_ntk_base_change_keeps_highest_divides_lowest():
    for d, alpha in ((8, 4.0), (128, 2.0), (64, 8.0)):
        w0 = O.rope_inv_freq(d, 1e6)
        w1 = O.rope_inv_freq(d, O.ntk_theta(1e6, alpha, d))
        assert w1[0] == w0[0] == 1.0
        assert np.isclose(w1[-1], w0[-1] / alpha, rtol=1e-12)


def test_frequency_tables_match_brute_force():
    # a scaled table through prefill and decode against the brute force with explicit R(pos)
    rng = np.random.default_rng(420)
    T, H, G, d = 7, 4, 2, 8
    q, k, v, cu, pos, gq, gk = _case(rng, [T], H=H, G=G, d=d)
    pos = np.array([0, 3, 4, 9, 10, 100, 1000])
    for w in (O.inv_freq_yarn_page(d, 1e4, 2048, 8192), O.inv_freq_linear(d, 1e4, 4.0)):
        out = O.prefill(q, k, v, pos, cu, gq, gk, 1e-6, w)
        want = brute.gqa_prefill(q.tolist(), k.tolist(), v.tolist(), pos.tolist(), gq.tolist(),
                                 gk.tolist(), 1e-6, w.tolist())
        assert np.allclose(out, np.array(want), atol=1e-12, rtol=0)
        kc, vc = _cache_from_prefix(q, k, v, pos, gq, gk, 0, T)  # empty cache
        _, kt = O.qk_norm_rope(q[:T - 1], k[:T - 1], pos[:T - 1], gq, gk, 1e-6, w)
        kc[0, :T - 1] = kt
        vc[0, :T - 1] = v[:T - 1]
        dec, _, _ = O.decode_one(q[T - 1], kc[0], vc[0], T, gq, gk, 1e-6, w, position=pos[T - 1],
                                 k_new=k[T - 1], v_new=v[T - 1])
        assert np.allclose(dec, out[T - 1], atol=1e-12, rtol=0)
