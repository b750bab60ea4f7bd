"""Pure-Python brute force (lists, ``math``) for tiny causal GQA cases.

TEST INFRASTRUCTURE: used only by the tests to check the NumPy oracle on tiny inputs. It
shares no code with ``gqa_oracle`` and builds each step the long way:

* RMSNorm element by element (zhanghao0806.com "Qwen3系列1-理论基础&真实结构", D2-1).
* RoPE as the explicit block-diagonal matrix R(pos) of D2-2, multiplied into the vector;
  the frequency of block j is theta^(-2j/d) (ewbang.com "深入剖析Qwen3模型架构", 3.4.1).
* GQA by first repeating every K/V head h times along the head axis (the repeat-interleave
  of the same article, 3.1.2), then plain multi-head attention with explicit loops, the
  causal mask as -inf before the softmax (Qwen3 series 1, D1-5) and the max-subtracted
  softmax (D1-2).
"""
from __future__ import annotations

import math


def rmsnorm_vec(x, gamma, eps):
    if gamma is None:
        return list(x)
    ms = sum(xi * xi for xi in x) / len(x)
    r = math.sqrt(ms + eps)
    return [g * xi / r for g, xi in zip(gamma, x)]


def rope_matrix(pos, d, theta):
    """The d x d block-diagonal rotation matrix R(pos). ``theta`` is the base, or a list of
    the d/2 block frequencies."""
    R = [[0.0] * d for _ in range(d)]
    for j in range(d // 2):
        w = theta[j] if isinstance(theta, (list, tuple)) else theta ** (-2.0 * j / d)
        a = pos * w
        c, s = math.cos(a), math.sin(a)
        R[2 * j][2 * j] = c
        R[2 * j][2 * j + 1] = -s
        R[2 * j + 1][2 * j] = s
        R[2 * j + 1][2 * j + 1] = c
    return R


def matvec(M, x):
    return [sum(M[r][c] * x[c] for c in range(len(x))) for r in range(len(M))]


def prologue_vec(x, pos, gamma, eps, theta):
    y = rmsnorm_vec(x, gamma, eps)
    if not isinstance(theta, (list, tuple)) and theta == 0:
        return y
    return matvec(rope_matrix(pos, len(x), theta), y)


def repeat_interleave_heads(x, h):
    """x[t][g] -> x[t][i] with i = g*h + r, r = 0..h-1."""
    return [[row[g] for g in range(len(row)) for _ in range(h)] for row in x]


def mha(q, k, v, causal, scale, visible=None):
    """Plain multi-head attention: q, k, v are [T][H][d] nested lists. ``visible(r, c)``,
    when given, decides alone which key c query r sees."""
    T = len(q)
    H = len(q[0])
    d = len(q[0][0])
    out = [[[0.0] * d for _ in range(H)] for _ in range(T)]
    for i in range(H):
        for r in range(T):
            scores = []
            for c in range(T):
                hidden = (not visible(r, c)) if visible else (causal and c > r)
                if hidden:
                    scores.append(-math.inf)
                else:
                    scores.append(sum(q[r][i][e] * k[c][i][e] for e in range(d)) * scale)
            m = max(scores)
            ex = [math.exp(s - m) if s != -math.inf else 0.0 for s in scores]
            z = sum(ex)
            for e in range(d):
                out[r][i][e] = sum(ex[c] / z * v[c][i][e] for c in range(T))
    return out


def gqa_prefill(q, k, v, positions, q_norm_w, k_norm_w, eps, theta, causal=True, scale=None,
                visible=None):
    """One sequence: q [T][H][d], k/v [T][G][d] nested lists of floats. ``visible(r, c)``
    replaces the causal test when given."""
    T = len(q)
    H = len(q[0])
    G = len(k[0])
    d = len(q[0][0])
    h = H // G
    qt = [[prologue_vec(q[t][i], positions[t], q_norm_w, eps, theta) for i in range(H)]
          for t in range(T)]
    kt = [[prologue_vec(k[t][g], positions[t], k_norm_w, eps, theta) for g in range(G)]
          for t in range(T)]
    kr = repeat_interleave_heads(kt, h)
    vr = repeat_interleave_heads(v, h)
    sc = scale if scale else 1.0 / math.sqrt(d)
    return mha(qt, kr, vr, causal, sc, visible)


def gqa_prefill_cached(q, k, v, k_cache, v_cache, past, q_norm_w, k_norm_w, eps, theta,
                       scale=None):
    """One sequence with ``past`` cached tokens (k_cache rows already after the prologue):
    the new tokens q/k/v [T][.][d] sit at positions past + t; new token t attends to cache
    rows 0..past-1 and new tokens 0..t, with explicit loops."""
    T = len(q)
    H = len(q[0])
    G = len(k[0])
    d = len(q[0][0])
    h = H // G
    sc = scale if scale else 1.0 / math.sqrt(d)
    qt = [[prologue_vec(q[t][i], past + t, q_norm_w, eps, theta) for i in range(H)]
          for t in range(T)]
    kt = [[prologue_vec(k[t][g], past + t, k_norm_w, eps, theta) for g in range(G)]
          for t in range(T)]
    keys = [list(map(list, k_cache[j])) for j in range(past)] + kt
    vals = [list(map(list, v_cache[j])) for j in range(past)] + [list(map(list, v[t])) for t in range(T)]
    out = [[[0.0] * d for _ in range(H)] for _ in range(T)]
    for t in range(T):
        for i in range(H):
            g = i // h
            scores = [sum(qt[t][i][e] * keys[j][g][e] for e in range(d)) * sc
                      for j in range(past + t + 1)]
            m = max(scores)
            ex = [math.exp(x - m) for x in scores]
            z = sum(ex)
            for e in range(d):
                out[t][i][e] = sum(ex[j] / z * vals[j][g][e] for j in range(past + t + 1))
    return out

