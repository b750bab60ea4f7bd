"""Plain, slow, float64 CPU oracle for causal grouped-query attention with QK-RMSNorm + RoPE.

TEST INFRASTRUCTURE. Only the tests, the smoke check of the graft entry module and the CPU
baseline leg of the benchmark may import this module. The product path (the HIP library and
its Python binding) never calls it, and this module imports nothing from that path.

Every function is the plain definition written out in NumPy float64, following the pages:

* zhanghao0806.com, "Qwen3系列1-理论基础&真实结构" (below: "Qwen3 series 1"), sections D1-2
  (stable softmax), D1-4 (scaled dot-product attention), D1-5 (causal mask), D2-1 (RMSNorm),
  D2-2 (QK-Norm, then RoPE; the block-diagonal rotation matrix R(pos)), D2-3 (GQA groups,
  KV cache, prefill and decode).
* ewbang.com, "深入剖析Qwen3模型架构" (below: "Qwen3 architecture"), section 3.1.2 (GQA module
  that repeat-interleaves K/V heads; RoPE on adjacent element pairs) and section 3.4.1 (RoPE
  inverse frequencies base^(-2j/d) with base 1e6).
* selfknow.cn, nano-vllm "Qwen3" page, "Attention 的 Forward 流程" steps (4) q_norm/k_norm,
  (5) rotary embedding, (6) attention reading and writing the KV cache.

Readings taken where the pages are silent (each also listed in the design notes):
norm before RoPE; RMSNorm with a learned weight (not L2 normalisation); eps inside the square
root; one weight vector shared by all Q heads and one by all K heads; rotation of adjacent
pairs (2j, 2j+1), counter-clockwise; angles in float64; positions feed RoPE only while the
causal mask uses the index inside the sequence; query head i uses KV head floor(i / h);
decode's seq_lens[b] counts the new token, whose K/V are in the cache before attention.

Every function here is pinned by the ``-m "not gpu"`` tests (closed forms, the pages'
properties, brute force on tiny inputs and a library special case).
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------- RMSNorm
def rms_norm(x: np.ndarray, gamma: np.ndarray | None, eps: float) -> np.ndarray:
    """gamma * x / sqrt(mean(x^2) + eps) over the last axis.

    Qwen3 series 1, D2-1 (RMSNorm formula: no centring, eps inside the root, learned gamma);
    D2-2 (applied per head to Q and to K after projection; one gamma for all Q heads and one
    for all K heads). ``gamma=None`` skips the norm."""
    x = np.asarray(x, dtype=np.float64)
    if gamma is None:
        return x.copy()
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(gamma, dtype=np.float64) * (x / np.sqrt(ms + eps))


# ----------------------------------------------------------------------------- RoPE
def rope_inv_freq(d: int, theta: float) -> np.ndarray:
    """omega_j = theta^(-2j/d), j = 0..d/2-1 (Qwen3 architecture, 3.4.1; base 1e6)."""
    j = np.arange(d // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * j / d)


def inv_freq_of(d: int, theta) -> np.ndarray:
    """The d/2 RoPE frequencies: ``theta`` is the base (``rope_inv_freq``) or already a table
    of d/2 frequencies (a scaled variant below)."""
    if np.ndim(theta) == 0:
        return rope_inv_freq(d, float(theta))
    w = np.asarray(theta, dtype=np.float64)
    if w.shape != (d // 2,):
        raise ValueError("a frequency table needs d/2 entries")
    return w


def rope(x: np.ndarray, positions: np.ndarray, theta) -> np.ndarray:
    """Rotate each adjacent pair (x_2j, x_2j+1) of x[t, head, :] counter-clockwise by
    positions[t] * omega_j.

    Qwen3 series 1, D2-2 (R(pos) is block-diagonal with 2x2 rotation blocks
    [[cos, -sin], [sin, cos]] of angle pos*theta_j); Qwen3 architecture, 3.1.2 (pairs are
    the even/odd elements, rotated as a complex product). ``theta`` is the base (0 skips
    RoPE) or a table of the d/2 frequencies. Positions may be fractional."""
    x = np.asarray(x, dtype=np.float64)
    if np.ndim(theta) == 0 and theta == 0:
        return x.copy()
    d = x.shape[-1]
    phi = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq_of(d, theta)[None, :]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    a = x[..., 0::2]
    b = x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = a * c - b * s
    y[..., 1::2] = a * s + b * c
    return y


# Scaled frequency tables (each passed as ``theta`` wherever a base is taken).
def inv_freq_linear(d: int, theta: float, alpha: float) -> np.ndarray:
    """Linear position interpolation: every position index divided by the extension factor
    alpha (zizhi168.cn technical-report summary, §4.2), i.e. every frequency divided by it."""
    return rope_inv_freq(d, theta) / float(alpha)


def inv_freq_yarn_page(d: int, theta: float, train_len: int, infer_len: int,
                       scale: float = 1.0) -> np.ndarray:
    """The frequency scaling that Qwen3 architecture, 3.4.2 prints under the name YaRN: past
    the training length, s = scale * log2(infer_len / train_len) and omega_j is multiplied by
    1 - s * 2j / d; otherwise the frequencies are unchanged."""
    w = rope_inv_freq(d, theta)
    if infer_len > train_len:
        s = float(scale) * np.log(infer_len / train_len) / np.log(2.0)
        w = w * (1.0 - s * (2.0 * np.arange(d // 2, dtype=np.float64) / d))
    return w


def ntk_theta(theta: float, alpha: float, d: int) -> float:
    """NTK-aware scaling (summary, §4.2) read as a change of base: theta' = theta *
    alpha^(d / (d - 2)), which keeps the highest frequency and divides the lowest by alpha."""
    return float(theta) * float(alpha) ** (d / (d - 2.0))


def qk_norm_rope(q, k, positions, q_norm_w, k_norm_w, eps, theta):
    """Prologue: per-head RMSNorm of Q (gamma_q) and K (gamma_k), then RoPE at positions.

    nano-vllm "Qwen3" page, forward steps (4) then (5); Qwen3 series 1, D2-2. V is neither
    normalised nor rotated. q: [N, H, d], k: [N, G, d], positions: [N]."""
    qt = rope(rms_norm(q, q_norm_w, eps), positions, theta)
    kt = rope(rms_norm(k, k_norm_w, eps), positions, theta)
    return qt, kt


# ----------------------------------------------------------------------------- attention core
def _scale(d: int, scale: float | None) -> float:
    # Qwen3 series 1, D1-4: scores are divided by sqrt(d_k).
    return 1.0 / np.sqrt(d) if not scale else float(scale)


def softmax_rows(S: np.ndarray) -> np.ndarray:
    """Row softmax with the row maximum subtracted first (Qwen3 series 1, D1-2).
    Entries equal to -inf get weight exactly 0 (D1-5)."""
    m = np.max(S, axis=-1, keepdims=True)
    E = np.exp(S - m)
    return E / np.sum(E, axis=-1, keepdims=True)


def visible_keys(Tq: int, Tk: int, causal: bool, window: int = 0, block_mask=None,
                 block: int = 64, q_index=None) -> np.ndarray:
    """Boolean [Tq, Tk]: which keys each query row may see. Query row r sits at key index
    i = r + (Tk - Tq) (or i = q_index[r] when given); key index j.

    * causal: j <= i (Qwen3 series 1, D1-5).
    * window W > 0: also j > i - W, the W most recent keys including itself (zizhi168.cn
      technical-report summary, §3.1: local attention inside a 512-token window).
    * block_mask [n_blocks, n_blocks] of bools: also block_mask[i // block, j // block], with
      the diagonal block always kept so that every row sees itself (same section:
      block-sparse attention over 64-token blocks)."""
    if q_index is None:
        i = np.arange(Tq)[:, None] + (Tk - Tq)
    else:
        i = np.asarray(q_index, dtype=np.int64)[:, None]
    j = np.arange(Tk)[None, :]
    vis = np.ones((Tq, Tk), dtype=bool)
    if causal:
        vis &= j <= i
    if window:
        vis &= j > i - int(window)
    if block_mask is not None:
        bm = np.asarray(block_mask, dtype=bool)
        vis &= bm[i // block, j // block] | (i // block == j // block)
    return vis


def attention_weights(qt_i: np.ndarray, kt_g: np.ndarray, causal: bool, scale=None,
                      window: int = 0, block_mask=None, block: int = 64):
    """P = softmax(q k^T / sqrt(d) + M) for one query head against its KV head.

    Qwen3 series 1, D1-4 (formula softmax(QK^T/sqrt(d_k) + M)); D1-5 (M is -inf where the
    key index exceeds the query index). qt_i: [Tq, d], kt_g: [Tk, d]; query row r sits at
    key index r + (Tk - Tq). M is -inf wherever ``visible_keys`` says False."""
    Tq, d = qt_i.shape
    Tk = kt_g.shape[0]
    S = (qt_i @ kt_g.T) * _scale(d, scale)
    if causal or window or block_mask is not None:
        S = np.where(visible_keys(Tq, Tk, causal, window, block_mask, block), S, -np.inf)
    return softmax_rows(S)


def attend(qt: np.ndarray, kt: np.ndarray, v: np.ndarray, causal: bool, scale=None,
           window: int = 0, block_mask=None, block: int = 64):
    """Grouped-query attention over one sequence.

    qt: [T, H, d]; kt, v: [T, G, d]. Query head i uses KV head g = floor(i / h), h = H / G:
    the mapping of repeating every K/V head h times along the head axis (Qwen3 architecture,
    3.1.2; Qwen3 series 1, D2-3). Each head: P V with P from ``attention_weights``."""
    T, H, d = qt.shape
    G = kt.shape[1]
    if H % G:
        raise ValueError("H must be a multiple of G")
    h = H // G
    out = np.empty((T, H, d), dtype=np.float64)
    for i in range(H):
        g = i // h
        P = attention_weights(qt[:, i, :], kt[:, g, :], causal, scale, window, block_mask,
                              block)
        out[:, i, :] = P @ v[:, g, :]
    return out


# ----------------------------------------------------------------------------- prefill
def prefill(q, k, v, positions, cu_seqlens, q_norm_w, k_norm_w, eps, theta, causal=True,
            scale=None, window=0, block_mask=None, block=64):
    """Packed prefill: prologue on every token, then attention inside each sequence.

    q: [N, H, d]; k, v: [N, G, d]; positions: [N]; cu_seqlens: [B+1] offsets. The masks
    (causal, window, block_mask: ``visible_keys``) use the index inside the sequence;
    positions feed RoPE only. One block_mask serves every sequence."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    qt, kt = qk_norm_rope(q, k, positions, q_norm_w, k_norm_w, eps, theta)
    out = np.zeros_like(q)
    for b in range(len(cu_seqlens) - 1):
        s, e = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        if e > s:
            out[s:e] = attend(qt[s:e], kt[s:e], v[s:e], causal, scale, window, block_mask,
                              block)
    return out


def prefill_rows(q, k, v, positions, cu_seqlens, rows, q_norm_w, k_norm_w, eps, theta,
                 causal=True, scale=None, window=0, block_mask=None, block=64,
                 max_elems=1 << 26):
    """Selected output rows of ``prefill``: rows are packed token indices. Each row is the
    same definition evaluated for that query token alone: its full score row over the keys
    of its sequence, masked by ``visible_keys`` at its index, softmax, times V (Qwen3 series
    1, D1-4, D1-5, D1-2). The rows of one sequence are evaluated together as one matrix per
    KV head: S = Q~[rows, heads of g] K~_g^T, in batches of rows of at most ``max_elems``
    scores (rows are independent, so batching changes nothing). Returns [len(rows), H, d]."""
    rows = np.asarray(rows, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    H, d = q.shape[1], q.shape[2]
    G = k.shape[1]
    h = H // G
    out = np.empty((len(rows), H, d), dtype=np.float64)
    seq_of = np.searchsorted(cu, rows, side="right") - 1
    for b in np.unique(seq_of):
        s, e = int(cu[b]), int(cu[b + 1])
        sel = np.flatnonzero(seq_of == b)
        kt = rope(rms_norm(np.asarray(k[s:e], np.float64), k_norm_w, eps), positions[s:e],
                  theta)
        vb = np.asarray(v[s:e], np.float64)
        qt = rope(rms_norm(np.asarray(q[rows[sel]], np.float64), q_norm_w, eps),
                  np.asarray(positions)[rows[sel]], theta)
        r_in = rows[sel] - s  # index of each row inside its sequence
        Tk = e - s
        step = max(1, max_elems // max(1, h * Tk))
        for c0 in range(0, len(sel), step):
            c = slice(c0, c0 + step)
            vis = visible_keys(len(r_in[c]), Tk, causal, window, block_mask, block,
                               q_index=r_in[c])
            for g in range(G):
                Q = qt[c, g * h:(g + 1) * h, :].reshape(-1, d)  # [rows * h, d]
                S = (Q @ kt[:, g, :].T) * _scale(d, scale)
                S = np.where(np.repeat(vis, h, axis=0), S, -np.inf)
                P = softmax_rows(S)
                out[sel[c], g * h:(g + 1) * h, :] = (P @ vb[:, g, :]).reshape(-1, h, d)
    return out


# ----------------------------------------------------------------------------- decode
def decode_one(q_b, k_rows, v_rows, seq_len, q_norm_w, k_norm_w, eps, theta, position=None,
               k_new=None, v_new=None, scale=None):
    """Single-token decode of one sequence.

    q_b: [H, d] raw query of the new token; k_rows, v_rows: [>= seq_len, G, d] cache rows,
    K taken as already normalised and rotated (the cache holds post-prologue K and raw V,
    nano-vllm "Qwen3" page step (6) after (5)). The new token sits at slot p = seq_len - 1
    (or ``position``): if k_new/v_new [G, d] are given, RoPE(RMSNorm(k_new)) and v_new are
    placed there before attention (Qwen3 series 1, D2-3: each layer writes its K/V into the
    cache before computing attention). The single query sees every cached row 0..seq_len-1.
    Returns (out [H, d], k_slot, v_slot) where the slots are the appended rows or None."""
    L = int(seq_len)
    H, d = q_b.shape
    if L == 0:
        return np.zeros((H, d)), None, None
    slot = L - 1
    pos = slot if position is None else int(position)
    kc = np.array(k_rows[:L], dtype=np.float64)
    vc = np.array(v_rows[:L], dtype=np.float64)
    k_slot = v_slot = None
    if k_new is not None:
        k_slot = rope(rms_norm(np.asarray(k_new, np.float64)[None], k_norm_w, eps),
                      np.array([pos]), theta)[0]
        v_slot = np.asarray(v_new, np.float64)
        kc[slot] = k_slot
        vc[slot] = v_slot
    qt = rope(rms_norm(np.asarray(q_b, np.float64)[None], q_norm_w, eps), np.array([pos]),
              theta)[0]
    G = kc.shape[1]
    h = H // G
    out = np.empty((H, d))
    for i in range(H):
        g = i // h
        p = attention_weights(qt[i:i + 1], kc[:, g, :], False, scale)[0]
        out[i] = p @ vc[:, g, :]
    return out, k_slot, v_slot


# ----------------------------------------------------------------------------- decode loop
def decode_steps(q_steps, k_steps, v_steps, k_cache, v_cache, cache_lens, q_norm_w, k_norm_w,
                 eps, theta, scale=None):
    """S successive decode steps of B sequences: generation is one forward pass per new token,
    each seeing every earlier token (Qwen3 series 1, D1-1, Q2 and Q5: generate() is many
    forward() calls; D2-3: each step's K/V join the cache before its attention).

    q_steps [S, B, H, d], k_steps / v_steps [S, B, G, d]: the new token of sequence b at step s
    (raw). Sequence b starts with cache_lens[b] rows in k_cache / v_cache [B, max_seq, G, d]
    (K after the prologue, raw V); step s is ``decode_one`` with seq_len cache_lens[b] + s + 1,
    appending at slot cache_lens[b] + s. Returns (out [S, B, H, d], k_cache', v_cache')."""
    q_steps = np.asarray(q_steps, np.float64)
    S, B, H, d = q_steps.shape
    kc = np.array(k_cache, dtype=np.float64)
    vc = np.array(v_cache, dtype=np.float64)
    out = np.zeros((S, B, H, d))
    for s in range(S):
        for b in range(B):
            L = int(cache_lens[b]) + s + 1
            o, k_slot, v_slot = decode_one(q_steps[s, b], kc[b], vc[b], L, q_norm_w, k_norm_w,
                                           eps, theta, k_new=k_steps[s][b], v_new=v_steps[s][b],
                                           scale=scale)
            out[s, b] = o
            kc[b, L - 1] = k_slot
            vc[b, L - 1] = v_slot
    return out, kc, vc


# ----------------------------------------------------------------------------- cached prefill
def prefill_cached(q, k_new, v_new, k_cache, v_cache, cache_lens, cu_seqlens, q_norm_w,
                   k_norm_w, eps, theta, positions=None, causal=True, scale=None, window=0,
                   block_mask=None, block=64):
    """Chunked (multi-turn) prefill of new tokens against a KV cache.

    Sequence b has past = cache_lens[b] earlier tokens in the cache: k_cache[b, :past] holds
    their K after the prologue, v_cache[b, :past] their V (nano-vllm "Qwen3" page, step (6);
    Qwen3 series 1, D2-3: the cache keeps the K/V of every earlier token). Its new tokens are
    q/k_new/v_new[cu[b]:cu[b+1]] at positions past + t (or ``positions``). Each layer writes
    the new tokens' K/V into the cache before attention (D2-3), here at slots past + t, and
    new token t attends to keys 0 .. past + t (the causal mask of D1-5 with the query at key
    index past + t). ``window`` and ``block_mask`` (see ``visible_keys``) count key indices
    over the whole sequence, cache included. Returns (out [N, H, d], k_cache', v_cache') with
    the rows appended."""
    q = np.asarray(q, np.float64)
    k_new = np.asarray(k_new, np.float64)
    v_new = np.asarray(v_new, np.float64)
    kc = np.array(k_cache, dtype=np.float64)
    vc = np.array(v_cache, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = np.zeros_like(q)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        past = int(cache_lens[b])
        if e == s:
            continue
        pos = (past + np.arange(e - s)) if positions is None else np.asarray(positions)[s:e]
        qt, kt = qk_norm_rope(q[s:e], k_new[s:e], pos, q_norm_w, k_norm_w, eps, theta)
        kc[b, past:past + e - s] = kt
        vc[b, past:past + e - s] = v_new[s:e]
        kv_k = kc[b, :past + e - s]
        kv_v = vc[b, :past + e - s]
        H = q.shape[1]
        h = H // k_new.shape[1]
        for i in range(H):
            g = i // h
            P = attention_weights(qt[:, i, :], kv_k[:, g, :], causal, scale, window,
                                  block_mask, block)
            out[s:e, i, :] = P @ kv_v[:, g, :]
    return out, kc, vc

