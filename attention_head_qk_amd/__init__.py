"""Causal grouped-query attention with QK-RMSNorm + RoPE on MI355X (gfx950).

Thin torch-facing binding of libgqa.so (include/gqa.h): it checks shapes, passes
``tensor.data_ptr()`` values and the current torch stream to the C ABI, and allocates the
workspace and outputs with torch when the caller does not pass them. Every step of the
computation runs in the library's HIP kernels; nothing here computes attention, and there is
no fallback when the library is missing (importing raises).

    out = prefill(q, k, v)                       # q [B, T, H, d], k/v [B, T, G, d]
    out = prefill(q, k, v, cu_seqlens=cu, max_seqlen=Tmax)   # packed q [N, H, d]
    out = decode(q, k_cache, v_cache, seq_lens)  # q [B, H, d], caches [B, S, G, d]
    g = DecodeGraph(q, k_cache, v_cache, seq_lens, k_new, v_new); g.launch()  # per token
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import GqaError  # noqa: F401

_lib.load()  # fail at import, loudly, if the HIP library is not built

__all__ = ["prefill", "prefill_cached", "decode", "DecodeGraph", "qk_norm_rope", "workspace_bytes",
           "decode_split_keys", "pack_block_mask", "rope_freq_table", "GqaError"]

_DTYPES = {torch.float32: _lib.GQA_F32, torch.bfloat16: _lib.GQA_BF16}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _params(dtype, q_norm_w, k_norm_w, eps, theta, scale, stream, device, rope_inv_freq=None):
    p = _lib.default_params()
    if rope_inv_freq is not None:
        import numpy as np
        w = np.ascontiguousarray(np.asarray(rope_inv_freq, dtype=np.float64).ravel())
        p._freqs = w  # kept alive with the struct: the library reads it during the call
        p.rope_inv_freq = w.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    p.dtype = _DTYPES[dtype]
    p.q_norm_w = _ptr(_dev(q_norm_w, "q_norm_w", dtype))
    p.k_norm_w = _ptr(_dev(k_norm_w, "k_norm_w", dtype))
    p.eps = float(eps)
    p.rope_theta = float(theta)
    p.scale = float(scale)
    s = stream if stream is not None else torch.cuda.current_stream(device)
    p.stream = ctypes.c_void_p(s.cuda_stream)
    return p


def workspace_bytes(op: str, B: int, T_or_max_seq: int, H: int, G: int, d: int,
                    dtype=torch.bfloat16) -> int:
    code = {"prefill": _lib.GQA_OP_PREFILL, "decode": _lib.GQA_OP_DECODE}[op]
    return int(_lib.load().gqa_workspace_bytes(code, B, T_or_max_seq, H, G, d, _DTYPES[dtype]))


def decode_split_keys(B: int, H: int, G: int, max_seq: int) -> int:
    """Keys per split of the decode pass for this decode shape."""
    return int(_lib.load().gqa_decode_split_keys(B, H, G, max_seq))


def _prof(p, prof):
    """prof = (start, stop) torch.cuda.Event pair recorded around the main kernel."""
    if prof is None:
        return
    start, stop = prof
    for ev in (start, stop):
        if not ev.cuda_event:  # torch creates the HIP event on its first record
            ev.record()
    p.prof_start = ctypes.c_void_p(start.cuda_event)
    p.prof_stop = ctypes.c_void_p(stop.cuda_event)


def _workspace(ws, nbytes, device):
    if ws is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _dev(ws, "workspace")
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return ws


def rope_freq_table(d, theta=1e6, kind="base", alpha=1.0, train_len=None, infer_len=None,
                    scale=1.0):
    """The d/2 RoPE frequencies for ``rope_inv_freq`` (host, float64):
    base   omega_j = theta^(-2j/d);
    linear position interpolation by the extension factor alpha: omega_j / alpha;
    yarn   the architecture article's 3.4.2 formula: past train_len, omega_j times
           1 - s 2j/d with s = scale * log2(infer_len / train_len);
    ntk    NTK-aware scaling as a change of base, theta * alpha^(d / (d - 2))."""
    import numpy as np
    j = np.arange(d // 2, dtype=np.float64)
    if kind == "ntk":
        theta = float(theta) * float(alpha) ** (d / (d - 2.0))
    w = float(theta) ** (-2.0 * j / d)
    if kind == "linear":
        w = w / float(alpha)
    elif kind == "yarn":
        if infer_len > train_len:
            w = w * (1.0 - float(scale) * np.log2(infer_len / train_len) * 2.0 * j / d)
    elif kind not in ("base", "ntk"):
        raise ValueError(f"unknown RoPE scaling {kind!r}")
    return w


def pack_block_mask(mask):
    """Bit rows of gqa_params.block_mask from a boolean [query blocks, key blocks] array
    (host, numpy): word w of row qb holds key blocks 32 w .. 32 w + 31, bit j = block
    32 w + j. Returns a host int32 array [rows, words]; move it to the device to use it."""
    import numpy as np
    m = np.asarray(mask, dtype=bool)
    rows, cols = m.shape
    words = max(1, (cols + 31) // 32)
    padded = np.zeros((rows, words * 32), dtype=np.uint64)
    padded[:, :cols] = m
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    packed = (padded.reshape(rows, words, 32) * weights).sum(axis=2)
    return packed.astype(np.uint32).view(np.int32)


def _masks(p, window, block_mask):
    p.window = int(window)
    if block_mask is not None:
        _dev(block_mask, "block_mask", torch.int32)
        if block_mask.dim() != 2:
            raise ValueError("block_mask must be [rows, words] int32 bit rows")
        p.block_mask = _ptr(block_mask)
        p.block_mask_words = block_mask.shape[1]


def prefill(q, k, v, positions=None, *, causal=True, q_norm_w=None, k_norm_w=None, eps=1e-6,
            theta=1e6, scale=0.0, cu_seqlens=None, max_seqlen=None, k_out=None, out=None,
            workspace=None, stream=None, prof=None, window=0, block_mask=None,
            rope_inv_freq=None):
    """gqa_prefill. Dense: q [B, T, H, d], k/v [B, T, G, d]. Packed: q [N, H, d], k/v
    [N, G, d] with cu_seqlens (device int32 [B+1]) and max_seqlen >= every length.
    positions: optional device int32 [N] (RoPE positions; default 0..T_b-1 per sequence).
    k_out: optional [N, G, d] receiving the normalised, rotated K. prof: optional
    (start, stop) torch.cuda.Event pair recorded around the attention kernel alone.
    window: keep only the `window` most recent keys (causal only); block_mask: device int32
    bit rows over 64-key blocks (``pack_block_mask``). rope_inv_freq: optional d/2 RoPE
    frequencies (``rope_freq_table``) in place of theta. Returns out like q."""
    _dev(q, "q")
    dtype = q.dtype
    _dev(k, "k", dtype)
    _dev(v, "v", dtype)
    if cu_seqlens is None:
        if q.dim() != 4:
            raise ValueError("dense prefill takes q [B, T, H, d]")
        B, T, H, d = q.shape
        G = k.shape[2]
        if k.shape != (B, T, G, d) or v.shape != k.shape:
            raise ValueError("k and v must be [B, T, G, d]")
    else:
        _dev(cu_seqlens, "cu_seqlens", torch.int32)
        if q.dim() != 3 or max_seqlen is None:
            raise ValueError("packed prefill takes q [N, H, d] and max_seqlen")
        N, H, d = q.shape
        G = k.shape[1]
        B = cu_seqlens.numel() - 1
        T = int(max_seqlen)
        if k.shape != (N, G, d) or v.shape != k.shape:
            raise ValueError("k and v must be [N, G, d]")
    _dev(positions, "positions", torch.int32)
    _dev(k_out, "k_out", dtype)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", dtype)
    p = _params(dtype, q_norm_w, k_norm_w, eps, theta, scale, stream, q.device, rope_inv_freq)
    nbytes = workspace_bytes("prefill", B, T, H, G, d, dtype)
    ws = _workspace(workspace, nbytes, q.device)
    p.workspace = _ptr(ws)
    p.workspace_bytes = ws.numel() * ws.element_size()
    p.cu_seqlens = _ptr(cu_seqlens)
    p.k_out = _ptr(k_out)
    _masks(p, window, block_mask)
    _prof(p, prof)
    rc = _lib.load().gqa_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(positions), _ptr(out), B, T,
                                 H, G, d, 1 if causal else 0, ctypes.byref(p))
    _lib.check(rc, "gqa_prefill")
    return out


def prefill_cached(q, k, v, k_cache, v_cache, cache_lens, positions=None, *, causal=True,
                   q_norm_w=None, k_norm_w=None, eps=1e-6, theta=1e6, scale=0.0,
                   cu_seqlens=None, max_seqlen=None, out=None, stream=None, prof=None,
                   window=0, block_mask=None, rope_inv_freq=None):
    """gqa_prefill_cached (bf16). New tokens of sequences that already have cache_lens[b]
    (device int32 [B]) tokens in k_cache / v_cache [B, max_seq, G, d]: dense q [B, T, H, d],
    k/v [B, T, G, d], or packed q [N, H, d], k/v [N, G, d] with cu_seqlens and max_seqlen.
    Their K (after norm + RoPE) and V are written into the caches at slots cache_lens[b] + t,
    then every new token attends to its sequence's keys up to its own. window / block_mask
    as in ``prefill``, over key indices of the whole sequence (cache first). Returns out
    like q."""
    _dev(q, "q")
    dtype = q.dtype
    _dev(k, "k", dtype)
    _dev(v, "v", dtype)
    _dev(k_cache, "k_cache", dtype)
    _dev(v_cache, "v_cache", dtype)
    _dev(cache_lens, "cache_lens", torch.int32)
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, max_seq, G, d]")
    Bc, S, G, d = k_cache.shape
    if cu_seqlens is None:
        if q.dim() != 4:
            raise ValueError("dense cached prefill takes q [B, T, H, d]")
        B, T, H, d_q = q.shape
        if k.shape != (B, T, G, d) or v.shape != k.shape:
            raise ValueError("k and v must be [B, T, G, d]")
    else:
        _dev(cu_seqlens, "cu_seqlens", torch.int32)
        if q.dim() != 3 or max_seqlen is None:
            raise ValueError("packed cached prefill takes q [N, H, d] and max_seqlen")
        N, H, d_q = q.shape
        B = cu_seqlens.numel() - 1
        T = int(max_seqlen)
        if k.shape != (N, G, d) or v.shape != k.shape:
            raise ValueError("k and v must be [N, G, d]")
    if d_q != d or Bc != B or cache_lens.numel() != B:
        raise ValueError("q, caches and cache_lens disagree on B or d")
    _dev(positions, "positions", torch.int32)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", dtype)
    p = _params(dtype, q_norm_w, k_norm_w, eps, theta, scale, stream, q.device, rope_inv_freq)
    p.cu_seqlens = _ptr(cu_seqlens)
    _masks(p, window, block_mask)
    _prof(p, prof)
    rc = _lib.load().gqa_prefill_cached(_ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(cache_lens), _ptr(positions), _ptr(out), B, T, H,
                                        G, d, S, 1 if causal else 0, ctypes.byref(p))
    _lib.check(rc, "gqa_prefill_cached")
    return out


def decode(q, k_cache, v_cache, seq_lens, *, k_new=None, v_new=None, positions=None,
           q_norm_w=None, k_norm_w=None, eps=1e-6, theta=1e6, scale=0.0, out=None,
           workspace=None, stream=None, prof=None, rope_inv_freq=None):
    """gqa_decode. q [B, H, d]; caches [B, max_seq, G, d] (K post-prologue, V raw);
    seq_lens device int32 [B] counting the new token; optional k_new/v_new [B, G, d] are
    normalised/rotated (K) and written at slot seq_lens[b]-1 first. prof: optional
    (start, stop) torch.cuda.Event pair recorded around the split-KV pass alone.
    Returns out [B, H, d]."""
    _dev(q, "q")
    dtype = q.dtype
    _dev(k_cache, "k_cache", dtype)
    _dev(v_cache, "v_cache", dtype)
    _dev(seq_lens, "seq_lens", torch.int32)
    _dev(k_new, "k_new", dtype)
    _dev(v_new, "v_new", dtype)
    _dev(positions, "positions", torch.int32)
    B, H, d = q.shape
    _, S, G, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape or k_cache.shape[0] != B:
        raise ValueError("caches must be [B, max_seq, G, d]")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", dtype)
    p = _params(dtype, q_norm_w, k_norm_w, eps, theta, scale, stream, q.device, rope_inv_freq)
    nbytes = workspace_bytes("decode", B, S, H, G, d, dtype)
    ws = _workspace(workspace, nbytes, q.device)
    p.workspace = _ptr(ws)
    p.workspace_bytes = ws.numel() * ws.element_size()
    p.k_new = _ptr(k_new)
    p.v_new = _ptr(v_new)
    p.positions = _ptr(positions)
    _prof(p, prof)
    rc = _lib.load().gqa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                _ptr(out), B, H, G, d, S, ctypes.byref(p))
    _lib.check(rc, "gqa_decode")
    return out


class DecodeGraph:
    """gqa_decode_graph_*: one generation step captured once as a HIP graph.

    Each ``launch()`` first advances seq_lens[b] by one on the device (capped at max_seq), then
    does what ``decode`` does with k_new / v_new: the new token's K/V are written at slot
    seq_lens[b] - 1 and its query attends to seq_lens[b] rows; out receives the result. So
    seq_lens starts at the number of tokens already cached. The tensors are bound at
    creation: write the next step's q / k_new / v_new into them (in stream order) between
    launches. The object keeps references to every bound tensor; ``close()`` (or leaving a
    ``with`` block) waits for the device and releases the graph."""

    def __init__(self, q, k_cache, v_cache, seq_lens, k_new, v_new, *, positions=None,
                 q_norm_w=None, k_norm_w=None, eps=1e-6, theta=1e6, scale=0.0, out=None,
                 workspace=None, rope_inv_freq=None):
        self._h = None
        _dev(q, "q")
        dtype = q.dtype
        for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (k_new, "k_new"),
                     (v_new, "v_new")):
            if t is None:
                raise ValueError(f"{n} is required")
            _dev(t, n, dtype)
        _dev(seq_lens, "seq_lens", torch.int32)
        _dev(positions, "positions", torch.int32)
        B, H, d = q.shape
        _, S, G, d2 = k_cache.shape
        if d2 != d or v_cache.shape != k_cache.shape or k_cache.shape[0] != B:
            raise ValueError("caches must be [B, max_seq, G, d]")
        if k_new.shape != (B, G, d) or v_new.shape != k_new.shape or seq_lens.numel() != B:
            raise ValueError("k_new / v_new must be [B, G, d] and seq_lens [B]")
        out = torch.empty_like(q) if out is None else _dev(out, "out", dtype)
        p = _params(dtype, q_norm_w, k_norm_w, eps, theta, scale, None, q.device, rope_inv_freq)
        ws = _workspace(workspace, workspace_bytes("decode", B, S, H, G, d, dtype), q.device)
        p.workspace = _ptr(ws)
        p.workspace_bytes = ws.numel() * ws.element_size()
        p.k_new = _ptr(k_new)
        p.v_new = _ptr(v_new)
        p.positions = _ptr(positions)
        self.device = q.device
        self.out = out
        self._keep = (q, k_cache, v_cache, seq_lens, k_new, v_new, positions, q_norm_w,
                      k_norm_w, out, ws)
        h = ctypes.c_void_p()
        rc = _lib.load().gqa_decode_graph_create(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                 _ptr(seq_lens), _ptr(out), B, H, G, d, S,
                                                 ctypes.byref(p), ctypes.byref(h))
        _lib.check(rc, "gqa_decode_graph_create")
        self._h = h

    def launch(self, stream=None):
        """Enqueue one step on ``stream`` (default: torch's current stream); returns out."""
        if self._h is None:
            raise RuntimeError("the decode graph is closed")
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        rc = _lib.load().gqa_decode_graph_launch(self._h, ctypes.c_void_p(s.cuda_stream))
        _lib.check(rc, "gqa_decode_graph_launch")
        return self.out

    def close(self):
        if self._h is not None:
            torch.cuda.synchronize(self.device)
            rc = _lib.load().gqa_decode_graph_destroy(self._h)
            self._h = None
            _lib.check(rc, "gqa_decode_graph_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def qk_norm_rope(q, k=None, positions=None, *, q_norm_w=None, k_norm_w=None, eps=1e-6,
                 theta=1e6, q_out=None, k_out=None, stream=None, rope_inv_freq=None):
    """gqa_qk_norm_rope: q [N, H, d] (and k [N, G, d]) -> normalised, rotated copies.
    positions: device int32 [N] or None for 0..N-1."""
    _dev(q, "q")
    dtype = q.dtype
    N, H, d = q.shape
    G = 1 if k is None else k.shape[1]
    _dev(k, "k", dtype)
    _dev(positions, "positions", torch.int32)
    q_out = torch.empty_like(q) if q_out is None else _dev(q_out, "q_out", dtype)
    if k is not None:
        k_out = torch.empty_like(k) if k_out is None else _dev(k_out, "k_out", dtype)
    p = _params(dtype, q_norm_w, k_norm_w, eps, theta, 0.0, stream, q.device, rope_inv_freq)
    rc = _lib.load().gqa_qk_norm_rope(_ptr(q), _ptr(k), _ptr(positions), _ptr(q_out),
                                      _ptr(k_out), N, H, G, d, ctypes.byref(p))
    _lib.check(rc, "gqa_qk_norm_rope")
    return q_out, k_out
