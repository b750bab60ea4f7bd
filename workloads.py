"""Seeded synthetic inputs for causal grouped-query attention (QK-RMSNorm + RoPE).

This module only draws numbers, encodes them in the storage dtype and (at the end) copies
them into device tensors. It holds none of the attention arithmetic, so both the fp64 CPU
oracle (under ``oracle/``) and the HIP path can take their inputs from here without sharing
any of the method's code.

Recipe (the pages measure nothing at the kernel level, so the inputs stand in for
post-projection Q/K/V activations at Qwen3 head shapes):

* Generator: ``numpy.random.default_rng`` (PCG64). Every draw is float32, then encoded in the
  case dtype (bf16 by round-to-nearest-even on the fp32 bit pattern; fp32 as drawn).
* Prefill draw order from ``default_rng(seed)``: sequence lengths (if drawn), q, k, v, then
  gamma_q and gamma_k (U(0.5, 1.5), or exactly 1).
* Decode draw order from ``default_rng(seed)``: lengths, q, k_new, v_new, gamma_q, gamma_k.
  The cache rows of sequence b come from their own stream ``default_rng([seed, b])`` (K rows
  then V rows), so one sequence can be regenerated on its own.
* Cached prefill: the new tokens are drawn as a prefill case (positions continue from each
  sequence's cache length); the cache rows of sequence b come from ``default_rng([seed, b])``
  as for decode. A named workload that draws its cache lengths does so from its own
  ``default_rng(seed)`` first.
* Decode loop: q, k, v of every step from ``default_rng(seed)`` (then gamma_q, gamma_k); the
  starting cache rows per sequence as for decode.
* Values are N(0, 1); positions restart at 0 in every packed sequence (prefill).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

F32 = "f32"
BF16 = "bf16"


# ----------------------------------------------------------------------------- encodings
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def encode(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return f32_to_bf16_bits(x_f32)
    if dtype == F32:
        return np.ascontiguousarray(x_f32, dtype=np.float32)
    raise ValueError(dtype)


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """The exact values a stored array holds, as float64."""
    if dtype == BF16:
        return bf16_bits_to_f64(stored)
    if dtype == F32:
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _gamma(rng, d, kind):
    if kind == "ones":
        return np.ones(d, dtype=np.float32)
    if kind == "uniform":
        return rng.uniform(0.5, 1.5, size=d).astype(np.float32)
    raise ValueError(kind)


# ----------------------------------------------------------------------------- prefill
@dataclasses.dataclass
class PrefillCase:
    """Packed (token-major) prefill inputs. Arrays are in storage form: float32 for f32
    cases, uint16 bf16 bit patterns for bf16 cases."""

    name: str
    seed: int
    dtype: str
    lengths: np.ndarray  # int64 [B]
    H: int
    G: int
    d: int
    causal: bool
    eps: float
    theta: float
    q: np.ndarray  # [N, H, d]
    k: np.ndarray  # [N, G, d]
    v: np.ndarray  # [N, G, d]
    q_norm_w: np.ndarray  # [d]
    k_norm_w: np.ndarray  # [d]
    positions: np.ndarray  # int32 [N]
    cu_seqlens: np.ndarray  # int32 [B + 1]

    @property
    def B(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def N(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def T_max(self) -> int:
        return int(self.lengths.max()) if self.B else 0

    @property
    def dense(self) -> bool:
        """All sequences share one length, so the batch can be passed as [B, T, ...]."""
        return bool(self.B > 0 and np.all(self.lengths == self.lengths[0]))

    def f64(self, name: str) -> np.ndarray:
        return to_f64(getattr(self, name), self.dtype)

    @property
    def flops(self) -> float:
        """Algorithmic FLOPs: 4*d*H per visible (query, key) pair (2d for QK^T, 2d for PV)."""
        L = self.lengths.astype(np.float64)
        pairs = np.sum(L * (L + 1) / 2) if self.causal else np.sum(L * L)
        return float(4.0 * self.d * self.H * pairs)


def default_positions(lengths: np.ndarray) -> np.ndarray:
    """Positions 0..T_b-1 inside each packed sequence."""
    if len(lengths) == 0:
        return np.zeros(0, dtype=np.int32)
    return np.concatenate([np.arange(int(t), dtype=np.int32) for t in lengths]).astype(np.int32)


def cu_seqlens_of(lengths: np.ndarray) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def make_prefill(name, seed, lengths=None, H=16, G=8, d=128, dtype=BF16, causal=True,
                 gamma="uniform", eps=1e-6, theta=1e6, length_range=None, n_seqs=None,
                 positions=None) -> PrefillCase:
    """Draw one prefill case. Either ``lengths`` is given, or ``n_seqs`` lengths are drawn
    uniformly from the integer range ``length_range`` (inclusive) first."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        lo, hi = length_range
        lengths = rng.integers(lo, hi + 1, size=n_seqs)
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = cu_seqlens_of(lengths)
    N = int(cu[-1])
    q = encode(_normal(rng, (N, H, d)), dtype)
    k = encode(_normal(rng, (N, G, d)), dtype)
    v = encode(_normal(rng, (N, G, d)), dtype)
    gq = encode(_gamma(rng, d, gamma), dtype)
    gk = encode(_gamma(rng, d, gamma), dtype)
    pos = default_positions(lengths) if positions is None else np.asarray(positions, np.int32)
    return PrefillCase(name=name, seed=seed, dtype=dtype, lengths=lengths, H=H, G=G, d=d,
                       causal=causal, eps=eps, theta=theta, q=q, k=k, v=v, q_norm_w=gq,
                       k_norm_w=gk, positions=pos, cu_seqlens=cu)


# ----------------------------------------------------------------------------- decode
@dataclasses.dataclass
class DecodeCase:
    """Single-token decode against a contiguous per-sequence cache [B, max_seq, G, d].

    ``seq_lens[b]`` counts the new token: its K/V sit (or are appended) at slot
    seq_lens[b]-1 before attention. Cache rows are produced on demand by ``cache_rows``."""

    name: str
    seed: int
    dtype: str
    seq_lens: np.ndarray  # int32 [B]
    max_seq: int
    H: int
    G: int
    d: int
    eps: float
    theta: float
    q: np.ndarray  # [B, H, d]
    k_new: np.ndarray  # [B, G, d]
    v_new: np.ndarray  # [B, G, d]
    q_norm_w: np.ndarray
    k_norm_w: np.ndarray

    @property
    def B(self) -> int:
        return int(self.seq_lens.shape[0])

    def f64(self, name: str) -> np.ndarray:
        return to_f64(getattr(self, name), self.dtype)

    def cache_rows(self, b: int):
        """(k_rows, v_rows) of sequence b, each [seq_lens[b], G, d] in storage form."""
        L = int(self.seq_lens[b])
        rng = np.random.default_rng([self.seed, b])
        k = encode(_normal(rng, (L, self.G, self.d)), self.dtype)
        v = encode(_normal(rng, (L, self.G, self.d)), self.dtype)
        return k, v

    def iter_cache_rows(self, threads: int | None = None):
        """Yield (b, k_rows, v_rows) for every sequence, drawn on a thread pool."""
        threads = threads or min(16, len(os.sched_getaffinity(0)))
        with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
            futs = {ex.submit(self.cache_rows, b): b for b in range(self.B)}
            for f in _cf.as_completed(futs):
                k, v = f.result()
                yield futs[f], k, v

    @property
    def kv_bytes(self) -> float:
        """Algorithmic decode bytes: visible K and V rows, plus q in and out."""
        el = 2 if self.dtype == BF16 else 4
        kv = float(np.sum(self.seq_lens.astype(np.float64))) * self.G * self.d * 2 * el
        return kv + 2.0 * self.B * self.H * self.d * el


def make_decode(name, seed, B=64, len_range=(1024, 32768), max_seq=32768, H=32, G=8, d=128,
                dtype=BF16, gamma="uniform", eps=1e-6, theta=1e6, seq_lens=None) -> DecodeCase:
    rng = np.random.default_rng(seed)
    if seq_lens is None:
        lo, hi = len_range
        seq_lens = rng.integers(lo, hi + 1, size=B)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.max(initial=0) <= max_seq
    q = encode(_normal(rng, (B, H, d)), dtype)
    k_new = encode(_normal(rng, (B, G, d)), dtype)
    v_new = encode(_normal(rng, (B, G, d)), dtype)
    gq = encode(_gamma(rng, d, gamma), dtype)
    gk = encode(_gamma(rng, d, gamma), dtype)
    return DecodeCase(name=name, seed=seed, dtype=dtype, seq_lens=seq_lens, max_seq=max_seq,
                      H=H, G=G, d=d, eps=eps, theta=theta, q=q, k_new=k_new, v_new=v_new,
                      q_norm_w=gq, k_norm_w=gk)


# ----------------------------------------------------------------------------- block layouts
def make_block_mask(seed, n_blocks, density, local=1, causal=True) -> np.ndarray:
    """Seeded boolean key-block layout [n_blocks, n_blocks] for the block-sparse mask: query
    block qb keeps its ``local`` preceding key blocks and each other earlier block (any
    block, without ``causal``) with probability ``density``; the diagonal is left to the
    mask's own rule. Drawn from ``default_rng(seed)``: one uniform per entry, row-major."""
    rng = np.random.default_rng(seed)
    u = rng.random((n_blocks, n_blocks))
    qb = np.arange(n_blocks)[:, None]
    kb = np.arange(n_blocks)[None, :]
    keep = u < density
    if causal:
        keep &= kb < qb
    keep |= (kb < qb) & (kb >= qb - local)
    return keep


# ----------------------------------------------------------------------------- decode loop
@dataclasses.dataclass
class DecodeStepsCase:
    """S generation steps of B sequences: step s brings one new token per sequence
    (q [S, B, H, d], k / v [S, B, G, d]); sequence b starts with cache_lens[b] cached rows in a
    contiguous cache [B, max_seq, G, d], drawn from ``default_rng([seed, b])`` as for decode."""

    name: str
    seed: int
    dtype: str
    cache_lens: np.ndarray  # int32 [B]
    max_seq: int
    H: int
    G: int
    d: int
    eps: float
    theta: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_norm_w: np.ndarray
    k_norm_w: np.ndarray

    @property
    def B(self) -> int:
        return int(self.cache_lens.shape[0])

    @property
    def S(self) -> int:
        return int(self.q.shape[0])

    def f64(self, name: str) -> np.ndarray:
        return to_f64(getattr(self, name), self.dtype)

    def cache_rows(self, b: int):
        L = int(self.cache_lens[b])
        rng = np.random.default_rng([self.seed, b])
        k = encode(_normal(rng, (L, self.G, self.d)), self.dtype)
        v = encode(_normal(rng, (L, self.G, self.d)), self.dtype)
        return k, v

    @property
    def kv_bytes(self) -> float:
        """Algorithmic bytes of all S steps: every visible K and V row at each step (step s
        of sequence b sees cache_lens[b] + s + 1 rows), plus q in and out."""
        el = 2 if self.dtype == BF16 else 4
        S = self.S
        rows = float(np.sum(self.cache_lens.astype(np.float64))) * S + self.B * S * (S + 1) / 2
        return rows * self.G * self.d * 2 * el + 2.0 * S * self.B * self.H * self.d * el


def make_decode_steps(name, seed, cache_lens, S, max_seq, H=32, G=8, d=128, dtype=BF16,
                      gamma="uniform", eps=1e-6, theta=1e6) -> DecodeStepsCase:
    """Draw order from ``default_rng(seed)``: q, k, v of all steps, gamma_q, gamma_k."""
    cache_lens = np.asarray(cache_lens, dtype=np.int32)
    B = cache_lens.shape[0]
    assert np.all(cache_lens.astype(np.int64) + S <= max_seq)
    rng = np.random.default_rng(seed)
    q = encode(_normal(rng, (S, B, H, d)), dtype)
    k = encode(_normal(rng, (S, B, G, d)), dtype)
    v = encode(_normal(rng, (S, B, G, d)), dtype)
    gq = encode(_gamma(rng, d, gamma), dtype)
    gk = encode(_gamma(rng, d, gamma), dtype)
    return DecodeStepsCase(name=name, seed=seed, dtype=dtype, cache_lens=cache_lens,
                           max_seq=int(max_seq), H=H, G=G, d=d, eps=eps, theta=theta, q=q, k=k,
                           v=v, q_norm_w=gq, k_norm_w=gk)


# ----------------------------------------------------------------------------- cached prefill
@dataclasses.dataclass
class CachedPrefillCase:
    """New tokens of sequences that already hold ``cache_lens[b]`` tokens in a contiguous
    cache [B, max_seq, G, d]. ``new`` holds the new tokens packed, at positions
    cache_lens[b] + t. Cache rows of sequence b come from ``default_rng([seed, b])`` (K rows
    then V rows), like the decode cache."""

    new: PrefillCase
    cache_lens: np.ndarray  # int32 [B]
    max_seq: int

    def __getattr__(self, name):
        if "new" not in self.__dict__:  # during copying, before the fields exist
            raise AttributeError(name)
        return getattr(self.__dict__["new"], name)

    def cache_rows(self, b: int):
        """(k_rows, v_rows) of sequence b, each [cache_lens[b], G, d] in storage form."""
        L = int(self.cache_lens[b])
        rng = np.random.default_rng([self.new.seed, b])
        k = encode(_normal(rng, (L, self.new.G, self.new.d)), self.new.dtype)
        v = encode(_normal(rng, (L, self.new.G, self.new.d)), self.new.dtype)
        return k, v

    @property
    def flops(self) -> float:
        """Algorithmic FLOPs: 4*d*H per visible (query, key) pair; new token t of sequence b
        sees cache_lens[b] + t + 1 keys (causal) or cache_lens[b] + T_b (not)."""
        T = self.new.lengths.astype(np.float64)
        P = self.cache_lens.astype(np.float64)
        pairs = np.sum(T * P + (T * (T + 1) / 2 if self.new.causal else T * T))
        return float(4.0 * self.new.d * self.new.H * pairs)


def make_cached_prefill(name, seed, lengths, cache_lens, max_seq, H=32, G=8, d=128,
                        causal=True, gamma="uniform", eps=1e-6, theta=1e6) -> CachedPrefillCase:
    """New tokens drawn as by ``make_prefill`` (positions cache_lens[b] + t), plus the
    per-sequence cache streams."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cache_lens = np.asarray(cache_lens, dtype=np.int32)
    assert lengths.shape == cache_lens.shape
    assert np.all(cache_lens.astype(np.int64) + lengths <= max_seq)
    pos = (np.concatenate([c + np.arange(int(t)) for c, t in zip(cache_lens, lengths)])
           if len(lengths) else np.zeros(0)).astype(np.int32)
    new = make_prefill(name, seed, lengths=lengths, H=H, G=G, d=d, causal=causal, gamma=gamma,
                       eps=eps, theta=theta, positions=pos)
    return CachedPrefillCase(new=new, cache_lens=cache_lens, max_seq=int(max_seq))


# ----------------------------------------------------------------------------- named workloads
def tiny_f32():
    """Tiny fp32 prefill: B=1, T=128, H=16, G=8, d=64, causal, gamma = 1."""
    return make_prefill("tiny_f32_T128_H16_G8_d64", 1, lengths=[128], H=16, G=8, d=64,
                        dtype=F32, gamma="ones")


def prefill_4k():
    """bf16 prefill: B=1, T=4096, H=16, G=8, d=128, causal, gamma ~ U(0.5, 1.5)."""
    return make_prefill("bf16_prefill_T4096_H16_G8_d128", 2, lengths=[4096], H=16, G=8, d=128)


def prefill_varlen():
    """bf16 packed prefill: 8 sequences, T_b ~ U{512..8192}, H=32, G=8, d=128."""
    return make_prefill("bf16_varlen_8x[512,8192]_H32_G8_d128", 3, length_range=(512, 8192),
                        n_seqs=8, H=32, G=8, d=128)


def decode_64():
    """bf16 decode: 64 sequences x 1 new token, L_b ~ U{1024..32768}, H=32, G=8, d=128."""
    return make_decode("bf16_decode_64x[1024,32768]_H32_G8_d128", 4)


def prefill_long(G=4):
    """bf16 long prefill: B=1, T=32768, H=64, G=4 (h=16) or G=1 (MQA), d=128."""
    seed = 5 if G == 4 else 6
    return make_prefill(f"bf16_prefill_T32768_H64_G{G}_d128", seed, lengths=[32768], H=64,
                        G=G, d=128)


def prefill_chunked():
    """bf16 chunked prefill: 4 sequences, each a 2048-token chunk after a cached prefix of
    U{2048..14336} tokens, cache of 16384 rows, H=32, G=8, d=128."""
    rng = np.random.default_rng(7)
    past = rng.integers(2048, 14336 + 1, size=4)
    return make_cached_prefill("bf16_chunked_4x2048_after_[2048,14336]_H32_G8_d128", 7,
                               lengths=[2048] * 4, cache_lens=past, max_seq=16384)


def decode_loop():
    """bf16 generation loop: 16 sequences x 64 steps, starting cache lengths U{256..2048}
    (drawn first from ``default_rng(8)``), cache of 4096 rows, H=32, G=8, d=128."""
    rng = np.random.default_rng(8)
    lens = rng.integers(256, 2048 + 1, size=16)
    return make_decode_steps("bf16_decode_loop_16x64_from_[256,2048]_H32_G8_d128", 8, lens, 64,
                             4096)


# ----------------------------------------------------------------------------- device placement
# Copies a case's stored arrays into device tensors (bit-exact: bf16 travels as its 16-bit
# pattern). torch is imported here only, so the CPU oracle never needs it.
def to_dev(arr: np.ndarray, dtype: str):
    import torch
    if dtype == BF16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def i32(arr):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32)).cuda()


def _device_caches(B, max_seq, G, d, dtype, rows, fill_invalid):
    """K/V caches [B, max_seq, G, d]: each (b, k, v) of ``rows`` fills the first rows of
    sequence b; the rest are zero, or ``fill_invalid``."""
    import torch
    tdt = torch.bfloat16 if dtype == BF16 else torch.float32
    kc = torch.zeros((B, max_seq, G, d), dtype=tdt, device="cuda")
    vc = torch.zeros((B, max_seq, G, d), dtype=tdt, device="cuda")
    if fill_invalid is not None:
        kc.fill_(fill_invalid)
        vc.fill_(fill_invalid)
    for b, k, v in rows:
        L = k.shape[0]
        if L:
            kc[b, :L] = to_dev(k, dtype)
            vc[b, :L] = to_dev(v, dtype)
    return kc, vc


def device_prefill_inputs(case: PrefillCase) -> dict:
    dt = case.dtype
    return dict(q=to_dev(case.q, dt), k=to_dev(case.k, dt), v=to_dev(case.v, dt),
                q_norm_w=to_dev(case.q_norm_w, dt), k_norm_w=to_dev(case.k_norm_w, dt),
                positions=i32(case.positions), cu=i32(case.cu_seqlens))


def device_decode_inputs(case: DecodeCase, fill_invalid=None) -> dict:
    """Device tensors for a decode case; the cache holds the first seq_lens[b] rows of each
    sequence."""
    dt = case.dtype
    kc, vc = _device_caches(case.B, case.max_seq, case.G, case.d, dt, case.iter_cache_rows(),
                            fill_invalid)
    return dict(q=to_dev(case.q, dt), k_cache=kc, v_cache=vc, seq_lens=i32(case.seq_lens),
                k_new=to_dev(case.k_new, dt), v_new=to_dev(case.v_new, dt),
                q_norm_w=to_dev(case.q_norm_w, dt), k_norm_w=to_dev(case.k_norm_w, dt))


def device_cached_inputs(case: CachedPrefillCase, fill_invalid=None) -> dict:
    """Device tensors for a cached-prefill case: the new tokens (packed) and caches holding
    cache_lens[b] rows per sequence."""
    dev = device_prefill_inputs(case.new)
    kc, vc = _device_caches(case.B, case.max_seq, case.G, case.d, BF16,
                            ((b, *case.cache_rows(b)) for b in range(case.B)), fill_invalid)
    dev.update(k_cache=kc, v_cache=vc, cache_lens=i32(case.cache_lens))
    return dev


def device_steps_inputs(case: DecodeStepsCase, fill_invalid=None) -> dict:
    """Device tensors for a decode-loop case: per-step q [S, B, H, d], k / v [S, B, G, d],
    caches holding cache_lens[b] rows, and seq_lens = cache_lens."""
    dt = case.dtype
    kc, vc = _device_caches(case.B, case.max_seq, case.G, case.d, dt,
                            ((b, *case.cache_rows(b)) for b in range(case.B)), fill_invalid)
    return dict(q=to_dev(case.q, dt), k=to_dev(case.k, dt), v=to_dev(case.v, dt), k_cache=kc,
                v_cache=vc, seq_lens=i32(case.cache_lens), q_norm_w=to_dev(case.q_norm_w, dt),
                k_norm_w=to_dev(case.k_norm_w, dt))
