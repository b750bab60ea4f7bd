"""Helpers shared by the GPU tests: move seeded inputs to the device, call the HIP path
through the binding, bring results back as float64, and compare with the tolerances the
path is held to (fp32: max abs <= 1e-5; bf16: max abs <= 2e-2 and mean abs <= 2e-3)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads as W
from workloads import (device_cached_inputs, device_decode_inputs,  # noqa: F401
                       device_prefill_inputs, device_steps_inputs, i32, to_dev)

F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3


def say(*a):
    """Name the case on stdout before a GPU step, so a fault can be traced to it."""
    print(*a, flush=True)
    sys.stdout.flush()






def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(got: np.ndarray, want: np.ndarray, dtype: str, what: str = "") -> dict:
    err = np.abs(got - want)
    stats = {"max_abs": float(err.max(initial=0.0)), "mean_abs": float(err.mean()) if err.size else 0.0}
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if dtype == W.F32:
        assert stats["max_abs"] <= F32_MAX_ABS, f"{what}: {stats}"
    else:
        assert stats["max_abs"] <= BF16_MAX_ABS and stats["mean_abs"] <= BF16_MEAN_ABS, f"{what}: {stats}"
    return stats




def run_prefill(case: W.PrefillCase, dev=None, packed=None, pass_positions=True, **kw):
    """Run gqa_prefill on a case; packed=None picks dense for one-length batches."""
    import attention_head_qk_amd as gqa
    dev = dev or device_prefill_inputs(case)
    if packed is None:
        packed = not case.dense
    pos = dev["positions"] if pass_positions else None
    common = dict(causal=case.causal, q_norm_w=dev["q_norm_w"], k_norm_w=dev["k_norm_w"],
                  eps=case.eps, theta=case.theta, **kw)
    if packed:
        out = gqa.prefill(dev["q"], dev["k"], dev["v"], pos, cu_seqlens=dev["cu"],
                          max_seqlen=max(case.T_max, 1), **common)
    else:
        B, T = case.B, case.T_max
        H, G, d = case.H, case.G, case.d
        out = gqa.prefill(dev["q"].view(B, T, H, d), dev["k"].view(B, T, G, d),
                          dev["v"].view(B, T, G, d), pos, **common).view(-1, H, d)
    return out


def oracle_prefill(case: W.PrefillCase, **masks):
    """masks: window / block_mask (boolean layout) as the oracle takes them."""
    from oracle import gqa_oracle as O
    return O.prefill(case.f64("q"), case.f64("k"), case.f64("v"), case.positions,
                     case.cu_seqlens, case.f64("q_norm_w"), case.f64("k_norm_w"), case.eps,
                     case.theta, case.causal, **masks)


def oracle_prefill_rows(case: W.PrefillCase, rows, **masks):
    from oracle import gqa_oracle as O
    return O.prefill_rows(case.f64("q"), case.f64("k"), case.f64("v"), case.positions,
                          case.cu_seqlens, rows, case.f64("q_norm_w"), case.f64("k_norm_w"),
                          case.eps, case.theta, case.causal, **masks)


def device_block_mask(mask: np.ndarray) -> torch.Tensor:
    """Boolean layout -> the library's device bit rows (packed by the binding's helper)."""
    import attention_head_qk_amd as gqa
    return torch.from_numpy(np.ascontiguousarray(gqa.pack_block_mask(mask))).cuda()


def sample_rows(case: W.PrefillCase, n_random: int, seed: int = 0, tile: int = 64):
    """Packed row indices: rows 0, 1, both sides of every tile boundary below 4*tile, the
    last row of every sequence, plus n_random seeded rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(case.B):
        s, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        if e == s:
            continue
        for r in (0, 1, tile - 1, tile, 2 * tile - 1, 2 * tile, e - s - 1, e - s - 2):
            if 0 <= r < e - s:
                rows.add(s + r)
    N = case.N
    rows.update(int(x) for x in rng.integers(0, N, size=n_random))
    return np.array(sorted(rows), dtype=np.int64)




def run_decode(case: W.DecodeCase, dev, append=True, positions=None, **kw):
    import attention_head_qk_amd as gqa
    return gqa.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["seq_lens"],
                      k_new=dev["k_new"] if append else None,
                      v_new=dev["v_new"] if append else None, positions=positions,
                      q_norm_w=dev["q_norm_w"], k_norm_w=dev["k_norm_w"], eps=case.eps,
                      theta=case.theta, **kw)


def oracle_decode_seq(case: W.DecodeCase, b: int, append=True, position=None):
    from oracle import gqa_oracle as O
    k, v = case.cache_rows(b)
    return O.decode_one(case.f64("q")[b], W.to_f64(k, case.dtype), W.to_f64(v, case.dtype),
                        int(case.seq_lens[b]), case.f64("q_norm_w"), case.f64("k_norm_w"),
                        case.eps, case.theta, position=position,
                        k_new=case.f64("k_new")[b] if append else None,
                        v_new=case.f64("v_new")[b] if append else None)




def run_prefill_cached(case: W.CachedPrefillCase, dev, packed=None, pass_positions=True, **kw):
    """Run gqa_prefill_cached; packed=None picks dense for one-length batches."""
    import attention_head_qk_amd as gqa
    if packed is None:
        packed = not case.new.dense
    pos = dev["positions"] if pass_positions else None
    common = dict(causal=case.causal, q_norm_w=dev["q_norm_w"], k_norm_w=dev["k_norm_w"],
                  eps=case.eps, theta=case.theta, **kw)
    args = (dev["k_cache"], dev["v_cache"], dev["cache_lens"], pos)
    if packed:
        return gqa.prefill_cached(dev["q"], dev["k"], dev["v"], *args, cu_seqlens=dev["cu"],
                                  max_seqlen=max(case.T_max, 1), **common)
    B, T, H, G, d = case.B, case.T_max, case.H, case.G, case.d
    return gqa.prefill_cached(dev["q"].view(B, T, H, d), dev["k"].view(B, T, G, d),
                              dev["v"].view(B, T, G, d), *args, **common).view(-1, H, d)


def oracle_prefill_cached_seq(case: W.CachedPrefillCase, b: int, positions=None, **masks):
    """Oracle of one sequence: (out [T_b, H, d], K rows [past + T_b, G, d], V rows)."""
    from oracle import gqa_oracle as O
    s, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
    past = int(case.cache_lens[b])
    k, v = case.cache_rows(b)
    kc = np.zeros((1, past + e - s, case.G, case.d))
    vc = np.zeros_like(kc)
    kc[0, :past] = W.to_f64(k, W.BF16)
    vc[0, :past] = W.to_f64(v, W.BF16)
    pos = case.positions[s:e] if positions is None else positions
    out, kc2, vc2 = O.prefill_cached(case.f64("q")[s:e], case.f64("k")[s:e], case.f64("v")[s:e],
                                     kc, vc, [past], np.array([0, e - s]), case.f64("q_norm_w"),
                                     case.f64("k_norm_w"), case.eps, case.theta, positions=pos,
                                     causal=case.causal, **masks)
    return out, kc2[0], vc2[0]




def oracle_decode_steps(case: W.DecodeStepsCase):
    """Oracle of every step: (out [S, B, H, d], k_cache', v_cache') in float64."""
    from oracle import gqa_oracle as O
    kc = np.zeros((case.B, case.max_seq, case.G, case.d))
    vc = np.zeros_like(kc)
    for b in range(case.B):
        k, v = case.cache_rows(b)
        kc[b, :k.shape[0]] = W.to_f64(k, case.dtype)
        vc[b, :k.shape[0]] = W.to_f64(v, case.dtype)
    return O.decode_steps(case.f64("q"), case.f64("k"), case.f64("v"), kc, vc, case.cache_lens,
                          case.f64("q_norm_w"), case.f64("k_norm_w"), case.eps, case.theta)
