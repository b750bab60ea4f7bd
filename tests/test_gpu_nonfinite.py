"""Non-finite inputs on the GPU: a NaN or infinity placed in q, k or v reaches exactly the
outputs the C header says it reaches, and every other output is finite and matches the fp64
oracle run on the same inputs without the planted values (those outputs do not depend on
them). Covers the bf16 prefill (plain and windowed), the fp32 prefill and decode."""
import numpy as np
import pytest
import torch

import workloads as W

from _gpu import (check, device_decode_inputs, device_prefill_inputs, oracle_decode_seq,
                  oracle_prefill, run_decode, run_prefill, say, to_f64)

pytestmark = pytest.mark.gpu

NAN, INF = float("nan"), float("inf")


def _plant(dev, name, index, value):
    t = dev[name]
    t[index] = value


def _bad_rows(got):
    """Boolean [N, H]: output rows (token, head) with any non-finite element."""
    return ~np.all(np.isfinite(got), axis=-1)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_prefill_nonfinite_reach(dtype):
    # two packed sequences of 300 and 200 tokens, H = 8, G = 2 (h = 4: a 128-column block of
    # the bf16 kernel holds 32 consecutive positions)
    case = W.make_prefill("nonfinite_" + dtype, 501, lengths=[300, 200], H=8, G=2, d=128,
                          dtype=dtype)
    want = oracle_prefill(case)  # clean inputs
    dev = device_prefill_inputs(case)
    s1 = 300  # first token of sequence 1
    _plant(dev, "q", (50, 3, 7), NAN)             # seq 0, position 50, head 3
    _plant(dev, "q", (s1 + 150, 6, 0), -INF)      # seq 1, position 150, head 6
    _plant(dev, "k", (120, 1, 5), INF)            # seq 0, position 120, group 1 (heads 4-7)
    _plant(dev, "v", (s1 + 80, 0, 9), NAN)        # seq 1, position 80, group 0 (heads 0-3)
    say("prefill non-finite inputs", dtype)
    got = to_f64(run_prefill(case, dev=dev))
    bad = _bad_rows(got)
    must = np.zeros_like(bad)
    must[50, 3] = True
    must[s1 + 150, 6] = True
    must[120:300, 4:8] = True                     # every query of seq 0 that sees key 120
    must[s1 + 80:s1 + 200, 0:4] = True            # every query of seq 1 that sees key 80
    may = must.copy()
    if dtype == W.BF16:
        # the V row's tile products: earlier positions of the same 32-position block
        may[s1 + 64:s1 + 80, 0:4] = True
    assert np.all(bad[must]), "a planted value did not reach an output that sees it"
    assert not np.any(bad & ~may), np.argwhere(bad & ~may)[:10]
    ok = ~may
    check(got[ok], want[ok], dtype, "outputs away from the planted values")


def test_prefill_window_nonfinite_reach():
    # with a 40-key window a key is seen by the 40 queries from its own position on
    case = W.make_prefill("nonfinite_win", 502, lengths=[400], H=8, G=2, d=128)
    want = oracle_prefill(case, window=40)
    dev = device_prefill_inputs(case)
    _plant(dev, "k", (200, 0, 3), NAN)
    say("prefill window non-finite K")
    got = to_f64(run_prefill(case, dev=dev, window=40))
    bad = _bad_rows(got)
    must = np.zeros_like(bad)
    must[200:240, 0:4] = True
    assert np.all(bad[must]) and not np.any(bad & ~must), np.argwhere(bad != must)[:10]
    check(got[~must], want[~must], W.BF16, "outputs away from the planted value")


def test_decode_nonfinite_reach():
    B, H, G, d = 5, 32, 8, 128
    lens = [700, 1500, 64, 2000, 1]
    case = W.make_decode("nonfinite_dec", 503, B=B, max_seq=2048, H=H, G=G, d=d, seq_lens=lens)
    dev = device_decode_inputs(case, fill_invalid=NAN)  # rows past each length: NaN, never read
    _plant(dev, "q", (1, 5, 11), NAN)              # seq 1, head 5 only
    _plant(dev, "k_cache", (2, 10, 3, 0), NAN)     # seq 2, key 10, group 3 (heads 12-15)
    _plant(dev, "v_cache", (3, 500, 0, 64), INF)   # seq 3, key 500, group 0 (heads 0-3)
    say("decode non-finite inputs")
    got = to_f64(run_decode(case, dev, append=False))
    bad = _bad_rows(got)
    must = np.zeros_like(bad)
    must[1, 5] = True
    must[2, 12:16] = True
    must[3, 0:4] = True
    assert np.all(bad[must]) and not np.any(bad & ~must), np.argwhere(bad != must)[:10]
    for b in range(B):
        want, _, _ = oracle_decode_seq(case, b, append=False)
        rows = ~must[b]
        check(got[b][rows], want[rows], W.BF16, f"decode seq {b}")
