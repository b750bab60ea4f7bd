"""The thread-pool drivers the GPU tests use to run the oracle over whole workloads
(tests/_oracle_pool.py) give exactly what the oracle's own entry points give (CPU only)."""
import numpy as np

import workloads as W
from oracle import gqa_oracle as O

import _oracle_pool as OP


def test_prefill_full_equals_oracle_prefill():
    case = W.make_prefill("pool", 7, lengths=[70, 0, 130, 1], H=8, G=2, d=64)
    want = O.prefill(case.f64("q"), case.f64("k"), case.f64("v"), case.positions,
                     case.cu_seqlens, case.f64("q_norm_w"), case.f64("k_norm_w"), case.eps,
                     case.theta, True)
    # same arithmetic; BLAS may order its sums differently with one thread than with several
    assert np.abs(OP.prefill_full(case, workers=3) - want).max() <= 1e-12
    bm = W.make_block_mask(3, 3, 0.5)
    want = O.prefill(case.f64("q"), case.f64("k"), case.f64("v"), case.positions,
                     case.cu_seqlens, case.f64("q_norm_w"), case.f64("k_norm_w"), case.eps,
                     case.theta, True, window=40, block_mask=bm)
    assert np.abs(OP.prefill_full(case, window=40, block_mask=bm, workers=4) - want).max() <= 1e-12


def test_decode_all_equals_decode_one():
    case = W.make_decode("pool", 9, B=5, max_seq=300, H=8, G=4, d=64,
                         seq_lens=[1, 0, 299, 64, 130])
    out, ks, vs = OP.decode_all(case, workers=3)
    for b in range(case.B):
        k, v = case.cache_rows(b)
        o, k1, v1 = O.decode_one(case.f64("q")[b], W.to_f64(k, case.dtype),
                                 W.to_f64(v, case.dtype), int(case.seq_lens[b]),
                                 case.f64("q_norm_w"), case.f64("k_norm_w"), case.eps,
                                 case.theta, k_new=case.f64("k_new")[b], v_new=case.f64("v_new")[b])
        assert np.abs(out[b] - o).max(initial=0.0) <= 1e-12
        assert (ks[b] is None and k1 is None) or np.array_equal(ks[b], k1)
        assert (vs[b] is None and v1 is None) or np.array_equal(vs[b], v1)


def test_sample_rows_cover_the_contract():
    # the row sample of the long workloads: >= 512 rows, rows 0 and 1, the last row, both
    # sides of key-tile boundaries and of column-block boundaries (checked on a stand-in
    # case of the same length and head shape, drawn small)
    case = W.make_prefill("rows", 1, lengths=[32768], H=4, G=1, d=8)
    case.H, case.G = 64, 4  # only lengths and h = H / G enter the sample
    rows = OP.sample_rows(case, 512, seed=3)
    assert len(rows) >= 512 and len(set(rows.tolist())) == len(rows)
    for r in (0, 1, 32766, 32767, 63, 64, 1024 + 63, 1024 + 64, 7, 8, 32759, 32760):
        assert r in rows, r
    assert rows.min() >= 0 and rows.max() < 32768
