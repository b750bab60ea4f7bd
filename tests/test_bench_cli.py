"""Host-side parts of the measurement (CPU): bench.py's one-GPU refusal, and the algorithmic
work behind every reported rate (FLOPs of plain, masked and cached prefill, bytes of decode),
counted against the oracle's own visibility mask or the cache rows one by one."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as W
from oracle import gqa_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("lengths,window,density", [
    ([1, 63, 64, 65, 200], 0, None), ([130, 7, 257], 5, None), ([300], 64, None),
    ([200, 129, 64], 0, 0.3), ([333, 1], 100, 0.5), ([256], 1, 0.0),
])
def test_visible_pairs_equals_the_oracle_mask(lengths, window, density):
    layout = None
    if density is not None:
        nb = -(-max(lengths) // 64)
        layout = W.make_block_mask(11, nb, density)
    want = 0
    for T in lengths:
        want += int(O.visible_keys(T, T, True, window, layout, 64).sum())
    assert bench.visible_pairs(np.array(lengths), window, layout) == want


def test_prefill_flops_count_the_oracle_mask():
    for causal in (True, False):
        case = W.make_prefill("c", 3, lengths=np.array([1, 70, 5]), H=6, G=3, d=64, causal=causal)
        pairs = sum(int(O.visible_keys(int(T), int(T), causal).sum()) for T in case.lengths)
        assert case.flops == 4.0 * 64 * 6 * pairs


def test_cached_prefill_flops_count_the_oracle_mask():
    for causal in (True, False):
        case = W.make_cached_prefill("c", 5, [3, 9], [0, 17], 64, H=4, G=2, d=64, causal=causal)
        pairs = sum(int(O.visible_keys(int(T), int(T + P), causal).sum())
                    for T, P in zip(case.new.lengths, case.cache_lens))
        assert case.flops == 4.0 * 64 * 4 * pairs


def test_decode_bytes_count_every_visible_row():
    case = W.make_decode("d", 2, B=5, max_seq=300, H=8, G=2, d=64, seq_lens=[0, 1, 77, 300, 5])
    rows = sum(int(L) for L in case.seq_lens)  # one K and one V row of every group per key
    assert case.kv_bytes == rows * 2 * 64 * 2 * 2 + 2 * 5 * 8 * 64 * 2
    steps = W.make_decode_steps("s", 4, [0, 10], 3, 16, H=4, G=2, d=64)
    rows = sum(int(P) + s + 1 for P in steps.cache_lens for s in range(3))
    assert steps.kv_bytes == rows * 2 * 64 * 2 * 2 + 2 * 3 * 2 * 4 * 64 * 2


def test_cpu_baseline_leg_on_small_cases():
    # the oracle baseline's pool, units and scaling, on small stand-ins of each kind of
    # configuration (a full prefill, a long single sequence timed on sampled rows, a varlen
    # batch timed on one head per group, a decode timed on every 4th sequence)
    cases = {"tiny_f32": W.make_prefill("t", 1, lengths=[100], H=4, G=2, d=64, dtype=W.F32),
             "long_x": W.make_prefill("l", 2, lengths=[16384], H=2, G=1, d=64),
             "varlen_x": W.make_prefill("v", 3, lengths=[300, 5000, 700], H=8, G=2, d=64),
             "decode": W.make_decode("d", 4, B=8, max_seq=600, H=4, G=2, d=64,
                                     seq_lens=[1, 600, 30, 200, 7, 64, 599, 2])}
    pool = bench.start_oracle_pool(cases)
    try:
        out = bench.cpu_baseline_all(pool, list(cases), "long_x")
    finally:
        pool.terminate()
    per = out["per_config"]
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s" and out["cores"] >= 1
    assert out["value"] == per["long_x"]["value"] > 0
    assert per["tiny_f32"]["scale"] == 1 and "full_s" in per["tiny_f32"]
    assert per["long_x"]["scale"] == 16384 / 64
    assert per["varlen_x"]["scale"] == 4 and per["decode"]["unit"] == "GB/s"
    lens = np.sort(cases["decode"].seq_lens)
    assert abs(per["decode"]["scale"] - lens.sum() / lens[::4].sum()) < 1e-3


@pytest.mark.parametrize("make,bound,peak", [(W.tiny_f32, "alu", bench.FP32_PEAK_TFLOPS),
                                             (W.prefill_4k, "mfma", bench.MFMA_BF16_PEAK_TFLOPS)])
def test_prefill_roofline_bound_follows_the_dtype(make, bound, peak):
    # the fp32 kernel's products run on the vector ALUs, the bf16 kernel's on the matrix cores
    r = object.__new__(bench.Prefill)
    r.case = make()
    assert r.bound == bound and r.peak == peak


def _record_file(tmp_path, src_text, sha):
    src = tmp_path / "k.hip"
    src.write_text(src_text)
    rec = tmp_path / "rec.md"
    rec.write_text("```\n    record: kernel=kern workload=wl sources=k.hip sha256=" + sha +
                   " fetch_kib=10.0 write_kib=4.0 fetch_factor=2.0000 write_factor=1.0000\n```\n")
    return rec


def test_traffic_record_is_used_only_while_the_sources_match(tmp_path, monkeypatch):
    import hashlib
    text = "kernel source\n"
    rec = _record_file(tmp_path, text, hashlib.sha256(text.encode()).hexdigest())
    monkeypatch.setattr(bench, "TRAFFIC_RECORDS", str(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # FETCH_SIZE x 2 + WRITE_SIZE x 1, in KiB
    assert bench.measured_traffic("kern", "wl") == (10.0 * 2.0 + 4.0 * 1.0) * 1024.0
    assert bench.measured_traffic("kern", "other") is None
    assert bench.measured_traffic("other", "wl") is None
    (tmp_path / "k.hip").write_text(text + "// changed\n")
    assert bench.measured_traffic("kern", "wl") is None

