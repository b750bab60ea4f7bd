"""Host-side parts of bench.py (CPU): the one-GPU refusal, and the algorithmic work it counts
for the mask variants, checked against the oracle's own visibility mask."""
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
