"""The C-ABI from C: tests/c_abi/client.c, a plain C program (no Python, no torch), links
libgqa.so and the HIP runtime, runs gqa_prefill and gqa_decode with the K/V append on inputs
this test writes, and its outputs are checked against the fp64 oracle like every other
parity test."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import workloads as W

from _gpu import check, oracle_decode_seq, oracle_prefill, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "attention_head_qk_amd")


def _build_client(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "gqa_client")
    cmd = [cc, "-std=c11", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "c_abi", "client.c"),
           "-L", PKG, "-lgqa", "-L", "/opt/rocm/lib", "-lamdhip64",
           f"-Wl,-rpath,{PKG}", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def test_c_client_prefill_and_decode(tmp_path):
    exe = _build_client(tmp_path)
    # the client takes one B, H, G, d and one gqa_params (so one pair of gammas) for both
    # calls: the decode case takes the prefill case's gammas
    Bc, T, H, G, d, S = 3, 150, 16, 4, 128, 300
    pre = W.make_prefill("c_abi_prefill", 301, lengths=[T] * Bc, H=H, G=G, d=d)
    dec = W.make_decode("c_abi_decode", 302, B=Bc, max_seq=S, H=H, G=G, d=d,
                        seq_lens=[1, 150, 300])
    dec.q_norm_w, dec.k_norm_w = pre.q_norm_w, pre.k_norm_w
    kc = np.zeros((Bc, S, G, d), np.uint16)
    vc = np.zeros((Bc, S, G, d), np.uint16)
    for b, k, v in dec.iter_cache_rows():
        kc[b, :k.shape[0]] = k
        vc[b, :v.shape[0]] = v
    inp = tmp_path / "in.bin"
    with open(inp, "wb") as f:
        f.write(np.array([Bc, T, H, G, d, S], np.int32).tobytes())
        for a in (pre.q, pre.k, pre.v, pre.q_norm_w, pre.k_norm_w, dec.q, dec.k_new, dec.v_new,
                  kc, vc):
            f.write(np.ascontiguousarray(a, dtype=np.uint16).tobytes())
        f.write(np.asarray(dec.seq_lens, np.int32).tobytes())
    out = tmp_path / "out.bin"
    say("C client: prefill B=3 T=150 H=16 G=4 + decode B=3 S=300")
    r = subprocess.run([exe, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = np.frombuffer(out.read_bytes(), np.uint16)
    n_pre, n_dec, n_c = Bc * T * H * d, Bc * H * d, Bc * S * G * d
    assert raw.size == n_pre + n_dec + 2 * n_c
    got_pre = W.to_f64(raw[:n_pre].reshape(Bc * T, H, d), W.BF16)
    got_dec = W.to_f64(raw[n_pre:n_pre + n_dec].reshape(Bc, H, d), W.BF16)
    got_kc = W.to_f64(raw[n_pre + n_dec:n_pre + n_dec + n_c].reshape(Bc, S, G, d), W.BF16)
    got_vc = raw[n_pre + n_dec + n_c:].reshape(Bc, S, G, d)
    check(got_pre, oracle_prefill(pre), W.BF16, "C client prefill")
    for b in range(Bc):
        want, k_slot, _ = oracle_decode_seq(dec, b)
        check(got_dec[b], want, W.BF16, f"C client decode b={b}")
        L = int(dec.seq_lens[b])
        assert np.all(np.abs(got_kc[b, L - 1] - k_slot) <= 2.0 ** -8 * np.abs(k_slot) + 1e-6)
        assert np.array_equal(got_vc[b, L - 1], dec.v_new[b])
