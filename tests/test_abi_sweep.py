"""A seeded property-based sweep of the C ABI's host-side checks (CPU only): random sizes,
flags, masks, workspace sizes and fake device pointers (the checks look at them and never
dereference them) for gqa_prefill and gqa_decode. Whatever the arguments, a call returns one
of the documented status codes; on a host without a GPU it reports success only when there
is nothing to do (anything else must fail at its first HIP call, or before); sizes that the
kernels' 32-bit indexing cannot hold, negative sizes and bad flags never get that far.

The sweep skips itself where a GPU is visible: a combination that passes every check would
then launch on the fake pointers."""
import ctypes
import os

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from attention_head_qk_amd import _lib


def _gpu_visible():
    # the kernel driver's device node: present wherever an AMD GPU can be opened
    return os.path.exists("/dev/kfd")


pytestmark = pytest.mark.skipif(_gpu_visible(), reason="fake device pointers: host-only sweep")

A = 0x10000      # aligned fake device address
MIS = 0x10008    # 8-byte aligned only
I32_MAX = 0x7FFFFFFF
STATUS = {_lib.GQA_OK, _lib.GQA_EINVAL, _lib.GQA_ENOTSUP, _lib.GQA_EWORKSPACE, _lib.GQA_EHIP}
REJECTED = {_lib.GQA_EINVAL, _lib.GQA_ENOTSUP, _lib.GQA_EWORKSPACE}

sizes = st.one_of(st.integers(-3, 70), st.sampled_from([I32_MAX, -I32_MAX - 1, 65535, 65536, 1 << 20]))
heads = st.one_of(st.integers(-1, 70), st.sampled_from([128, 256, 1 << 16, I32_MAX]))
ptrs = st.sampled_from([None, A, MIS])
SWEEP = settings(max_examples=400, derandomize=True, deadline=None,
                 suppress_health_check=[HealthCheck.too_slow])


def _params(dtype, window, bm, words, ws, ws_bytes, cu=None):
    p = _lib.default_params()
    p.dtype = dtype
    p.window = window
    p.block_mask = bm
    p.block_mask_words = words
    p.workspace = ws
    p.workspace_bytes = ws_bytes
    if cu is not None:
        p.cu_seqlens = cu
    return p


@SWEEP
@given(B=sizes, T=sizes, H=heads, G=heads, d=st.sampled_from([-1, 0, 32, 64, 96, 128, 256]),
       causal=st.integers(-1, 2), dtype=st.sampled_from([-1, 0, 1, 2, 7]),
       window=st.sampled_from([-1, 0, 1, 7, I32_MAX]), bm=st.sampled_from([None, A, A + 2]),
       words=st.sampled_from([-1, 0, 1, 64, 1 << 30]), ws=st.sampled_from([None, A, MIS]),
       ws_bytes=st.sampled_from([0, 1, 1 << 62]), q=ptrs, k=ptrs, v=ptrs, out=ptrs,
       cu=st.sampled_from([None, A, A + 2]))
def test_prefill_host_checks_sweep(B, T, H, G, d, causal, dtype, window, bm, words, ws, ws_bytes,
                                   q, k, v, out, cu):
    p = _params(dtype, window, bm, words, ws, ws_bytes, cu)
    r = _lib.load().gqa_prefill(q, k, v, None, out, B, T, H, G, d, causal, ctypes.byref(p))
    assert r in STATUS
    if r == _lib.GQA_OK:
        assert B == 0 or T == 0
    if B < 0 or T < 0 or causal not in (0, 1) or B * T > I32_MAX:
        assert r in REJECTED
    if dtype == _lib.GQA_BF16 and G > 0 and H > 0 and H % G == 0 and T * (H // G) > I32_MAX:
        assert r in REJECTED


@SWEEP
@given(B=sizes, S=sizes, H=heads, G=heads, d=st.sampled_from([-1, 0, 32, 64, 96, 128, 256]),
       dtype=st.sampled_from([-1, 0, 1, 2, 7]), window=st.sampled_from([0, 0, 5]),
       ws=st.sampled_from([None, A, MIS]), ws_bytes=st.sampled_from([0, 1, 1 << 62]),
       q=ptrs, kc=ptrs, vc=ptrs, sl=st.sampled_from([None, A, A + 2]), out=ptrs,
       append=st.sampled_from([None, (A, A), (A, None), (MIS, A)]))
def test_decode_host_checks_sweep(B, S, H, G, d, dtype, window, ws, ws_bytes, q, kc, vc, sl, out,
                                  append):
    p = _params(dtype, window, None, 0, ws, ws_bytes)
    if append is not None:
        p.k_new, p.v_new = append
    lib = _lib.load()
    r = lib.gqa_decode(q, kc, vc, sl, out, B, H, G, d, S, ctypes.byref(p))
    assert r in STATUS
    if r == _lib.GQA_OK:
        assert B == 0
    if B < 0 or S <= 0 or window != 0:
        assert r in REJECTED
    # the entry point without a workspace: same checks, its own size limit instead
    r = lib.gqa_decode_noalloc(q, kc, vc, sl, out, B, H, G, d, S, ctypes.byref(p))
    assert r in STATUS
    if r == _lib.GQA_OK:
        assert B == 0
    if B < 0 or S <= 0 or window != 0:
        assert r in REJECTED


@SWEEP
@given(B=sizes, T=sizes, S=sizes, H=heads, G=heads, d=st.sampled_from([-1, 64, 96, 128]),
       causal=st.integers(-1, 2), dtype=st.sampled_from([-1, 0, 1, 7]),
       window=st.sampled_from([-1, 0, 3]), cl=st.sampled_from([None, A, A + 2]), q=ptrs,
       kc=ptrs, out=ptrs, cu=st.sampled_from([None, A, A + 2]))
def test_prefill_cached_host_checks_sweep(B, T, S, H, G, d, causal, dtype, window, cl, q, kc, out,
                                          cu):
    p = _params(dtype, window, None, 0, None, 0, cu)
    r = _lib.load().gqa_prefill_cached(q, A, A, kc, A, cl, None, out, B, T, H, G, d, S, causal,
                                       ctypes.byref(p))
    assert r in STATUS
    if r == _lib.GQA_OK:
        assert B == 0 or T == 0
    if B < 0 or T < 0 or causal not in (0, 1) or dtype == _lib.GQA_F32:
        assert r in REJECTED


@SWEEP
@given(N=sizes, H=heads, G=heads, d=st.sampled_from([-1, 0, 64, 96, 128]),
       dtype=st.sampled_from([-1, 0, 1, 7]), q=ptrs, k=ptrs, qo=ptrs, ko=ptrs,
       pos=st.sampled_from([None, A, A + 2]))
def test_qk_norm_rope_host_checks_sweep(N, H, G, d, dtype, q, k, qo, ko, pos):
    p = _params(dtype, 0, None, 0, None, 0)
    r = _lib.load().gqa_qk_norm_rope(q, k, pos, qo, ko, N, H, G, d, ctypes.byref(p))
    assert r in STATUS
    if r == _lib.GQA_OK:
        assert N == 0
    if N < 0:
        assert r in REJECTED


@SWEEP
@given(B=sizes, S=sizes, H=heads, G=heads, d=st.sampled_from([-1, 64, 128]),
       steps=st.sampled_from([-1, 0, 1, 2, 256, 257]), dtype=st.sampled_from([0, 1, 7]),
       q=ptrs, sl=st.sampled_from([None, A, A + 2]), out=ptrs,
       append=st.sampled_from([(A, A), (None, None), (A, None)]))
def test_decode_graph_host_checks_sweep(B, S, H, G, d, steps, dtype, q, sl, out, append):
    p = _params(dtype, 0, None, 0, A, 1 << 62)
    p.k_new, p.v_new = append
    g = ctypes.c_void_p()
    lib = _lib.load()
    r = lib.gqa_decode_graph_create_steps(q, A, A, sl, out, B, H, G, d, S, steps,
                                          ctypes.byref(p), ctypes.byref(g))
    assert r in STATUS
    if r == _lib.GQA_OK:
        lib.gqa_decode_graph_destroy(g)
    if B < 0 or S <= 0 or not 1 <= steps <= 256:
        assert r in REJECTED
