"""gqa_decode_noalloc (the decode entry point that allocates nothing: its scratch is a fixed
device array inside the library) against gqa_decode with a caller workspace, both called
through the C ABI with ctypes: two calls in a row, the second on a smaller input, each bit for
bit equal to gqa_decode on the same inputs (same kernels, same order of arithmetic); plus the
size limit and the host checks."""
import ctypes

import pytest
import torch

import workloads as W

from _gpu import device_decode_inputs, say

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _params(dev, case, stream, workspace=None, append=True):
    from attention_head_qk_amd import _lib
    p = _lib.default_params()
    p.dtype = _lib.GQA_BF16 if case.dtype == W.BF16 else _lib.GQA_F32
    p.q_norm_w = _ptr(dev["q_norm_w"])
    p.k_norm_w = _ptr(dev["k_norm_w"])
    p.eps = case.eps
    p.rope_theta = case.theta
    if append:
        p.k_new = _ptr(dev["k_new"])
        p.v_new = _ptr(dev["v_new"])
    if workspace is not None:
        p.workspace = _ptr(workspace)
        p.workspace_bytes = workspace.numel()
    p.stream = ctypes.c_void_p(stream.cuda_stream)
    return p


def _call(fn, dev, case, out, p):
    return fn(_ptr(dev["q"]), _ptr(dev["k_cache"]), _ptr(dev["v_cache"]), _ptr(dev["seq_lens"]),
              _ptr(out), case.B, case.H, case.G, case.d, case.max_seq, ctypes.byref(p))


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_noalloc_equals_workspace_decode(dtype):
    from attention_head_qk_amd import _lib
    lib = _lib.load()
    stream = torch.cuda.current_stream()
    cases = [W.make_decode("noalloc_big", 601, B=24, max_seq=20000, H=32, G=8, d=128, dtype=dtype,
                           len_range=(1, 20000)),
             W.make_decode("noalloc_small", 602, B=3, max_seq=700, H=16, G=4, d=64, dtype=dtype,
                           seq_lens=[700, 1, 333])]
    for n, case in enumerate(cases):
        say("decode_noalloc call", n, case.name, dtype)
        need = lib.gqa_workspace_bytes(_lib.GQA_OP_DECODE, case.B, case.max_seq, case.H, case.G,
                                       case.d, _lib.GQA_BF16 if dtype == W.BF16 else _lib.GQA_F32)
        assert 0 < need <= _lib.GQA_DECODE_NOALLOC_MAX_BYTES
        dev_a = device_decode_inputs(case)
        dev_b = {k: v.clone() for k, v in dev_a.items()}
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        out_a = torch.empty_like(dev_a["q"])
        out_b = torch.full_like(dev_b["q"], float("nan"))
        rc = _call(lib.gqa_decode, dev_a, case, out_a, _params(dev_a, case, stream, ws))
        assert rc == _lib.GQA_OK
        rc = _call(lib.gqa_decode_noalloc, dev_b, case, out_b, _params(dev_b, case, stream))
        assert rc == _lib.GQA_OK
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), f"call {n}: outputs differ"
        assert torch.equal(dev_a["k_cache"], dev_b["k_cache"]), f"call {n}: appended K differs"
        assert torch.equal(dev_a["v_cache"], dev_b["v_cache"]), f"call {n}: appended V differs"


def test_noalloc_limits_and_checks():
    from attention_head_qk_amd import _lib
    lib = _lib.load()
    stream = torch.cuda.current_stream()
    # 64 sequences x 64 heads over a 65536-row cache need more scratch than the array holds:
    # refused before anything is enqueued (the pointers are never touched)
    case = W.make_decode("noalloc_huge", 603, B=64, max_seq=65536, H=64, G=8, d=128,
                         seq_lens=[1] * 64)
    need = lib.gqa_workspace_bytes(_lib.GQA_OP_DECODE, 64, 65536, 64, 8, 128, _lib.GQA_BF16)
    assert need > _lib.GQA_DECODE_NOALLOC_MAX_BYTES
    fake = {k: torch.empty(16, dtype=torch.bfloat16, device="cuda")
            for k in ("q", "k_cache", "v_cache", "q_norm_w", "k_norm_w", "k_new", "v_new")}
    fake["seq_lens"] = torch.ones(64, dtype=torch.int32, device="cuda")
    out = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    say("decode_noalloc size limit")
    rc = _call(lib.gqa_decode_noalloc, fake, case, out, _params(fake, case, stream))
    assert rc == _lib.GQA_EWORKSPACE
    # the host checks of gqa_decode apply unchanged
    small = W.make_decode("noalloc_chk", 604, B=2, max_seq=64, H=6, G=4, d=128, seq_lens=[1, 1])
    assert _call(lib.gqa_decode_noalloc, fake, small, out, _params(fake, small, stream)) == \
        _lib.GQA_EINVAL  # H % G != 0
    assert lib.gqa_decode_noalloc(None, None, None, None, None, 0, 8, 8, 128, 64, None) == \
        _lib.GQA_EINVAL
