"""The C ABI of libgqa.so on the CPU: it loads, exports every function include/gqa.h
declares, sizes workspaces, and rejects bad arguments before any HIP call (no GPU needed:
every call here returns from the host-side checks)."""
import ctypes
import os
import re

import pytest

from attention_head_qk_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa.h")

# Fake device addresses: the checks only look at them, never dereference them.
A = 0x10000
MIS = 0x10008  # 8-byte aligned only


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[\w\s\*]*?\b(gqa_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for fn in ("gqa_prefill", "gqa_prefill_cached", "gqa_decode", "gqa_decode_graph_create",
               "gqa_decode_graph_launch", "gqa_decode_graph_destroy", "gqa_qk_norm_rope",
               "gqa_workspace_bytes", "gqa_status_str", "gqa_params_init", "gqa_decode_split_keys",
               "gqa_rope_freq_table", "gqa_decode_noalloc", "gqa_decode_graph_create_steps"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for fn in declared_functions():
        assert hasattr(lib, fn), fn
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_params_layout_matches_header(tmp_path):
    # the ctypes mirror of gqa_params must have the header's size and field offsets
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f[0] for f in _lib.GqaParams._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"gqa.h\"\nint main(void){\n"
                   + 'printf("size %zu\\n", sizeof(gqa_params));\n'
                   + "".join(f'printf("{f} %zu\\n", offsetof(gqa_params, {f}));\n' for f in fields)
                   + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                      check=True).stdout.splitlines())
    assert int(out["size"]) == ctypes.sizeof(_lib.GqaParams)
    for f in fields:
        assert int(out[f]) == getattr(_lib.GqaParams, f).offset, f


def test_params_init_clears_masks():
    p = _lib.default_params()
    assert p.window == 0 and not p.block_mask and p.block_mask_words == 0


def test_pack_block_mask_bits():
    import numpy as np
    from attention_head_qk_amd import pack_block_mask
    rng = np.random.default_rng(5)
    m = rng.random((7, 70)) < 0.3
    w = pack_block_mask(m).view(np.uint32)
    assert w.shape == (7, 3)
    for qb in range(7):
        for kb in range(96):
            bit = (int(w[qb, kb // 32]) >> (kb % 32)) & 1
            assert bit == (1 if kb < 70 and m[qb, kb] else 0)


def test_rope_table_checked_before_launch():
    bad = (ctypes.c_double * 64)(*([1.0] * 63 + [float("nan")]))
    good = (ctypes.c_double * 64)(*([0.5] * 64))
    short_ok = (ctypes.c_double * 32)(*([0.5] * 31 + [float("inf")]))  # d = 64 reads 32
    assert _prefill(rope_inv_freq=ctypes.cast(bad, ctypes.POINTER(ctypes.c_double))) == _lib.GQA_EINVAL
    assert _decode(rope_inv_freq=ctypes.cast(bad, ctypes.POINTER(ctypes.c_double))) == _lib.GQA_EINVAL
    assert _prefill(rope_inv_freq=ctypes.cast(good, ctypes.POINTER(ctypes.c_double)), B=0) == _lib.GQA_OK
    assert _prefill(d=64, rope_inv_freq=ctypes.cast(short_ok, ctypes.POINTER(ctypes.c_double))) == _lib.GQA_EINVAL


def test_rope_freq_table_matches_the_oracle_tables():
    import numpy as np
    from attention_head_qk_amd import rope_freq_table
    from oracle import gqa_oracle as O
    for d in (64, 128):
        assert np.allclose(rope_freq_table(d, 1e6), O.rope_inv_freq(d, 1e6), rtol=1e-14)
        assert np.allclose(rope_freq_table(d, 1e6, "linear", alpha=4.0),
                           O.inv_freq_linear(d, 1e6, 4.0), rtol=1e-14)
        assert np.allclose(rope_freq_table(d, 1e6, "yarn", train_len=32768, infer_len=131072),
                           O.inv_freq_yarn_page(d, 1e6, 32768, 131072), rtol=1e-12, atol=1e-300)
        assert np.allclose(rope_freq_table(d, 1e6, "ntk", alpha=4.0),
                           O.rope_inv_freq(d, O.ntk_theta(1e6, 4.0, d)), rtol=1e-12)


def test_rope_freq_table_c_function_pinned():
    # gqa_rope_freq_table called through ctypes directly, against the oracle's own rules, at
    # several sizes and arguments, including the YaRN-named rule below the training length
    # (unchanged) and past 2^(1/scale) times it (the lowest frequencies turn negative)
    import numpy as np
    from oracle import gqa_oracle as O
    f = _lib.load().gqa_rope_freq_table

    def table(kind, d, theta=1e6, alpha=1.0, train=0.0, infer=0.0, scale=1.0):
        out = np.full(d // 2, -7.0)
        rc = f(kind, d, theta, alpha, train, infer, scale,
               out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
        return rc, out

    for d in (2, 8, 64, 128):
        for theta in (1e4, 1e6):
            rc, w = table(_lib.GQA_ROPE_BASE, d, theta)
            assert rc == _lib.GQA_OK and np.allclose(w, O.rope_inv_freq(d, theta), rtol=1e-14)
            for alpha in (0.5, 4.0, 16.0):
                rc, w = table(_lib.GQA_ROPE_LINEAR, d, theta, alpha)
                assert rc == _lib.GQA_OK
                assert np.allclose(w, O.inv_freq_linear(d, theta, alpha), rtol=1e-14)
                if d > 2:
                    rc, w = table(_lib.GQA_ROPE_NTK, d, theta, alpha)
                    assert rc == _lib.GQA_OK
                    assert np.allclose(w, O.rope_inv_freq(d, O.ntk_theta(theta, alpha, d)),
                                       rtol=1e-12)
            for train, infer, scale in ((32768, 131072, 1.0), (4096, 32768, 0.5),
                                        (8192, 4096, 1.0), (1000, 1000, 2.0), (2048, 65536, 0.1)):
                rc, w = table(_lib.GQA_ROPE_YARN, d, theta, 1.0, train, infer, scale)
                assert rc == _lib.GQA_OK
                want = O.inv_freq_yarn_page(d, theta, train, infer, scale)
                assert np.allclose(w, want, rtol=1e-12, atol=1e-300), (d, train, infer, scale)
    # errors: nothing written
    for args in ((7, 64, 1e6), (_lib.GQA_ROPE_BASE, 63, 1e6), (_lib.GQA_ROPE_BASE, 130, 1e6),
                 (_lib.GQA_ROPE_BASE, 0, 1e6), (_lib.GQA_ROPE_BASE, 64, 0.0),
                 (_lib.GQA_ROPE_BASE, 64, float("inf")), (_lib.GQA_ROPE_BASE, 64, -1.0)):
        rc, w = table(*args)
        assert rc == _lib.GQA_EINVAL and np.all(w == -7.0), args
    assert table(_lib.GQA_ROPE_LINEAR, 64, 1e6, 0.0)[0] == _lib.GQA_EINVAL
    assert table(_lib.GQA_ROPE_NTK, 64, 1e6, -2.0)[0] == _lib.GQA_EINVAL
    assert table(_lib.GQA_ROPE_NTK, 2, 1e6, 2.0)[0] == _lib.GQA_EINVAL
    assert table(_lib.GQA_ROPE_YARN, 64, 1e6, 1.0, 0.0, 100.0)[0] == _lib.GQA_EINVAL
    assert table(_lib.GQA_ROPE_YARN, 64, 1e6, 1.0, 100.0, 400.0, float("nan"))[0] == _lib.GQA_EINVAL
    assert f(_lib.GQA_ROPE_BASE, 64, 1e6, 1.0, 0.0, 0.0, 1.0, None) == _lib.GQA_EINVAL


def test_binding_computes_no_frequencies():
    # the binding's rope_freq_table marshals only: its source has no power or log of its own
    import inspect
    import attention_head_qk_amd as gqa
    src = inspect.getsource(gqa.rope_freq_table)
    for token in ("**", "np.power", "np.log", "math.", "np.arange"):
        assert token not in src, token


def test_binding_shape_checks():
    # the checks that keep a wrong shape from becoming an out-of-bounds device access; they
    # look at shapes only, so CPU tensors serve
    import numpy as np
    import torch
    import attention_head_qk_amd as gqa
    t = torch.zeros(4, 3, 8)
    gqa._shape(t, "t", (4, 3, 8))
    gqa._shape(t, "t", 96)
    gqa._shape(None, "t", (1,))
    for bad in ((4, 3, 7), (3, 4, 8), (4, 24), 95):
        with pytest.raises(ValueError):
            gqa._shape(t, "t", bad)
    assert gqa._rope_table(np.ones(64), 128).shape == (64,)
    for bad in (np.ones(63), np.ones(65), np.ones((8, 8)), np.ones(32)):
        with pytest.raises(ValueError):
            gqa._rope_table(bad, 128)
    bm = torch.zeros(64, 2, dtype=torch.int32)
    gqa._block_mask_check(bm, 4096)
    gqa._block_mask_check(bm, 64 * 64)
    with pytest.raises(ValueError):
        gqa._block_mask_check(bm, 64 * 64 + 1)  # one query block too many
    with pytest.raises(ValueError):
        gqa._block_mask_check(torch.zeros(130, 4, dtype=torch.int32), 130 * 64)  # 5 words needed
    with pytest.raises(ValueError):
        gqa._block_mask_check(torch.zeros(64, dtype=torch.int32), 64)


def test_decode_noalloc_host_checks():
    # the allocation-free decode makes every host check of gqa_decode (here with fake device
    # addresses, so only rejections and the empty batch are called) and refuses decodes whose
    # scratch would not fit its fixed array
    lib = _lib.load()
    f = lib.gqa_decode_noalloc
    p = _lib.default_params()
    sl = ctypes.c_void_p(A)
    assert f(A, A, A, sl, A, 2, 6, 4, 128, 64, ctypes.byref(p)) == _lib.GQA_EINVAL   # H % G
    assert f(A, A, A, sl, A, 2, 8, 8, 96, 64, ctypes.byref(p)) == _lib.GQA_ENOTSUP   # d
    assert f(A, A, A, None, A, 2, 8, 8, 128, 64, ctypes.byref(p)) == _lib.GQA_EINVAL
    assert f(MIS, A, A, sl, A, 2, 8, 8, 128, 64, ctypes.byref(p)) == _lib.GQA_EINVAL
    assert f(A, A, A, sl, A, 0, 8, 8, 128, 64, ctypes.byref(p)) == _lib.GQA_OK       # no work
    assert f(A, A, A, sl, A, 2, 8, 8, 128, 64, None) == _lib.GQA_EINVAL
    need = lib.gqa_workspace_bytes(_lib.GQA_OP_DECODE, 64, 65536, 64, 8, 128, _lib.GQA_BF16)
    assert need > _lib.GQA_DECODE_NOALLOC_MAX_BYTES
    assert f(A, A, A, sl, A, 64, 64, 8, 128, 65536, ctypes.byref(p)) == _lib.GQA_EWORKSPACE
    # p->workspace is ignored: a caller workspace that is too small changes nothing
    p.workspace = ctypes.c_void_p(A)
    p.workspace_bytes = 1
    assert f(A, A, A, sl, A, 0, 8, 8, 128, 64, ctypes.byref(p)) == _lib.GQA_OK


def test_status_strings():
    for code, tag in [(0, "GQA_OK"), (1, "GQA_EINVAL"), (2, "GQA_ENOTSUP"),
                      (3, "GQA_EWORKSPACE"), (4, "GQA_EHIP")]:
        assert _lib.status_str(code).startswith(tag)


def test_params_init_defaults():
    p = _lib.default_params()
    assert p.dtype == _lib.GQA_BF16
    assert abs(p.eps - 1e-6) < 1e-12 and p.rope_theta == 1e6 and p.scale == 0.0
    assert not p.workspace and not p.stream and not p.cu_seqlens


def test_workspace_bytes():
    lib = _lib.load()
    ws = lib.gqa_workspace_bytes
    # prefill: k~ [N,G,d] in the element type (fp32 also q~ [N,H,d]), each rounded up to
    # 256 bytes; the bf16 attention kernel prepares Q itself and has G block counters, and
    # grids of at most 512 workgroups (B G ceil(T h / 128)) may run the paired schedule: one
    # counter and two fp32 partial states (128 columns x (d + 2)) per pair of column blocks
    def part(pairs, d):
        return pairs * 2 * (128 * d + 256) * 4
    pairs = 8 * 32                                       # T=4096, h=2: 64 blocks per group
    assert ws(_lib.GQA_OP_PREFILL, 1, 4096, 16, 8, 128, _lib.GQA_BF16) == (
        4096 * 8 * 128 * 2 + 1280 + part(pairs, 128))    # (8 + 256) counters -> 1280 bytes
    assert ws(_lib.GQA_OP_PREFILL, 1, 3, 2, 1, 64, _lib.GQA_F32) == 1536 + 768
    assert ws(_lib.GQA_OP_PREFILL, 1, 3, 1, 1, 64, _lib.GQA_BF16) == 512 + 256 + part(1, 64)
    # a grid of more than 512 workgroups (T=32768, h=16: 4096 blocks x 4 groups): no pairs
    assert ws(_lib.GQA_OP_PREFILL, 1, 32768, 64, 4, 128, _lib.GQA_BF16) == 32768 * 4 * 256 + 256
    # the boundary: T=4097 gives 65 blocks per group, 520 workgroups: no pairs; a dense batch
    # of two at T=2048 (2 x 8 x 32 = 512 workgroups) keeps them, 16 blocks' pairs per sequence
    def up(n):
        return -(-n // 256) * 256
    assert ws(_lib.GQA_OP_PREFILL, 1, 4097, 16, 8, 128, _lib.GQA_BF16) == (
        up(4097 * 8 * 128 * 2) + 256)
    assert ws(_lib.GQA_OP_PREFILL, 2, 2048, 16, 8, 128, _lib.GQA_BF16) == (
        2 * 2048 * 8 * 128 * 2 + up((8 + 2 * 8 * 16) * 4) + part(2 * 8 * 16, 128))
    # odd block counts round the pairs up (the middle block has no partner): T=4000, h=4
    # gives 125 blocks per group, 63 pairs
    assert ws(_lib.GQA_OP_PREFILL, 1, 4000, 8, 2, 128, _lib.GQA_BF16) == (
        up(4000 * 2 * 128 * 2) + up((2 + 2 * 63) * 4) + part(2 * 63, 128))
    # decode: q~ + fp32 partial O + fp32 (m, l) per split + two [B] step-length buffers
    S = lib.gqa_decode_split_keys(64, 32, 8, 32768)
    assert S == 1024
    ns = -(-32768 // S)
    want = 64 * 32 * 128 * 2 + 64 * 32 * ns * 128 * 4 + 64 * 32 * ns * 2 * 4 + 2 * 256
    assert ws(_lib.GQA_OP_DECODE, 64, 32768, 32, 8, 128, _lib.GQA_BF16) == want
    assert ws(_lib.GQA_OP_QK_NORM_ROPE, 4, 4, 4, 4, 128, _lib.GQA_BF16) == 0
    assert ws(_lib.GQA_OP_PREFILL, 1, 8, 6, 4, 128, _lib.GQA_BF16) == 0  # H % G != 0
    assert ws(_lib.GQA_OP_PREFILL, 1, 8, 8, 4, 96, _lib.GQA_BF16) == 0   # d unsupported


def test_decode_split_rule():
    f = _lib.load().gqa_decode_split_keys
    assert f(64, 32, 8, 32768) == 1024            # 16384 blocks at 1024 keys
    assert f(16, 32, 8, 16384) == 1024            # exactly 2048 blocks
    assert f(16, 32, 8, 16383) == 1024
    assert f(16, 32, 8, 8192) == 512              # 1024 blocks at 1024 keys, 2048 at 512
    assert f(16, 32, 8, 4096) == 256
    assert f(13, 32, 8, 3100) == 256              # stops at the shortest split
    assert f(1, 64, 1, 32768) == 256              # MQA: 2 head tiles of 32
    assert f(256, 64, 1, 32768) == 1024           # 256 x 2 x 32 blocks
    assert f(0, 32, 8, 100) == 0 and f(4, 6, 4, 100) == 0 and f(4, 8, 4, 0) == 0
    ws = _lib.load().gqa_workspace_bytes
    # the workspace follows the split: 16 splits of 256 keys at max_seq 4096
    assert ws(_lib.GQA_OP_DECODE, 16, 4096, 32, 8, 128, _lib.GQA_BF16) == (
        16 * 32 * 128 * 2 + 16 * 32 * 16 * 128 * 4 + 16 * 32 * 16 * 2 * 4 + 2 * 256)


def _params(**kw):
    p = _lib.default_params()
    p.workspace = A
    p.workspace_bytes = 1 << 40
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _prefill(q=A, k=A, v=A, pos=None, out=A, B=1, T=8, H=4, G=2, d=128, causal=1, **kw):
    p = _params(**kw)
    return _lib.load().gqa_prefill(q, k, v, pos, out, B, T, H, G, d, causal, ctypes.byref(p))


def _decode(q=A, kc=A, vc=A, sl=A, out=A, B=2, H=4, G=2, d=128, S=16, **kw):
    p = _params(**kw)
    return _lib.load().gqa_decode(q, kc, vc, sl, out, B, H, G, d, S, ctypes.byref(p))


def test_prefill_mask_checks():
    # window needs the causal mask and a non-negative size; block_mask needs 4-byte alignment
    # and rows wide enough for T keys; both are bf16 only
    assert _prefill(window=-1) == _lib.GQA_EINVAL
    assert _prefill(window=4, causal=0) == _lib.GQA_EINVAL
    assert _prefill(block_mask=A + 2, block_mask_words=1) == _lib.GQA_EINVAL
    assert _prefill(block_mask=A, block_mask_words=0) == _lib.GQA_EINVAL
    assert _prefill(T=2049, block_mask=A, block_mask_words=1) == _lib.GQA_EINVAL  # 33 blocks
    assert _prefill(T=2048, block_mask=A, block_mask_words=1, B=0) == _lib.GQA_OK
    assert _prefill(window=4, dtype=_lib.GQA_F32) == _lib.GQA_ENOTSUP
    assert _prefill(block_mask=A, block_mask_words=1, dtype=_lib.GQA_F32) == _lib.GQA_ENOTSUP
    assert _prefill(window=4, B=0) == _lib.GQA_OK
    assert _prefill_cached(window=4, causal=0) == _lib.GQA_EINVAL
    assert _prefill_cached(S=2049, block_mask=A, block_mask_words=1) == _lib.GQA_EINVAL
    assert _prefill_cached(window=3, B=0) == _lib.GQA_OK
    assert _decode(window=8) == _lib.GQA_ENOTSUP
    assert _decode(block_mask=A, block_mask_words=4) == _lib.GQA_ENOTSUP


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.GQA_EINVAL), (dict(k=None), _lib.GQA_EINVAL),
    (dict(v=None), _lib.GQA_EINVAL), (dict(out=None), _lib.GQA_EINVAL),
    (dict(q=MIS), _lib.GQA_EINVAL), (dict(out=MIS), _lib.GQA_EINVAL),
    (dict(pos=A + 2), _lib.GQA_EINVAL),
    (dict(H=6, G=4), _lib.GQA_EINVAL), (dict(H=0), _lib.GQA_EINVAL), (dict(G=0), _lib.GQA_EINVAL),
    (dict(B=-1), _lib.GQA_EINVAL), (dict(T=-3), _lib.GQA_EINVAL), (dict(causal=2), _lib.GQA_EINVAL),
    (dict(d=96), _lib.GQA_ENOTSUP), (dict(d=256), _lib.GQA_ENOTSUP),
    (dict(dtype=7), _lib.GQA_ENOTSUP),
    (dict(eps=-1.0), _lib.GQA_EINVAL), (dict(scale=-0.5), _lib.GQA_EINVAL),
    (dict(rope_theta=float("nan")), _lib.GQA_EINVAL),
    (dict(q_norm_w=A + 4), _lib.GQA_EINVAL), (dict(cu_seqlens=A + 1), _lib.GQA_EINVAL),
    (dict(workspace=None), _lib.GQA_EWORKSPACE), (dict(workspace_bytes=100), _lib.GQA_EWORKSPACE),
    (dict(B=0), _lib.GQA_OK), (dict(T=0), _lib.GQA_OK), (dict(B=0, q=None), _lib.GQA_OK),
    (dict(B=65536, T=1, dtype=_lib.GQA_F32), _lib.GQA_ENOTSUP),  # fp32 grid: B on dimension z
])
def test_prefill_rejects_before_launch(kw, code):
    assert _prefill(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.GQA_EINVAL), (dict(kc=None), _lib.GQA_EINVAL),
    (dict(vc=MIS), _lib.GQA_EINVAL), (dict(sl=None), _lib.GQA_EINVAL),
    (dict(sl=A + 2), _lib.GQA_EINVAL), (dict(out=None), _lib.GQA_EINVAL),
    (dict(S=0), _lib.GQA_EINVAL), (dict(S=-1), _lib.GQA_EINVAL),
    (dict(H=5, G=2), _lib.GQA_EINVAL), (dict(d=32), _lib.GQA_ENOTSUP),
    (dict(k_new=A), _lib.GQA_EINVAL), (dict(v_new=A), _lib.GQA_EINVAL),
    (dict(k_new=MIS, v_new=A), _lib.GQA_EINVAL), (dict(positions=A + 1), _lib.GQA_EINVAL),
    (dict(workspace_bytes=10), _lib.GQA_EWORKSPACE),
    (dict(B=0), _lib.GQA_OK), (dict(B=-2), _lib.GQA_EINVAL),
    (dict(B=65536), _lib.GQA_ENOTSUP),  # sequences index a grid dimension of <= 65535
])
def test_decode_rejects_before_launch(kw, code):
    assert _decode(**kw) == code


def _prefill_cached(q=A, k=A, v=A, kc=A, vc=A, cl=A, pos=None, out=A, B=2, T=8, H=4, G=2,
                    d=128, S=64, causal=1, **kw):
    p = _params(**kw)
    return _lib.load().gqa_prefill_cached(q, k, v, kc, vc, cl, pos, out, B, T, H, G, d, S, causal,
                                          ctypes.byref(p))


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.GQA_EINVAL), (dict(k=None), _lib.GQA_EINVAL),
    (dict(v=MIS), _lib.GQA_EINVAL), (dict(kc=None), _lib.GQA_EINVAL),
    (dict(vc=MIS), _lib.GQA_EINVAL), (dict(cl=None), _lib.GQA_EINVAL),
    (dict(cl=A + 2), _lib.GQA_EINVAL), (dict(pos=A + 1), _lib.GQA_EINVAL),
    (dict(out=None), _lib.GQA_EINVAL), (dict(S=0), _lib.GQA_EINVAL),
    (dict(causal=3), _lib.GQA_EINVAL), (dict(H=6, G=4), _lib.GQA_EINVAL),
    (dict(d=96), _lib.GQA_ENOTSUP), (dict(dtype=_lib.GQA_F32), _lib.GQA_ENOTSUP),
    (dict(S=1 << 20, H=8, G=8), _lib.GQA_ENOTSUP),  # one sequence's cache rows past 2^31 bytes
    (dict(cu_seqlens=A + 1), _lib.GQA_EINVAL),
    (dict(B=0), _lib.GQA_OK), (dict(T=0, q=None), _lib.GQA_OK), (dict(B=-1), _lib.GQA_EINVAL),
])
def test_prefill_cached_rejects_before_launch(kw, code):
    assert _prefill_cached(**kw) == code


def _graph_create(q=A, kc=A, vc=A, sl=A, out=A, B=2, H=4, G=2, d=128, S=16, out_handle=True,
                  steps=None, **kw):
    kw.setdefault("k_new", A)
    kw.setdefault("v_new", A)
    p = _params(**kw)
    h = ctypes.c_void_p()
    hp = ctypes.byref(h) if out_handle else None
    if steps is None:
        rc = _lib.load().gqa_decode_graph_create(q, kc, vc, sl, out, B, H, G, d, S,
                                                 ctypes.byref(p), hp)
    else:
        rc = _lib.load().gqa_decode_graph_create_steps(q, kc, vc, sl, out, B, H, G, d, S, steps,
                                                       ctypes.byref(p), hp)
    assert not h.value  # nothing is created on a rejected call
    return rc


@pytest.mark.parametrize("kw,code", [
    (dict(out_handle=False), _lib.GQA_EINVAL),
    (dict(k_new=None), _lib.GQA_EINVAL), (dict(v_new=None), _lib.GQA_EINVAL),
    (dict(k_new=None, v_new=None), _lib.GQA_EINVAL),
    (dict(q=None), _lib.GQA_EINVAL), (dict(sl=None), _lib.GQA_EINVAL),
    (dict(S=0), _lib.GQA_EINVAL), (dict(H=5, G=2), _lib.GQA_EINVAL),
    (dict(d=96), _lib.GQA_ENOTSUP), (dict(workspace_bytes=10), _lib.GQA_EWORKSPACE),
    (dict(positions=A + 2), _lib.GQA_EINVAL), (dict(B=-1), _lib.GQA_EINVAL),
    (dict(steps=0), _lib.GQA_EINVAL), (dict(steps=257), _lib.GQA_EINVAL),
    (dict(steps=-3), _lib.GQA_EINVAL), (dict(steps=8, k_new=None), _lib.GQA_EINVAL),
    (dict(steps=8, d=96), _lib.GQA_ENOTSUP), (dict(steps=2, workspace_bytes=10), _lib.GQA_EWORKSPACE),
])
def test_decode_graph_create_rejects_before_any_hip_call(kw, code):
    assert _graph_create(**kw) == code


def test_decode_graph_launch_and_destroy_null():
    lib = _lib.load()
    assert lib.gqa_decode_graph_launch(None, None) == _lib.GQA_EINVAL
    assert lib.gqa_decode_graph_destroy(None) == _lib.GQA_OK


def test_qk_norm_rope_rejects_before_launch():
    lib = _lib.load()
    p = _params()
    f = lib.gqa_qk_norm_rope
    assert f(None, None, None, A, None, 4, 4, 2, 128, ctypes.byref(p)) == _lib.GQA_EINVAL
    assert f(A, A, None, A, None, 4, 4, 2, 128, ctypes.byref(p)) == _lib.GQA_EINVAL
    assert f(A, None, None, A, None, 4, 4, 2, 80, ctypes.byref(p)) == _lib.GQA_ENOTSUP
    assert f(A, None, None, A, None, -1, 4, 2, 128, ctypes.byref(p)) == _lib.GQA_EINVAL
    assert f(A, None, None, A, None, 0, 4, 2, 128, ctypes.byref(p)) == _lib.GQA_OK
    assert f(A, None, None, A, None, 4, 4, 2, 128, None) == _lib.GQA_EINVAL


def test_c_client_compiles_and_links():
    # the header is plain C: tests/c_abi/client.c (the GPU test's C client) builds with gcc
    # against include/gqa.h and links libgqa.so and the HIP runtime
    import shutil
    import subprocess
    import tempfile
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no gcc")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg = os.path.join(root, "attention_head_qk_amd")
    with tempfile.TemporaryDirectory() as t:
        r = subprocess.run([cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                            "-I", os.path.join(root, "include"), "-I", "/opt/rocm/include",
                            os.path.join(root, "tests", "c_abi", "client.c"), "-L", pkg, "-lgqa",
                            "-L", "/opt/rocm/lib", "-lamdhip64", "-o", os.path.join(t, "client")],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
