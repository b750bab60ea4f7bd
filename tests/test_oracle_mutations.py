"""Mutation check of the oracle's pins (CPU only): each case plants one plausible mistake in
a copy of the oracle (a dropped term, a wrong sign or index, a transposed operand, an
off-by-one mask or cache slot, a wrong frequency rule) and runs the oracle pins
(tests/test_oracle.py) against that copy in a subprocess; every planted mistake must make
some pin fail. The repository's own oracle is never modified."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (what the mistake is, exact text in oracle/gqa_oracle.py, replacement)
MUTATIONS = [
    ("RMSNorm sums instead of averaging", "ms = np.mean(x * x, axis=-1, keepdims=True)",
     "ms = np.sum(x * x, axis=-1, keepdims=True)"),
    ("RMSNorm drops eps", "x / np.sqrt(ms + eps)", "x / np.sqrt(ms)"),
    ("RoPE frequency exponent halved", "np.power(float(theta), -2.0 * j / d)",
     "np.power(float(theta), -1.0 * j / d)"),
    ("RoPE even lane sign", "y[..., 0::2] = a * c - b * s", "y[..., 0::2] = a * c + b * s"),
    ("RoPE odd lane sign", "y[..., 1::2] = a * s + b * c", "y[..., 1::2] = -a * s + b * c"),
    ("RoPE split-half pairing", "a = x[..., 0::2]\n    b = x[..., 1::2]",
     "a = x[..., :d // 2]\n    b = x[..., d // 2:]"),
    ("RoPE before the norm", "qt = rope(rms_norm(q, q_norm_w, eps), positions, theta)",
     "qt = rms_norm(rope(q, positions, theta), q_norm_w, eps)"),
    ("score scale 1/d", "return 1.0 / np.sqrt(d) if not scale", "return 1.0 / d if not scale"),
    ("causal mask drops the diagonal", "vis &= j <= i\n", "vis &= j < i\n"),
    ("transposed scores", "S = (qt_i @ kt_g.T)", "S = (kt_g @ qt_i.T)"),
    ("head i reads group i mod G", "g = i // h\n        P = attention_weights(qt[:, i, :]",
     "g = i % G\n        P = attention_weights(qt[:, i, :]"),
    ("softmax over columns", "return E / np.sum(E, axis=-1, keepdims=True)",
     "return E / np.sum(E, axis=0, keepdims=True)"),
    ("every head reads V head 0", "out[:, i, :] = P @ v[:, g, :]", "out[:, i, :] = P @ v[:, 0, :]"),
    ("gamma_q applied to K", "kt = rope(rms_norm(k, k_norm_w, eps), positions, theta)",
     "kt = rope(rms_norm(k, q_norm_w, eps), positions, theta)"),
    ("decode position one past the token", "pos = slot if position is None else int(position)",
     "pos = L if position is None else int(position)"),
    ("sampled rows ignore the causal mask",
     "vis = visible_keys(len(r_in[c]), Tk, causal, window, block_mask, block,",
     "vis = visible_keys(len(r_in[c]), Tk, False, window, block_mask, block,"),
    ("sampled rows pair a head with another row's mask",
     "S = np.where(np.repeat(vis, h, axis=0), S, -np.inf)",
     "S = np.where(np.tile(vis, (h, 1)), S, -np.inf)"),
    ("cached positions restart at 0", "pos = (past + np.arange(e - s))", "pos = (np.arange(e - s))"),
    ("appended rows one slot late", "kc[b, past:past + e - s] = kt",
     "kc[b, past + 1:past + 1 + e - s] = kt"),
    ("decode step one key short", "L = int(cache_lens[b]) + s + 1", "L = int(cache_lens[b]) + s"),
    ("decode step writes K one slot early", "kc[b, L - 1] = k_slot", "kc[b, L - 2] = k_slot"),
    ("decode step writes V one slot late", "vc[b, L - 1] = v_slot",
     "vc[b, min(L, vc.shape[1] - 1)] = v_slot"),
    ("window one key too wide", "vis &= j > i - int(window)", "vis &= j >= i - int(window)"),
    ("linear interpolation multiplies", "return rope_inv_freq(d, theta) / float(alpha)",
     "return rope_inv_freq(d, theta) * float(alpha)"),
    ("YaRN-named rule: natural log", "s = float(scale) * np.log(infer_len / train_len) / np.log(2.0)",
     "s = float(scale) * np.log(infer_len / train_len)"),
    ("YaRN-named rule: j instead of 2j",
     "w = w * (1.0 - s * (2.0 * np.arange(d // 2, dtype=np.float64) / d))",
     "w = w * (1.0 - s * (np.arange(d // 2, dtype=np.float64) / d))"),
    ("NTK base exponent inverted", "return float(theta) * float(alpha) ** (d / (d - 2.0))",
     "return float(theta) * float(alpha) ** ((d - 2.0) / d)"),
    ("frequency table ignored", "    w = np.asarray(theta, dtype=np.float64)\n    if w.shape",
     "    w = rope_inv_freq(d, 1e6)\n    if w.shape"),
    ("block layout drops the diagonal block",
     "vis &= bm[i // block, j // block] | (i // block == j // block)",
     "vis &= bm[i // block, j // block]"),
    ("block layout transposed", "vis &= bm[i // block, j // block] | (i // block == j // block)",
     "vis &= bm[j // block, i // block] | (i // block == j // block)"),
    ("softmax without the row maximum", "    E = np.exp(S - m)\n", "    E = np.exp(S)\n"),
    ("decode head i reads group i mod G",
     "        g = i // h\n        p = attention_weights(qt[i:i + 1]",
     "        g = i % G\n        p = attention_weights(qt[i:i + 1]"),
    ("decode appends K without its norm",
     "k_slot = rope(rms_norm(np.asarray(k_new, np.float64)[None], k_norm_w, eps),",
     "k_slot = rope(np.asarray(k_new, np.float64)[None],"),
    ("decode query rotated at position 0",
     "qt = rope(rms_norm(np.asarray(q_b, np.float64)[None], q_norm_w, eps), np.array([pos]),",
     "qt = rope(rms_norm(np.asarray(q_b, np.float64)[None], q_norm_w, eps), np.array([0]),"),
    ("decode keeps the stale V slot", "        vc[slot] = v_slot\n", "        pass\n"),
    ("sampled rows ignore the window",
     "vis = visible_keys(len(r_in[c]), Tk, causal, window, block_mask, block,",
     "vis = visible_keys(len(r_in[c]), Tk, causal, 0, block_mask, block,"),
]


@pytest.mark.parametrize("what,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(what, old, new, tmp_path):
    for sub in ("oracle", "tests"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub,
                        ignore=shutil.ignore_patterns("__pycache__"))
    for f in ("workloads.py", "pytest.ini"):
        shutil.copy(os.path.join(ROOT, f), tmp_path / f)
    path = tmp_path / "oracle" / "gqa_oracle.py"
    src = path.read_text()
    assert old in src, f"mutation site not found: {what}"
    path.write_text(src.replace(old, new, 1))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle.py"], cwd=tmp_path, capture_output=True, text=True,
                       env=env, timeout=600)
    assert r.returncode != 0, f"no pin failed with the planted mistake: {what}\n{r.stdout[-2000:]}"
