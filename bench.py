#!/usr/bin/env python3
"""Benchmark of the causal GQA hot path (QK-RMSNorm + RoPE prologue, prefill attention,
decode split-KV + combine) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload default|...]

Default workload. A step is one pass of the whole path over one batch of synthetic input,
inputs resident in HBM before the timed region: gqa_prefill on the bf16 long prefill
(B=1, T=32768, H=64, G=4, d=128, causal, gamma ~ U(0.5, 1.5), theta 1e6: the largest
single-GPU configuration), then gqa_decode on 64 sequences x 1 new token with cache lengths
U{1024..32768}, H=32, G=8, d=128 (the new token's K/V appended first). Prints one JSON line:

* value: TFLOP/s of the whole gqa_prefill call (prologue + attention) on the long prefill,
  algorithmic FLOPs 4*d*H*sum T_b(T_b+1)/2, from the median of per-call HIP-event times.
* roofline: the prefill attention kernel alone on that workload (HIP events the library
  records right around its launch, on the launch stream; achieved = FLOPs / mean duration),
  against the 2.5 PFLOP/s bf16 dense MFMA peak; traffic from the rocprofv3 counter record in
  profiles/ while the kernel's sources are unchanged, else null.
* configs: every configuration measured the same way -- the long prefill with G=4 and with
  G=1 (MQA), the 8-sequence varlen prefill (H=32, G=8), the T=4096 prefill (H=16, G=8), the
  tiny fp32 prefill and the 64-sequence decode -- each with the whole call and its main
  kernel (median, min, mean), the rate and the fraction of the roofline.
* clocks: shader and memory clock samples (sysfs) taken during the timed loops, when the
  device exposes them.
* cpu_baseline: the fp64 CPU oracle, unchanged, timed on the host's cores (a pool of
  processes forked before the GPU is touched, one BLAS thread each) on a bounded sample of
  every configuration, scaled to the full configuration and labelled so.

Other workloads (--workload): tiny_f32, prefill_4k, varlen, decode, long_g4, long_g1 (one
configuration each), long_window / long_blocks (the T=32768 G=4 prefill with a 512-key window
or a 64-key block layout; FLOPs count the visible pairs only), chunked (gqa_prefill_cached: 4
sequences, each a 2048-token chunk after a cached prefix of U{2048..14336}), decode_loop (a
generation loop replayed as a HIP graph against the eager step), copy_calibration (a 1 GiB
device copy for scaling the rocprofv3 byte counters).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3    # vector fp32: 256 CUs x 128 FMA lanes per clock x 2 FLOP x 2.4 GHz
HBM_PEAK_GBS = 8000.0

WORKLOADS = ("default", "tiny_f32", "prefill_4k", "varlen", "decode", "long_g4", "long_g1",
             "long_window", "long_blocks", "chunked", "decode_loop", "copy_calibration")
WINDOW = 512          # sliding-window workload: keys per query
BLOCK_DENSITY = 0.1   # block-sparse workload: share of earlier 64-key blocks kept
ROPE_ALPHA = {"linear": 4.0, "ntk": 8.0, "yarn": 1.0}  # --rope-scaling extension factors
COPY_BYTES = 1 << 30  # bytes read (and written) per step of the copy calibration
MAX_POOL = 16         # CPU workers of the oracle baseline: at most one GPU's share of the host

TRAFFIC_RECORDS = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the rocprofv3 FETCH_SIZE /
    WRITE_SIZE record kept in profiles/ (KiB per dispatch, each scaled by the factor the same
    counter gives for a plain copy of known size). None when there is no record, or when the
    kernel's sources have changed since the counters were taken (sha256 of those files)."""
    import hashlib
    try:
        text = open(TRAFFIC_RECORDS).read()
    except OSError:
        return None
    for line in text.splitlines():
        line = line.strip().strip("`")
        if not line.startswith("record:"):
            continue
        rec = dict(kv.split("=", 1) for kv in line[len("record:"):].split())
        if rec.get("kernel") != kernel or rec.get("workload") != workload:
            continue
        h = hashlib.sha256()
        for rel in rec["sources"].split(","):
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["sha256"]:
            return None
        return (float(rec["fetch_kib"]) * float(rec["fetch_factor"]) +
                float(rec["write_kib"]) * float(rec["write_factor"])) * 1024.0
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_case(name):
    import workloads as W
    return {"tiny_f32": W.tiny_f32, "prefill_4k": W.prefill_4k, "varlen": W.prefill_varlen,
            "long_g4": lambda: W.prefill_long(4), "long_g1": lambda: W.prefill_long(1),
            "long_window": lambda: W.prefill_long(4),
            "long_blocks": lambda: W.prefill_long(4)}[name]()


def visible_pairs(lengths, window=0, block_mask=None):
    """(query, key) pairs a causal prefill with these masks must compute, per head: the
    algorithmic work of the mask variants (64-key blocks, the diagonal block always kept)."""
    import numpy as np
    total = 0
    for T in (int(t) for t in lengths):
        i = np.arange(T, dtype=np.int64)
        if block_mask is None:
            lo = np.maximum(0, i - window + 1) if window else np.zeros(T, np.int64)
            total += int(np.sum(i - lo + 1))
            continue
        for qb in range(-(-T // 64)):
            rows = np.arange(64 * qb, min(T, 64 * qb + 64))
            lo = np.maximum(0, rows - window + 1) if window else np.zeros(len(rows), np.int64)
            kb = np.flatnonzero(block_mask[qb, :qb + 1] | (np.arange(qb + 1) == qb))
            for k in kb:  # keys [64 k, 64 k + 64) intersected with [lo, row]
                a = np.maximum(lo, 64 * k)
                b = np.minimum(rows, 64 * k + 63)
                total += int(np.sum(np.maximum(0, b - a + 1)))
    return total


# ----------------------------------------------------------------------------- GPU calls
class Prefill:
    def __init__(self, case, window=0, block_mask=None, rope_inv_freq=None):
        import torch
        import attention_head_qk_amd as gqa
        from workloads import device_prefill_inputs
        self.case = case
        self.dev = device_prefill_inputs(case)
        self.gqa = gqa
        c = case
        self.ws = torch.empty(gqa.workspace_bytes("prefill", c.B, max(c.T_max, 1), c.H, c.G, c.d,
                                                  self.dev["q"].dtype), dtype=torch.uint8,
                              device="cuda")
        self.out = torch.empty_like(self.dev["q"])
        self.window = window
        self.block_mask = block_mask
        self.masks = {}
        self.rope = {} if rope_inv_freq is None else {"rope_inv_freq": rope_inv_freq}
        if window:
            self.masks["window"] = window
        if block_mask is not None:
            self.masks["block_mask"] = torch.from_numpy(gqa.pack_block_mask(block_mask)).cuda()

    def __call__(self, prof=None):
        c, dv = self.case, self.dev
        kw = dict(causal=c.causal, q_norm_w=dv["q_norm_w"], k_norm_w=dv["k_norm_w"], eps=c.eps,
                  theta=c.theta, workspace=self.ws, prof=prof, **self.masks, **self.rope)
        if c.dense:
            B, T = c.B, c.T_max
            return self.gqa.prefill(dv["q"].view(B, T, c.H, c.d), dv["k"].view(B, T, c.G, c.d),
                                    dv["v"].view(B, T, c.G, c.d), dv["positions"],
                                    out=self.out.view(B, T, c.H, c.d), **kw)
        return self.gqa.prefill(dv["q"], dv["k"], dv["v"], dv["positions"], cu_seqlens=dv["cu"],
                                max_seqlen=c.T_max, out=self.out, **kw)

    @property
    def work(self):
        if not self.masks:
            return self.case.flops
        c = self.case
        return 4.0 * c.d * c.H * visible_pairs(c.lengths, self.window, self.block_mask)

    @property
    def kernel(self):
        import workloads as W
        return "prefill_bf16_kernel" if self.case.dtype == W.BF16 else "prefill_f32_kernel"

    @property
    def peak(self):
        import workloads as W
        return FP32_PEAK_TFLOPS if self.case.dtype == W.F32 else MFMA_BF16_PEAK_TFLOPS

    @property
    def bound(self):
        # the fp32 kernel's products run on the vector ALUs, the bf16 kernel's on the matrix cores
        import workloads as W
        return "alu" if self.case.dtype == W.F32 else "mfma"


class PrefillCached:
    """gqa_prefill_cached on a chunk workload. Every call appends the same new rows at the
    same cache slots (cache_lens is not advanced), so repeated calls do identical work."""

    kernel = "prefill_bf16_kernel"
    peak = MFMA_BF16_PEAK_TFLOPS
    masks = {}

    def __init__(self, case):
        import attention_head_qk_amd as gqa
        from workloads import device_cached_inputs
        self.case = case
        self.dev = device_cached_inputs(case)
        self.gqa = gqa
        self.out = self.dev["q"].new_empty(self.dev["q"].shape)

    def __call__(self, prof=None):
        c, dv = self.case, self.dev
        return self.gqa.prefill_cached(dv["q"], dv["k"], dv["v"], dv["k_cache"], dv["v_cache"],
                                       dv["cache_lens"], dv["positions"], causal=c.causal,
                                       q_norm_w=dv["q_norm_w"], k_norm_w=dv["k_norm_w"],
                                       eps=c.eps, theta=c.theta, cu_seqlens=dv["cu"],
                                       max_seqlen=c.T_max, out=self.out, prof=prof)

    @property
    def work(self):
        return self.case.flops


class Decode:
    kernel = "decode_split_rows_kernel"

    def __init__(self, case):
        import torch
        import attention_head_qk_amd as gqa
        from workloads import device_decode_inputs
        self.case = case
        self.dev = device_decode_inputs(case)
        self.gqa = gqa
        c = case
        self.ws = torch.empty(gqa.workspace_bytes("decode", c.B, c.max_seq, c.H, c.G, c.d),
                              dtype=torch.uint8, device="cuda")
        self.out = torch.empty_like(self.dev["q"])

    def __call__(self, prof=None):
        c, dv = self.case, self.dev
        return self.gqa.decode(dv["q"], dv["k_cache"], dv["v_cache"], dv["seq_lens"],
                               k_new=dv["k_new"], v_new=dv["v_new"], q_norm_w=dv["q_norm_w"],
                               k_norm_w=dv["k_norm_w"], eps=c.eps, theta=c.theta,
                               workspace=self.ws, out=self.out, prof=prof)

    @property
    def work(self):
        return self.case.kv_bytes


# ----------------------------------------------------------------------------- timing
def _stats(xs):
    return {"median": round(statistics.median(xs), 5), "min": round(min(xs), 5),
            "mean": round(sum(xs) / len(xs), 5)}


def timed(fn, steps, warmup):
    """Warm up, then ``steps`` calls with events around each whole call, and ``steps`` more
    with events around the main kernel only (recorded by the library on the launch stream),
    so that neither measurement carries the other's event records. Returns per-call lists of
    milliseconds (call, kernel)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for e in ev:
        for x in e:
            x.record()
    torch.cuda.synchronize()
    for e in ev:
        e[0].record()
        fn()
        e[3].record()
    torch.cuda.synchronize()
    for e in ev:
        fn(prof=(e[1], e[2]))
    torch.cuda.synchronize()
    call = [e[0].elapsed_time(e[3]) for e in ev]
    kern = [e[1].elapsed_time(e[2]) for e in ev]
    return call, kern


class ClockSampler:
    """Shader and memory clock of the GPU, sampled from sysfs every 20 ms on a thread while
    the timed loops run (hwmon freq*_input in Hz, else the current pp_dpm level). Reports
    None for a clock the device does not expose."""

    def __init__(self):
        import glob
        self.files = {}
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            for hw in sorted(glob.glob(dev + "/hwmon/hwmon*")):
                for lab in glob.glob(hw + "/freq*_label"):
                    try:
                        name = open(lab).read().strip().lower()
                    except OSError:
                        continue
                    if name in ("sclk", "mclk") and name not in self.files:
                        self.files[name] = ("hz", lab.replace("_label", "_input"))
            for name in ("sclk", "mclk"):
                f = f"{dev}/pp_dpm_{name}"
                if name not in self.files and os.path.exists(f):
                    self.files[name] = ("dpm", f)
            if self.files:
                break
        self.samples = {k: [] for k in self.files}
        self._stop = threading.Event()
        self._t = None

    def _read(self, kind, path):
        try:
            text = open(path).read()
        except OSError:
            return None
        if kind == "hz":
            return int(text.strip()) / 1e6
        for line in text.splitlines():
            if line.strip().endswith("*"):
                v = line.split(":")[1].strip().rstrip("*").strip().lower().replace("mhz", "")
                return float(v)
        return None

    def _run(self):
        while not self._stop.is_set():
            for k, (kind, path) in self.files.items():
                v = self._read(kind, path)
                if v is not None:
                    self.samples[k].append(v)
            self._stop.wait(0.02)

    def __enter__(self):
        if self.files:
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._t:
            self._t.join()

    def report(self):
        out = {"source": "sysfs " + ", ".join(f"{k}:{v[0]}" for k, v in self.files.items())
               if self.files else None}
        for k in ("sclk", "mclk"):
            xs = self.samples.get(k) or []
            out[k + "_mhz"] = ({"median": round(statistics.median(xs), 1),
                                "min": round(min(xs), 1), "max": round(max(xs), 1),
                                "samples": len(xs)} if xs else None)
        return out


def measure(runner, steps, warmup, workload_name):
    """One configuration's sub-object: the whole call and its main kernel, median / min /
    mean over ``steps`` calls each, rates and the roofline fraction of the kernel."""
    call, kern = timed(runner, steps, warmup)
    cs, ks = _stats(call), _stats(kern)
    work = runner.work
    if isinstance(runner, Decode):
        rate = lambda ms: work / (ms * 1e-3) / 1e9  # noqa: E731
        unit, peak, bound = "GB/s", HBM_PEAK_GBS, "hbm"
    else:
        rate = lambda ms: work / (ms * 1e-3) / 1e12  # noqa: E731
        unit, peak, bound = "TFLOP/s", runner.peak, getattr(runner, "bound", "mfma")
    return {
        "workload": workload_name, "unit": unit, "work": work,
        "work_unit": "B" if unit == "GB/s" else "FLOP",
        "call_ms": cs, "kernel_ms": ks,
        "call_rate": round(rate(cs["median"]), 3),
        "kernel_rate": round(rate(ks["mean"]), 3),
        "kernel_rate_best": round(rate(ks["min"]), 3),
        "roofline": {"bound": bound, "achieved": round(rate(ks["mean"]), 3), "peak": peak,
                     "unit": unit, "frac": round(rate(ks["mean"]) / peak, 4),
                     "frac_median": round(rate(ks["median"]) / peak, 4),
                     "traffic": measured_traffic(runner.kernel, workload_name),
                     "kernel": runner.kernel},
    }


# ----------------------------------------------------------------------------- CPU baseline
# The oracle, as it stands, on a pool of worker processes. The pool is forked before the
# parent touches the GPU (before torch is imported), so the workers hold no GPU state; the
# host inputs they need are module globals set before the fork and shared copy-on-write.
_CASES = {}


def _worker_init():
    try:
        import threadpoolctl
        threadpoolctl.threadpool_limits(1)
    except Exception:
        pass


def _oracle_unit(spec):
    """Time one unit of oracle work. spec = ("prefill", key, b, head) for one (sequence,
    query head) of a prefill, ("rows", key, head, rows) for sampled query rows of one head,
    ("decode", key, b) for one decode sequence. Input preparation (decoding the stored
    bf16 bits, drawing a decode sequence's cache rows) is not timed."""
    import numpy as np
    import workloads as W
    from oracle import gqa_oracle as O
    kind, key = spec[0], spec[1]
    c = _CASES[key]
    if kind == "decode":
        b = spec[2]
        k, v = c.cache_rows(b)
        args = (c.f64("q")[b], W.to_f64(k, c.dtype), W.to_f64(v, c.dtype), int(c.seq_lens[b]),
                c.f64("q_norm_w"), c.f64("k_norm_w"), c.eps, c.theta)
        kw = dict(k_new=c.f64("k_new")[b], v_new=c.f64("v_new")[b])
        t0 = time.perf_counter()
        O.decode_one(*args, **kw)
        return time.perf_counter() - t0, os.getpid()
    h = c.H // c.G
    gq, gk = c.f64("q_norm_w"), c.f64("k_norm_w")
    if kind == "prefill":
        b, i = spec[2], spec[3]
        s, e = int(c.cu_seqlens[b]), int(c.cu_seqlens[b + 1])
        g = i // h
        q = W.to_f64(c.q[s:e, i:i + 1], c.dtype)
        k = W.to_f64(c.k[s:e, g:g + 1], c.dtype)
        v = W.to_f64(c.v[s:e, g:g + 1], c.dtype)
        t0 = time.perf_counter()
        O.prefill(q, k, v, c.positions[s:e], np.array([0, e - s]), gq, gk, c.eps, c.theta,
                  c.causal)
        return time.perf_counter() - t0, os.getpid()
    i, rows = spec[2], spec[3]
    g = i // h
    q = W.to_f64(c.q[:, i:i + 1], c.dtype)
    k = W.to_f64(c.k[:, g:g + 1], c.dtype)
    v = W.to_f64(c.v[:, g:g + 1], c.dtype)
    t0 = time.perf_counter()
    O.prefill_rows(q, k, v, c.positions, c.cu_seqlens, rows, gq, gk, c.eps, c.theta, c.causal)
    return time.perf_counter() - t0, os.getpid()


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _pool_size():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(MAX_POOL, n))


def start_oracle_pool(cases):
    """Fork the worker pool now (before any GPU use) with the host cases in place."""
    import multiprocessing as mp
    _CASES.update(cases)
    return mp.get_context("fork").Pool(_pool_size(), initializer=_worker_init)


def _run_units(pool, units):
    """Run units; the time on C cores is the busiest worker's total (its makespan)."""
    t0 = time.perf_counter()
    res = pool.map(_oracle_unit, units, chunksize=1)
    wall = time.perf_counter() - t0
    per_pid = {}
    for dt, pid in res:
        per_pid[pid] = per_pid.get(pid, 0.0) + dt
    return max(per_pid.values()), wall


def cpu_baseline_all(pool, keys, headline):
    """Oracle time per configuration on the pool, on a bounded sample of each, scaled to the
    whole configuration (the oracle materialises every score row, so its cost per prefill
    row is the same for every row of a sequence, and a decode sequence's cost grows with its
    length). Returns the cpu_baseline object for the headline configuration with the others
    under per_config."""
    import numpy as np
    per = {}
    for key in keys:
        c = _CASES[key]
        if key.startswith("decode"):
            # every 4th sequence by length rank; scaled by the cached rows they hold
            order = np.argsort(c.seq_lens)
            pick = [int(b) for b in order[::4]]
            busy, wall = _run_units(pool, [("decode", key, b) for b in pick])
            scale = float(c.seq_lens.sum()) / float(c.seq_lens[pick].sum())
            per[key] = {"work": c.kv_bytes, "unit": "GB/s",
                        "sample": f"{len(pick)} of {c.B} sequences (every 4th by length), "
                                  f"scaled by cached rows", "scale": round(scale, 3),
                        "busy_s": busy, "wall_s": wall}
        elif c.B == 1 and c.N >= 16384:
            # long prefill: 64 seeded query rows (row 0 and the last among them), all heads
            rng = np.random.default_rng(12)
            rows = np.unique(np.concatenate([[0, c.N - 1], rng.integers(0, c.N, 62)]))
            busy, wall = _run_units(pool, [("rows", key, i, rows) for i in range(c.H)])
            scale = c.N / len(rows)
            per[key] = {"work": c.flops, "unit": "TFLOP/s",
                        "sample": f"{len(rows)} of {c.N} query rows, every head, scaled by "
                                  f"rows (each row's full score row is materialised)",
                        "scale": round(scale, 3), "busy_s": busy, "wall_s": wall}
        else:
            # (sequence, head) units; the varlen workload takes one head of every group
            heads = range(c.H) if c.N <= 4096 else range(0, c.H, c.H // c.G)
            units = [("prefill", key, b, i) for b in range(c.B) for i in heads
                     if c.cu_seqlens[b + 1] > c.cu_seqlens[b]]
            scale = c.H / len(heads)
            per[key] = {"work": c.flops, "unit": "TFLOP/s",
                        "sample": "every (sequence, head)" if scale == 1 else
                                  f"{len(heads)} of {c.H} heads (one per group), every "
                                  f"sequence, scaled by heads",
                        "scale": round(scale, 3)}
            per[key]["busy_s"], per[key]["wall_s"] = _run_units(pool, units)
        e = per[key]
        e["full_s_extrapolated" if e["scale"] != 1 else "full_s"] = round(e["busy_s"] * e["scale"], 3)
        full = e["busy_s"] * e["scale"]
        e["value"] = round(e["work"] / full / (1e9 if e["unit"] == "GB/s" else 1e12), 6)
        e["busy_s"], e["wall_s"] = round(e["busy_s"], 3), round(e["wall_s"], 3)
        log(f"bench: oracle {key}: {e['value']} {e['unit']} ({e['sample']})")
    h = per[headline]
    return {"value": h["value"], "unit": h["unit"], "cores": _pool_size(), "kind": "oracle",
            "sample": f"{headline}: {h['sample']}; fp64 NumPy oracle on a pool of "
                      f"{_pool_size()} processes (one BLAS thread each), time = the busiest "
                      f"worker's total, x{h['scale']} to the full configuration (extrapolated)",
            "cpu_model": _cpu_model(), "per_config": per}


# ----------------------------------------------------------------------------- other workloads
def copy_calibration(steps, warmup):
    """A plain device-to-device copy of COPY_BYTES per step (torch's copy kernel). Profiled
    with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE, it gives the factor that turns those
    counters into HBM bytes."""
    import torch
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"metric": "device copy GB/s (calibration)", "value": round(2 * COPY_BYTES / ms / 1e6, 2),
            "unit": "GB/s", "bytes_read_per_step": COPY_BYTES, "bytes_written_per_step": COPY_BYTES,
            "ms_per_step": round(ms, 4), "steps": steps, "n_gpus": 1}


class DecodeLoop:
    """A generation loop on the decode-loop workload: every step advances seq_lens by one and
    decodes one token per sequence (the new K/V appended first). The step's inputs are the
    workload's first-step tokens, bound once; every 64 steps seq_lens goes back to the
    starting cache lengths (one 64-byte device copy, inside the timed region), so each block of
    64 steps repeats the workload's lengths. Three ways to run it: eager gqa_decode calls, a
    one-step graph replayed per token, and a graph of MULTI steps replayed per MULTI tokens
    (a graph launch costs about 5 us more than stream launches, once per replay)."""

    MULTI = 8

    def __init__(self, case):
        import attention_head_qk_amd as gqa
        import torch
        from workloads import device_steps_inputs
        self.case = c = case
        dev = device_steps_inputs(case)
        self.gqa, self.dev = gqa, dev
        self.sl0 = dev["seq_lens"]
        self.kc, self.vc = dev["k_cache"], dev["v_cache"]
        self.sl = self.sl0.clone()
        self.q, self.k, self.v = dev["q"][0].clone(), dev["k"][0].clone(), dev["v"][0].clone()
        self.ws = torch.empty(gqa.workspace_bytes("decode", c.B, c.max_seq, c.H, c.G, c.d),
                              dtype=torch.uint8, device="cuda")
        self.out = torch.empty_like(self.q)
        self.kw = dict(q_norm_w=dev["q_norm_w"], k_norm_w=dev["k_norm_w"], eps=c.eps,
                       theta=c.theta)
        self.graph = gqa.DecodeGraph(self.q, self.kc, self.vc, self.sl, self.k, self.v,
                                     out=self.out, workspace=self.ws, **self.kw)
        m = self.MULTI
        assert c.S % m == 0
        self.qm = self.q.unsqueeze(0).repeat(m, 1, 1, 1)
        self.km = self.k.unsqueeze(0).repeat(m, 1, 1, 1)
        self.vm = self.v.unsqueeze(0).repeat(m, 1, 1, 1)
        self.outm = torch.empty_like(self.qm)
        self.graph_m = gqa.DecodeGraph(self.qm, self.kc, self.vc, self.sl, self.km, self.vm,
                                       out=self.outm, workspace=self.ws, steps=m, **self.kw)

    def eager(self, i, prof=None):
        if i % self.case.S == 0:
            self.sl.copy_(self.sl0)
        self.sl.add_(1)
        self.gqa.decode(self.q, self.kc, self.vc, self.sl, k_new=self.k, v_new=self.v,
                        out=self.out, workspace=self.ws, prof=prof, **self.kw)

    def replay(self, i):
        if i % self.case.S == 0:
            self.sl.copy_(self.sl0)
        self.graph.launch()

    def replay_multi(self, i):
        """Steps i .. i + MULTI - 1 in one launch (called for every i, launches at multiples)."""
        if i % self.MULTI:
            return
        if i % self.case.S == 0:
            self.sl.copy_(self.sl0)
        self.graph_m.launch()

    def step_bytes(self, i):
        """Algorithmic bytes of step i: the K and V rows it sees, plus q in and out."""
        c = self.case
        rows = float(c.cache_lens.astype("float64").sum()) + c.B * (i % c.S + 1)
        return rows * c.G * c.d * 2 * 2 + 2.0 * c.B * c.H * c.d * 2


def bench_decode_loop(args, dev_name):
    import torch
    import workloads as W
    loop = DecodeLoop(W.decode_loop())
    c = loop.case
    log(f"bench: decode loop inputs ready ({c.name})")
    # whole launches of the multi-step graph: steps and warmup rounded up to multiples of MULTI
    m = loop.MULTI
    K = -(-args.steps // m) * m
    warm = -(-args.warmup // m) * m
    nbytes = sum(loop.step_bytes(i) for i in range(K))

    def run(fn):
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / K

    def gpu_only(fn):
        """Per-step GPU time: the steps are queued behind a spin kernel long enough for the
        host to enqueue all of them, so the events see the device run them back to back."""
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(max(20_000_000, K * 200_000))
        a.record()
        for i in range(K):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K

    graph_ms = run(loop.replay)
    multi_ms = run(loop.replay_multi)
    eager_ms = run(loop.eager)
    graph_gpu_ms = gpu_only(loop.replay)
    multi_gpu_ms = gpu_only(loop.replay_multi)
    eager_gpu_ms = gpu_only(loop.eager)
    # the split-KV kernel alone, from the library's events around it in eager steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for i, e in enumerate(ev):
        loop.eager(i, prof=e)
    torch.cuda.synchronize()
    kern_ms = sum(a.elapsed_time(b) for a, b in ev) / K
    gbs = lambda ms: nbytes / K / (ms * 1e-3) / 1e9  # noqa: E731
    log(f"bench: decode loop graph {graph_ms * 1e3:.2f} us/step, {loop.MULTI}-step graph "
        f"{multi_ms * 1e3:.2f}, eager {eager_ms * 1e3:.2f} us/step (GPU only: graph "
        f"{graph_gpu_ms * 1e3:.2f}, {loop.MULTI}-step graph {multi_gpu_ms * 1e3:.2f}, eager "
        f"{eager_gpu_ms * 1e3:.2f}), split kernel {kern_ms * 1e3:.2f} us")
    line = {"metric": f"decode loop GB/s (generation steps replayed {loop.MULTI} per HIP graph)",
            "value": round(gbs(multi_ms), 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
            "warmup": warm, "ms_per_step": round(multi_ms, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "device": dev_name,
            "graph_multi": {"steps_per_launch": loop.MULTI,
                            "us_per_step": round(multi_ms * 1e3, 3),
                            "GB/s": round(gbs(multi_ms), 2),
                            "tokens_per_s": round(c.B / (multi_ms * 1e-3), 1),
                            "gpu_us_per_step": round(multi_gpu_ms * 1e3, 3)},
            "graph": {"us_per_step": round(graph_ms * 1e3, 3), "GB/s": round(gbs(graph_ms), 2),
                      "tokens_per_s": round(c.B / (graph_ms * 1e-3), 1),
                      "gpu_us_per_step": round(graph_gpu_ms * 1e3, 3)},
            "eager": {"us_per_step": round(eager_ms * 1e3, 3), "GB/s": round(gbs(eager_ms), 2),
                      "tokens_per_s": round(c.B / (eager_ms * 1e-3), 1),
                      "gpu_us_per_step": round(eager_gpu_ms * 1e3, 3)},
            "roofline": {"bound": "hbm", "achieved": round(gbs(kern_ms), 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs(kern_ms) / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_split_rows_kernel", c.name),
                         "kernel": "decode_split_rows_kernel", "kernel_ms": round(kern_ms, 5)},
            "config": {"workload": c.name, "B": c.B, "steps_per_block": c.S,
                       "cache_lens": c.cache_lens.tolist(), "max_seq": c.max_seq, "H": c.H,
                       "G": c.G, "d": c.d, "seed": c.seed},
            "cpu_baseline": None}
    loop.graph.close()
    loop.graph_m.close()
    print(json.dumps(line), flush=True)
    return 0


# ----------------------------------------------------------------------------- main
METRIC = "GQA prefill TFLOP/s (% bf16 MFMA peak); decode KV GB/s (% HBM peak)"


def _config_desc(runner):
    c = runner.case
    if isinstance(runner, Decode):
        return {"B": c.B, "sum_L": int(c.seq_lens.sum()), "max_seq": c.max_seq, "H": c.H,
                "G": c.G, "d": c.d, "seed": c.seed}
    d = {"B": c.B, "lengths_sum": c.N, "T_max": c.T_max, "H": c.H, "G": c.G, "d": c.d,
         "causal": c.causal, "seed": c.seed}
    if c.B > 1 and len(set(c.lengths.tolist())) > 1:
        d["lengths"] = c.lengths.tolist()
    return d


def _wname(runner, rope_scaling="none"):
    name = runner.case.name
    if getattr(runner, "window", 0):
        name += f"_window{runner.window}"
    if getattr(runner, "block_mask", None) is not None:
        name += "_blocks64"
    if getattr(runner, "rope", None):
        name += "_rope_" + rope_scaling
    return name


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=WORKLOADS, default="default")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rope-scaling", choices=("none", "linear", "yarn", "ntk"), default="none",
                    help="prefill workloads: RoPE through a scaled frequency table (linear x4; "
                         "yarn from 32768 to 131072 training/inference tokens; ntk x8)")
    args = ap.parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        return 2
    log(f"bench: workload={args.workload} steps={args.steps} warmup={args.warmup}")

    import workloads as W
    # host inputs first; the oracle's worker pool is forked before the GPU is touched
    host = {}
    if args.workload == "default":
        host = {"long_g4": W.prefill_long(4), "long_g1": W.prefill_long(1),
                "varlen": W.prefill_varlen(), "prefill_4k": W.prefill_4k(),
                "tiny_f32": W.tiny_f32(), "decode": W.decode_64()}
    elif args.workload in ("tiny_f32", "prefill_4k", "varlen", "long_g4", "long_g1"):
        host = {args.workload: prefill_case(args.workload)}
    elif args.workload == "decode":
        host = {"decode": W.decode_64()}
    pool = None
    if host and not args.no_cpu_baseline and args.rope_scaling == "none":
        pool = start_oracle_pool(host)
        log(f"bench: oracle pool of {_pool_size()} processes started")

    import torch
    if args.workload == "copy_calibration":
        print(json.dumps(copy_calibration(args.steps, args.warmup)), flush=True)
        return 0
    torch.cuda.init()
    dev_name = torch.cuda.get_device_name(0)
    if args.workload == "decode_loop":
        return bench_decode_loop(args, dev_name)

    runners = {}
    if args.workload == "chunked":
        runners["chunked"] = PrefillCached(W.prefill_chunked())
    elif args.workload == "long_window":
        runners["long_window"] = Prefill(prefill_case("long_window"), window=WINDOW)
    elif args.workload == "long_blocks":
        case = prefill_case("long_blocks")
        runners["long_blocks"] = Prefill(case, block_mask=W.make_block_mask(
            9, -(-case.T_max // 64), BLOCK_DENSITY))
    else:
        for key, case in host.items():
            if key == "decode":
                runners[key] = Decode(case)
            elif args.rope_scaling != "none":
                import attention_head_qk_amd as gqa
                table = gqa.rope_freq_table(case.d, case.theta, args.rope_scaling,
                                            alpha=ROPE_ALPHA[args.rope_scaling],
                                            train_len=32768, infer_len=131072)
                runners[key] = Prefill(case, rope_inv_freq=table)
            else:
                runners[key] = Prefill(case)
    torch.cuda.synchronize()
    log("bench: device inputs ready: " + ", ".join(r.case.name for r in runners.values()))

    # the step: one pass of the whole path (prefill of the headline configuration, then the
    # decode) when both are present, else the one configuration
    head_key = "long_g4" if "long_g4" in runners else next(iter(runners))
    step_fns = [runners[head_key]] + ([runners["decode"]] if "decode" in runners
                                      and head_key != "decode" else [])

    def step():
        for f in step_fns:
            f()

    sampler = ClockSampler()
    with sampler:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        log(f"bench: {args.steps} steps, {step_ms:.3f} ms/step")
        configs = {}
        for key, r in runners.items():
            configs[key] = measure(r, args.steps, 1, _wname(r, args.rope_scaling))
            cfg = configs[key]
            cfg.update(_config_desc(r))
            log(f"bench: {key}: call {cfg['call_ms']['median']:.4f} ms, kernel "
                f"{cfg['kernel_ms']['median']:.4f} ms (median), {cfg['kernel_rate']} "
                f"{cfg['unit']} = {cfg['roofline']['frac']:.3f} of peak")

    head = configs[head_key]
    hr = runners[head_key]
    dtype = "f32" if head_key == "tiny_f32" else "bf16"
    line = {"metric": METRIC, "value": head["call_rate"], "unit": head["unit"], "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic", "device": dev_name}
    roof = dict(head["roofline"])
    roof["kernel_ms"] = head["kernel_ms"]["mean"]
    roof["work_per_launch"] = head["work"]
    line["roofline"] = roof
    line["config"] = {"workload": head["workload"], "step": " + ".join(
        configs[k]["workload"] for k in ([head_key] + (["decode"] if len(step_fns) > 1 else []))),
        **_config_desc(hr)}
    if getattr(hr, "window", 0):
        line["config"]["window"] = hr.window
    if getattr(hr, "block_mask", None) is not None:
        line["config"]["block_mask"] = {"block": 64, "kept": int(hr.block_mask.sum()),
                                        "density": BLOCK_DENSITY, "local": 1, "seed": 9}
    if args.rope_scaling != "none":
        line["config"]["rope_scaling"] = args.rope_scaling
    if isinstance(hr, PrefillCached):
        line["config"].update(cache_lens=hr.case.cache_lens.tolist(), max_seq=hr.case.max_seq)
    line["configs"] = configs
    line["clocks"] = sampler.report()
    if pool is not None:
        log("bench: timing the CPU oracle")
        try:
            line["cpu_baseline"] = cpu_baseline_all(pool, list(host), head_key)
        finally:
            pool.terminate()
    elif not args.no_cpu_baseline:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
