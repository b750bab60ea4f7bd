#!/usr/bin/env python3
"""Benchmark of the causal GQA hot path (QK-RMSNorm + RoPE prologue, prefill attention,
decode split-KV + combine) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload default|...]

A step of the default workload is one pass of the whole path over one batch of synthetic
input: gqa_prefill on the bf16 prefill T=4096, H=16, G=8, d=128 (causal, gamma ~ U(0.5,1.5),
theta 1e6), then gqa_decode on 64 sequences x 1 new token with cache lengths U{1024..32768},
H=32, G=8, d=128 (the new token's K/V appended first). Inputs are resident in HBM before the
timed region. Prints one JSON line:

* value: prefill TFLOP/s of the whole gqa_prefill call (prologue + attention), algorithmic
  FLOPs 4*d*H*sum T_b(T_b+1)/2; ``decode`` carries the decode GB/s of the whole gqa_decode
  call, algorithmic bytes = visible K and V rows + q + out.
* roofline: the prefill attention kernel alone (HIP events recorded by the library right
  around its launch, on the launch stream), against the 2.5 PFLOP/s bf16 dense MFMA peak;
  roofline_decode: the decode split-KV kernel alone against 8 TB/s HBM.
* --workload chunked: gqa_prefill_cached on 4 sequences, each a 2048-token chunk after a
  cached prefix of U{2048..14336} tokens (H=32, G=8, d=128); FLOPs count every visible
  (new query, key) pair, cached keys included.
* --workload long_window / long_blocks: the T=32768, H=64, G=4 prefill with a 512-key
  sliding window, or with a 64-key block layout (each query block keeps its previous block
  and 10% of the earlier ones, seed 9); FLOPs count only the visible (query, key) pairs.
* --workload decode_loop: a generation loop, 16 sequences from cache lengths U{256..2048};
  each step advances seq_lens on the device and decodes one token per sequence. value = GB/s
  of the step replayed as one HIP graph (gqa_decode_graph_*); the eager step (a torch add and
  gqa_decode) is reported beside it.
* cpu_baseline: the fp64 CPU oracle timed on the host CPU of the same machine, on a bounded
  sample of the same prefill workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0

WORKLOADS = ("default", "tiny_f32", "prefill_4k", "varlen", "decode", "long_g4", "long_g1",
             "long_window", "long_blocks", "chunked", "decode_loop", "copy_calibration")
WINDOW = 512          # sliding-window workload: keys per query
BLOCK_DENSITY = 0.1   # block-sparse workload: share of earlier 64-key blocks kept
ROPE_ALPHA = {"linear": 4.0, "ntk": 8.0, "yarn": 1.0}  # --rope-scaling extension factors
COPY_BYTES = 1 << 30  # bytes read (and written) per step of the copy calibration


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
    return {"tiny_f32": W.tiny_f32, "prefill_4k": W.prefill_4k, "default": W.prefill_4k,
            "varlen": W.prefill_varlen, "long_g4": lambda: W.prefill_long(4),
            "long_g1": lambda: W.prefill_long(1), "long_window": lambda: W.prefill_long(4),
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


class PrefillCached:
    """gqa_prefill_cached on a chunk workload. Every call appends the same new rows at the
    same cache slots (cache_lens is not advanced), so repeated calls do identical work."""

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


def cpu_baseline(case, budget_s=12.0):
    """Time the fp64 oracle (as it stands) on whole query heads of the prefill workload,
    head after head, until about ``budget_s`` seconds of CPU work; report TFLOP/s over the
    algorithmic FLOPs of the heads done."""
    import numpy as np
    from oracle import gqa_oracle as O
    try:
        import threadpoolctl
        cores = max(i["num_threads"] for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        cores = os.cpu_count() or 1
    q, k, v = case.f64("q"), case.f64("k"), case.f64("v")
    gq, gk = case.f64("q_norm_w"), case.f64("k_norm_w")
    t0 = time.perf_counter()
    qt, kt = O.qk_norm_rope(q, k, case.positions, gq, gk, case.eps, case.theta)
    h = case.H // case.G
    heads = 0
    L = case.lengths.astype(np.float64)
    per_head = 4.0 * case.d * float(np.sum(L * (L + 1) / 2 if case.causal else L * L))
    while heads < case.H and (time.perf_counter() - t0) < budget_s:
        i = heads
        for b in range(case.B):
            s, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
            P = O.attention_weights(qt[s:e, i], kt[s:e, i // h], case.causal)
            _ = P @ v[s:e, i // h]
        heads += 1
    dt = time.perf_counter() - t0
    return {"value": round(per_head * heads / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"fp64 NumPy oracle on {heads} of {case.H} query heads of {case.name} "
                      f"(prologue on all tokens + full score matrix per head), {dt:.1f} s"}


def timed(fn, steps, warmup):
    """Warm up, then time ``steps`` calls with events around each whole call, and ``steps``
    more with events around the main kernel only (recorded by the library on the launch
    stream), so that neither measurement carries the other's event records."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for e in ev:
        for x in e:
            x.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        fn()
        e[3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for e in ev:
        fn(prof=(e[1], e[2]))
    torch.cuda.synchronize()
    call_ms = sum(e[0].elapsed_time(e[3]) for e in ev) / steps
    kern_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    return wall, call_ms, kern_ms


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
    64 steps repeats the workload's lengths."""

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
    K = args.steps
    nbytes = sum(loop.step_bytes(i) for i in range(K))

    def run(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / K

    graph_ms = run(loop.replay)
    eager_ms = run(loop.eager)
    # the split-KV kernel alone, from the library's events around it in eager steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for i, e in enumerate(ev):
        loop.eager(i, prof=e)
    torch.cuda.synchronize()
    kern_ms = sum(a.elapsed_time(b) for a, b in ev) / K
    gbs = lambda ms: nbytes / K / (ms * 1e-3) / 1e9  # noqa: E731
    log(f"bench: decode loop graph {graph_ms * 1e3:.2f} us/step, eager {eager_ms * 1e3:.2f} "
        f"us/step, split kernel {kern_ms * 1e3:.2f} us")
    line = {"metric": "decode loop GB/s (graph-replayed generation step)",
            "value": round(gbs(graph_ms), 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
            "warmup": args.warmup, "ms_per_step": round(graph_ms, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "device": dev_name,
            "graph": {"us_per_step": round(graph_ms * 1e3, 3), "GB/s": round(gbs(graph_ms), 2),
                      "tokens_per_s": round(c.B / (graph_ms * 1e-3), 1)},
            "eager": {"us_per_step": round(eager_ms * 1e3, 3), "GB/s": round(gbs(eager_ms), 2),
                      "tokens_per_s": round(c.B / (eager_ms * 1e-3), 1)},
            "roofline": {"bound": "hbm", "achieved": round(gbs(kern_ms), 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs(kern_ms) / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_split_mfma_kernel", c.name),
                         "kernel": "decode_split_mfma_kernel", "kernel_ms": round(kern_ms, 5)},
            "config": {"workload": c.name, "B": c.B, "steps_per_block": c.S,
                       "cache_lens": c.cache_lens.tolist(), "max_seq": c.max_seq, "H": c.H,
                       "G": c.G, "d": c.d, "seed": c.seed},
            "cpu_baseline": None}
    loop.graph.close()
    print(json.dumps(line), flush=True)
    return 0


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

    import torch
    import workloads as W
    log(f"bench: workload={args.workload} steps={args.steps} warmup={args.warmup}")
    if args.workload == "copy_calibration":
        print(json.dumps(copy_calibration(args.steps, args.warmup)), flush=True)
        return 0
    torch.cuda.init()
    dev_name = torch.cuda.get_device_name(0)
    if args.workload == "decode_loop":
        return bench_decode_loop(args, dev_name)

    pre = dec = None
    if args.workload == "chunked":
        pre = PrefillCached(W.prefill_chunked())
        log(f"bench: cached prefill inputs ready ({pre.case.name}, N={pre.case.N})")
    elif args.rope_scaling != "none" and args.workload != "decode":
        import attention_head_qk_amd as gqa
        case = prefill_case(args.workload)
        table = gqa.rope_freq_table(case.d, case.theta, args.rope_scaling, alpha=ROPE_ALPHA[args.rope_scaling],
                                    train_len=32768, infer_len=131072)
        pre = Prefill(case, rope_inv_freq=table)
    elif args.workload == "long_window":
        pre = Prefill(prefill_case(args.workload), window=WINDOW)
    elif args.workload == "long_blocks":
        case = prefill_case(args.workload)
        pre = Prefill(case, block_mask=W.make_block_mask(9, -(-case.T_max // 64), BLOCK_DENSITY))
    elif args.workload != "decode":
        pre = Prefill(prefill_case(args.workload))
        log(f"bench: prefill inputs ready ({pre.case.name}, N={pre.case.N})")
    if args.workload in ("default", "decode"):
        dec = Decode(W.decode_64())
        log(f"bench: decode inputs ready ({dec.case.name}, sum L={int(dec.case.seq_lens.sum())})")
    torch.cuda.synchronize()

    def step(prof=None):
        if pre is not None:
            pre(prof)
        if dec is not None:
            dec()

    # whole-step wall clock (both calls), events per call and per main kernel
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"bench: {args.steps} steps, {step_ms:.3f} ms/step")

    res = {}
    if pre is not None:
        _, call_ms, kern_ms = timed(pre, args.steps, 1)
        res["prefill"] = (call_ms, kern_ms)
        log(f"bench: prefill call {call_ms:.4f} ms, attention kernel {kern_ms:.4f} ms")
    if dec is not None:
        _, call_ms, kern_ms = timed(dec, args.steps, 1)
        res["decode"] = (call_ms, kern_ms)
        log(f"bench: decode call {call_ms:.4f} ms, split kernel {kern_ms:.4f} ms")

    line = {"metric": "GQA prefill TFLOP/s (% bf16 MFMA peak); decode KV GB/s (% HBM peak)",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "data": "synthetic", "device": dev_name}
    cfg = {}
    if pre is not None:
        c = pre.case
        call_ms, kern_ms = res["prefill"]
        tf_call = pre.work / (call_ms * 1e-3) / 1e12
        tf_kern = pre.work / (kern_ms * 1e-3) / 1e12
        peak = FP32_PEAK_TFLOPS if c.dtype == W.F32 else MFMA_BF16_PEAK_TFLOPS
        kname = "prefill_bf16_kernel" if c.dtype == W.BF16 else "prefill_f32_kernel"
        wname = c.name
        if getattr(pre, "window", 0):
            wname += f"_window{pre.window}"
        if getattr(pre, "block_mask", None) is not None:
            wname += "_blocks64"
        if getattr(pre, "rope", None):
            wname += "_rope_" + args.rope_scaling
        line.update({"value": round(tf_call, 3), "unit": "TFLOP/s",
                     "dtype": "f32" if c.dtype == W.F32 else "bf16"})
        line["roofline"] = {"bound": "mfma", "achieved": round(tf_kern, 3), "peak": peak,
                            "unit": "TFLOP/s", "frac": round(tf_kern / peak, 4),
                            "traffic": measured_traffic(kname, wname),
                            "kernel": kname,
                            "kernel_ms": round(kern_ms, 5), "flops_per_launch": pre.work}
        line["prefill"] = {"ms": round(call_ms, 5), "tflops": round(tf_call, 3),
                           "frac_of_peak": round(tf_call / peak, 4)}
        cfg["prefill"] = {"name": wname, "B": c.B, "lengths_sum": c.N, "T_max": c.T_max, "H": c.H,
                          "G": c.G, "d": c.d, "causal": c.causal, "seed": c.seed}
        if isinstance(pre, PrefillCached):
            cfg["prefill"].update(cache_lens=c.cache_lens.tolist(), max_seq=c.max_seq)
        if getattr(pre, "window", 0):
            cfg["prefill"]["window"] = pre.window
        if getattr(pre, "rope", None):
            cfg["prefill"]["rope_scaling"] = args.rope_scaling
        if getattr(pre, "block_mask", None) is not None:
            cfg["prefill"]["block_mask"] = {"block": 64, "kept": int(pre.block_mask.sum()),
                                            "density": BLOCK_DENSITY, "local": 1, "seed": 9}
    if dec is not None:
        c = dec.case
        call_ms, kern_ms = res["decode"]
        gbs_call = dec.work / (call_ms * 1e-3) / 1e9
        gbs_kern = dec.work / (kern_ms * 1e-3) / 1e9
        line["decode"] = {"value": round(gbs_call, 2), "unit": "GB/s", "ms": round(call_ms, 5),
                          "frac_of_peak": round(gbs_call / HBM_PEAK_GBS, 4),
                          "bytes": dec.work}
        line["roofline_decode"] = {"bound": "hbm", "achieved": round(gbs_kern, 2),
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(gbs_kern / HBM_PEAK_GBS, 4),
                                   "traffic": measured_traffic("decode_split_mfma_kernel", c.name),
                                   "kernel": "decode_split_mfma_kernel", "kernel_ms": round(kern_ms, 5)}
        cfg["decode"] = {"name": c.name, "B": c.B, "sum_L": int(c.seq_lens.sum()), "max_seq": c.max_seq,
                         "H": c.H, "G": c.G, "d": c.d, "seed": c.seed}
        if pre is None:
            line.update({"value": round(gbs_call, 2), "unit": "GB/s", "dtype": "bf16",
                         "roofline": line.pop("roofline_decode")})
    names = [v["name"] for v in cfg.values()]
    line["config"] = {"workload": " + ".join(names), **cfg}
    if (not args.no_cpu_baseline and pre is not None and not isinstance(pre, PrefillCached)
            and not pre.masks):
        log("bench: timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(pre.case)
    elif not args.no_cpu_baseline:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
