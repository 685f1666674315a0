#!/usr/bin/env python3
"""Benchmark of the attention forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one full forward of the workload (attention launch + split
combine when the plan splits), inputs resident in HBM.  Prints ONE JSON line
with the headline metric (split-KV long-context decode by default: achieved
HBM GB/s on the algorithmic bytes Q + K + V + O), a roofline object for the
dominant kernel (its duration measured with HIP events on the launch stream)
and the CPU oracle timed on the host as a reported baseline.  Secondary
workloads (GQA decode, fp8 short prefix, varlen prefill) are timed by HIP
graph replay as the fp8 split-K page times its shapes (5 eager and 5 graph
warmups, then the median of 7 rounds of 100 forwards; the graph holds 20
forwards back to back so the host's replay cost stays off the GPU's clock,
the one-forward-graph figure is reported beside it) under "others";
the fp8 short prefix, whose K/V fit the Infinity Cache, is timed cold
(replays cycle through K/V copies spanning 1 GiB) with the warm same-buffer
figure beside it.

Algorithmic work (the accounting of the split-KV decode table on
"[Cute,Fwd,Sm100] Support q_stage=1 for inference", section Benchmarks, pinned
by tests/golden/decode_split_sweep_sm100.csv):
  bytes = Q + K + V + O at their storage dtypes, K/V once per kv head, LSE
          not counted;
  flops = 2 * (Dqk + Dv) * Hq * (attended (query, key) pairs).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "split-KV decode µs + HBM GB/s (% peak); varlen prefill TFLOPS (% MFMA peak)"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "fp8_e4m3": 5000.0, "f32": 157.3}
ELEM = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Sources a kernel's code depends on (the host plan, shared helpers and its own
# header): a traffic measurement is used only while their hash is unchanged.
_SHARED_SOURCES = ["fmha_fwd_kernel.h", "fmha_params.h", "fmha_host.cpp"]
KERNEL_SOURCES = {
    "fmha_decode_kernel": _SHARED_SOURCES + ["fmha_decode_kernel.h"],
    "fmha_prefill_kernel": _SHARED_SOURCES + ["fmha_decode_kernel.h", "fmha_prefill_kernel.h"],
    "fmha_prefill8_kernel": _SHARED_SOURCES + ["fmha_decode_kernel.h", "fmha_prefill_kernel.h",
                                              "fmha_prefill8_kernel.h"],
    "fmha_fwd_kernel": _SHARED_SOURCES,
}


# ---- workloads (shapes only; tensors come from fmha_synth) -----------------

def _spec(name, dtype, lens_q, lens_k, hq, hkv, dqk, dv, *, causal=False, window=(-1, -1),
          varlen_q=False, varlen_k=False, seed=0, desc=""):
    return dict(name=name, dtype=dtype, lens_q=list(lens_q), lens_k=list(lens_k), hq=hq,
                hkv=hkv, dqk=dqk, dv=dv, causal=causal, window=tuple(window),
                varlen_q=varlen_q, varlen_k=varlen_k, seed=seed, desc=desc)


def workloads():
    import fmha_synth as fs
    gd = fs.gqa_decode_lengths()
    return {
        "long_decode": _spec("long_decode", "bf16", [1], [131072], 32, 32, 128, 128, seed=1,
                             desc="long-context decode B=1 Q=1 K=131072 Hq=Hkv=32 D=128 bf16"),
        "gqa_decode": _spec("gqa_decode", "bf16", [1] * 16, gd, 32, 8, 128, 128, varlen_k=True,
                            seed=2, desc="GQA batched decode B=16 Q=1 Hq=32 Hkv=8 D=128 bf16 "
                                         "KV~U[1024,32768]"),
        "fp8_prefix_16384": _spec("fp8_prefix_16384", "fp8_e4m3", [70], [16384], 12, 12, 192,
                                  128, seed=3, desc="fp8 short prefix B=1 Q=70 H=12 Dqk=192 "
                                                    "Dv=128 KV=16384"),
        "fp8_prefix_11008": _spec("fp8_prefix_11008", "fp8_e4m3", [70], [11008], 12, 12, 192,
                                  128, seed=3, desc="fp8 short prefix B=1 Q=70 H=12 Dqk=192 "
                                                    "Dv=128 KV=11008"),
        "varlen_skewed": _spec("varlen_skewed", "f16", fs.VARLEN_SKEWED, fs.VARLEN_SKEWED, 16,
                               16, 128, 128, varlen_q=True, varlen_k=True, seed=4,
                               desc="varlen prefill fp16 H=16 D=128 skewed 16384 tokens"),
        "varlen_skewed_causal": _spec("varlen_skewed_causal", "f16", fs.VARLEN_SKEWED,
                                      fs.VARLEN_SKEWED, 16, 16, 128, 128, causal=True,
                                      varlen_q=True, varlen_k=True, seed=4,
                                      desc="varlen prefill fp16 H=16 D=128 skewed causal"),
        "varlen_equal": _spec("varlen_equal", "f16", fs.VARLEN_EQUAL, fs.VARLEN_EQUAL, 16, 16,
                              128, 128, varlen_q=True, varlen_k=True, seed=4,
                              desc="varlen prefill fp16 H=16 D=128 8x2048"),
        "varlen_equal_causal": _spec("varlen_equal_causal", "f16", fs.VARLEN_EQUAL,
                                     fs.VARLEN_EQUAL, 16, 16, 128, 128, causal=True,
                                     varlen_q=True, varlen_k=True, seed=4,
                                     desc="varlen prefill fp16 H=16 D=128 8x2048 causal"),
        # 128 sequences (more than the in-kernel longest-first search serves):
        # the device-sorted tile table
        "varlen_many_causal": _spec("varlen_many_causal", "f16", fs.many_lengths(),
                                    fs.many_lengths(), 16, 16, 128, 128, causal=True,
                                    varlen_q=True, varlen_k=True, seed=6,
                                    desc="varlen prefill fp16 H=16 D=128 128 sequences "
                                         "U[64,2048] causal"),
        # head dim 256 (the same flops per token with half the heads)
        "varlen_equal_d256": _spec("varlen_equal_d256", "f16", fs.VARLEN_EQUAL, fs.VARLEN_EQUAL,
                                   8, 8, 256, 256, varlen_q=True, varlen_k=True, seed=4,
                                   desc="varlen prefill fp16 H=8 D=256 8x2048"),
        "varlen_equal_causal_d256": _spec("varlen_equal_causal_d256", "f16", fs.VARLEN_EQUAL,
                                          fs.VARLEN_EQUAL, 8, 8, 256, 256, causal=True,
                                          varlen_q=True, varlen_k=True, seed=4,
                                          desc="varlen prefill fp16 H=8 D=256 8x2048 causal"),
    }


def attended_pairs(sq, sk, causal, window):
    """Number of (query, key) pairs the mask allows (bottom-right aligned)."""
    return sum(_row_pairs(i, sq, sk, causal, window) for i in range(sq))


def alg_bytes(w):
    e = ELEM[w["dtype"]]
    eo = 2 if w["dtype"] == "fp8_e4m3" else e
    tq, tk = sum(w["lens_q"]), sum(w["lens_k"])
    return (tq * w["hq"] * w["dqk"] * e + tk * w["hkv"] * (w["dqk"] + w["dv"]) * e
            + tq * w["hq"] * w["dv"] * eo)


def alg_flops(w):
    pairs = sum(attended_pairs(sq, sk, w["causal"], w["window"])
                for sq, sk in zip(w["lens_q"], w["lens_k"]))
    return 2 * (w["dqk"] + w["dv"]) * w["hq"] * pairs


def kernel_name(kernel_id):
    """Kernel family of a plan's kernel_id (dtype * 1000 + instance id)."""
    i = kernel_id % 1000
    if i >= 210:
        return "fmha_prefill8_kernel"
    if i >= 200:
        return "fmha_prefill_kernel"
    if i >= 100:
        return "fmha_decode_kernel"
    return "fmha_fwd_kernel"


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "split_kv_flash_fmha_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ---- GPU side -------------------------------------------------------------

class Runner:
    """Prebuilt C-ABI arguments for one workload, so a step is two C calls."""

    def __init__(self, w, splits, device="cuda", combine_in_kernel=False):
        import ctypes

        import torch

        import fmha_synth as fs
        import split_kv_flash_fmha_amd as fmha
        self.ctypes, self.torch, self.fmha = ctypes, torch, fmha
        self.w = w
        prob = fs.make_problem(w["name"], dtype=w["dtype"], lens_q=w["lens_q"],
                               lens_k=w["lens_k"], hq=w["hq"], hkv=w["hkv"], dqk=w["dqk"],
                               dv=w["dv"], seed=w["seed"], varlen_q=w["varlen_q"],
                               varlen_k=w["varlen_k"], causal=w["causal"],
                               window=w["window"], device=device)
        self.prob = prob
        B = prob.batch
        if prob.varlen_q:
            q = prob.q
            cu_q = torch.from_numpy(prob.cu_q).to(device)
            out = torch.empty((q.shape[0], prob.hq, prob.dv), device=device,
                              dtype=torch.bfloat16 if w["dtype"] == "fp8_e4m3" else q.dtype)
            lse = torch.empty((prob.hq, q.shape[0]), device=device, dtype=torch.float32)
        else:
            q = prob.q.view(B, -1, prob.hq, prob.dqk)
            cu_q = None
            out = torch.empty((B, q.shape[1], prob.hq, prob.dv), device=device,
                              dtype=torch.bfloat16 if w["dtype"] == "fp8_e4m3" else q.dtype)
            lse = torch.empty((B, prob.hq, q.shape[1]), device=device, dtype=torch.float32)
        if prob.varlen_k:
            k, v = prob.k, prob.v
            cu_k = torch.from_numpy(prob.cu_k).to(device)
        else:
            k = prob.k.view(B, -1, prob.hkv, prob.dqk)
            v = prob.v.view(B, -1, prob.hkv, prob.dv)
            cu_k = None
        desc = {}
        if w["dtype"] == "fp8_e4m3":
            for n, val in (("q_descale", prob.q_descale), ("k_descale", prob.k_descale),
                           ("v_descale", prob.v_descale)):
                desc[n] = torch.tensor([val], dtype=torch.float32, device=device)
        self.tensors = dict(q=q, k=k, v=v, out=out, lse=lse, cu_q=cu_q, cu_k=cu_k, **desc)
        self.args = fmha.make_args(q, k, v, out=out, lse=lse, cu_seqlens_q=cu_q,
                                   cu_seqlens_k=cu_k, max_seqlen_q=prob.max_seqlen_q,
                                   max_seqlen_k=prob.max_seqlen_k, causal=w["causal"],
                                   window=w["window"], num_kv_splits=splits,
                                   num_cus=fmha.device_num_cus(),
                                   combine_in_kernel=combine_in_kernel, **desc)
        nbytes = fmha.workspace_size(self.args)
        self.ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        self.args.workspace = self.ws.data_ptr()
        self.args.workspace_bytes = self.ws.numel()
        self.plan = fmha.plan(self.args)
        # split partials combined by a second launch (timed separately from
        # the attention launch), or inside the attention launch
        self.split = self.plan.num_splits > 1 and not self.plan.combine_in_kernel
        if self.split:
            c = fmha.CombineArgs()
            c.o_part = self.ws.data_ptr() + self.plan.o_part_offset
            c.lse_part = self.ws.data_ptr() + self.plan.lse_part_offset
            c.out, c.lse = out.data_ptr(), lse.data_ptr()
            c.cu_seqlens_q = self.args.cu_seqlens_q
            c.cu_seqlens_k = self.args.cu_seqlens_k
            c.batch, c.seqlen_q, c.seqlen_k = self.args.batch, self.args.seqlen_q, self.args.seqlen_k
            c.max_seqlen_q = prob.max_seqlen_q
            c.total_q = sum(prob.lens_q)
            c.num_heads_q, c.head_dim_v = prob.hq, prob.dv
            c.num_splits, c.split_chunk = self.plan.num_splits, self.plan.split_chunk
            c.o_stride_batch, c.o_stride_tok, c.o_stride_head = (
                self.args.o_stride_batch, self.args.o_stride_tok, self.args.o_stride_head)
            c.lse_stride_batch, c.lse_stride_head = self.args.lse_stride_batch, self.args.lse_stride_head
            c.out_dtype = self.args.out_dtype
            self.cargs = c

    def stream(self):
        return self.torch.cuda.current_stream().cuda_stream

    def main_kernel(self, s):
        L, byref = self.fmha.lib, self.ctypes.byref
        fn = L.fmha_fwd_splitkv_partials if self.split else L.fmha_fwd
        st = fn(byref(self.args), s)
        if st:
            raise RuntimeError(f"forward failed with status {st}")

    def combine(self, s):
        if self.split:
            st = self.fmha.lib.fmha_splitkv_combine(self.ctypes.byref(self.cargs), s)
            if st:
                raise RuntimeError(f"combine failed with status {st}")

    def step(self, s, args=None):
        if args is None:
            self.main_kernel(s)
        else:
            fn = self.fmha.lib.fmha_fwd_splitkv_partials if self.split else self.fmha.lib.fmha_fwd
            st = fn(self.ctypes.byref(args), s)
            if st:
                raise RuntimeError(f"forward failed with status {st}")
        self.combine(s)

    def rotated_args(self, min_bytes):
        """Argument sets over copies of K and V that together span at least
        `min_bytes`, so that graph replays cycling through them find no K/V
        byte in the caches from the previous use (cold-cache timing)."""
        k, v = self.tensors["k"], self.tensors["v"]
        foot = k.numel() * k.element_size() + v.numel() * v.element_size()
        n = max(1, -(-min_bytes // foot))
        self.rot = [(k.clone(), v.clone()) for _ in range(n)]
        out = []
        for kc, vc in self.rot:
            a = type(self.args).from_buffer_copy(self.args)
            a.k, a.v = kc.data_ptr(), vc.data_ptr()
            out.append(a)
        return out


def time_eager(r, steps, warmup):
    """K eager steps; HIP events around every attention launch."""
    torch = r.torch
    s = r.stream()
    for _ in range(warmup):
        r.step(s)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(steps):
        ev[i][0].record()
        r.main_kernel(s)
        ev[i][1].record()
        r.combine(s)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    kern_ms = [a.elapsed_time(b) for a, b in ev]
    return total_ms / steps, sum(kern_ms) / len(kern_ms), wall


def time_graph(r, arg_sets=None, rounds=7, calls_per_round=100, per_graph=20, eager_warmup=5,
               graph_warmup=5):
    """Per-call time by HIP graph replay: 5 eager and 5 graph warmups, then
    `rounds` rounds of about `calls_per_round` forwards (attention + combine),
    each round timed with events; returns (median, stdev) of the per-call
    round means in ms.

    The graph holds `per_graph` forwards back to back, so the GPU never waits
    for the host between them; with `arg_sets` (K/V copies: cold-cache
    timing) it holds one forward per set, so a set is reused only after all
    the others.  per_graph=1 is the one-forward graph the fp8 split-K page
    replays, whose per-call time includes the host's replay cost."""
    import statistics
    torch = r.torch
    sets = arg_sets or [None]
    n = len(sets) if arg_sets else per_graph
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(eager_warmup):
            r.step(side.cuda_stream, sets[i % len(sets)])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(n):
                r.step(side.cuda_stream, sets[i % len(sets)])
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(graph_warmup):
        g.replay()
    torch.cuda.synchronize()
    replays = max(1, -(-calls_per_round // n))
    per = []
    for _ in range(rounds):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(replays):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) / (replays * n))
    return statistics.median(per), statistics.stdev(per)


def cpu_baseline(r, sample_rows=2048):
    """The oracle, as it stands, on this workload's inputs on the host cores.

    Decode and short-prefix workloads run whole (seconds).  Varlen prefill
    would take minutes in fp64, so a bounded random sample of output rows is
    computed one by one and its own attended pairs are counted.
    """
    import numpy as np

    import fmha_synth as fs
    from oracle import oracle as _oracle
    w, prob = r.w, r.prob
    orc = _oracle.load()
    q, k, v = (fs.raw_bits(x.cpu()) for x in (prob.q, prob.k, prob.v))
    kw = dict(cu_q=prob.cu_q, cu_k=prob.cu_k, batch=prob.batch, scale=1 / math.sqrt(w["dqk"]),
              q_descale=prob.q_descale, k_descale=prob.k_descale, v_descale=prob.v_descale,
              causal=w["causal"], window=w["window"])
    if not w["name"].startswith("varlen"):
        t0 = time.perf_counter()
        orc.attention(q, k, v, w["dtype"], **kw)
        dt = time.perf_counter() - t0
        return dict(value=round(alg_bytes(w) / dt / 1e9, 4), unit="GB/s",
                    cores=orc.num_threads(), kind="oracle",
                    sample=f"full workload ({w['desc']}), one fp64 pass in {dt:.2f} s")
    rng = np.random.default_rng(0)
    tq = sum(w["lens_q"])
    rt = rng.integers(0, tq, size=sample_rows)
    rh = rng.integers(0, w["hq"], size=sample_rows)
    starts = np.cumsum([0] + w["lens_q"])
    pairs = 0
    for t in rt:
        b = int(np.searchsorted(starts, t, side="right") - 1)
        sq, sk, i = w["lens_q"][b], w["lens_k"][b], int(t - starts[b])
        pairs += _row_pairs(i, sq, sk, w["causal"], w["window"])
    t0 = time.perf_counter()
    orc.attention_rows(q, k, v, w["dtype"], rt, rh, **kw)
    dt = time.perf_counter() - t0
    flops = 2 * (w["dqk"] + w["dv"]) * pairs
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=orc.num_threads(),
                kind="oracle", sample=f"{sample_rows} random output rows of {w['desc']} "
                                      f"({pairs} attended pairs) in {dt:.2f} s")


def _row_pairs(i, sq, sk, causal, window):
    wl, wr = window
    if causal:
        wr = 0
    d0 = i + sk - sq
    lo = max(0, d0 - wl) if wl >= 0 else 0
    hi = min(sk - 1, d0 + wr) if wr >= 0 else sk - 1
    return max(0, hi - lo + 1)


def load_traffic(name):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(name)
    except (OSError, ValueError):
        return None
    if not t or t.get("kernel") not in KERNEL_SOURCES or t.get("kernel_src_sha") != kernel_source_hash(t["kernel"]):
        return None
    return t.get("bytes_per_launch")


def summarize_pmc(fetch_csv, write_csv, workload, kernel_substr, copy_bytes):
    """Per-launch HBM bytes of the dominant kernel from two rocprofv3 --pmc runs.

    FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by what the
    same counter reads for the plain device copy of ``copy_bytes`` bytes that
    bench.py --copy-calibration-gib runs in the same process.  Writes the
    result (with a hash of the kernel sources) into profiles/traffic.json.
    """
    import csv

    def read(path):
        rows = list(csv.DictReader(open(path)))
        kern = [float(r["Counter_Value"]) for r in rows if kernel_substr in r["Kernel_Name"]]
        copies = [float(r["Counter_Value"]) for r in rows
                  if "copyBuffer" in r["Kernel_Name"] and float(r["Counter_Value"]) > 0.25 * copy_bytes / 1024]
        if not kern or len(copies) != 1:
            raise SystemExit(f"{path}: found {len(kern)} kernel and {len(copies)} calibration dispatches")
        return sum(kern) / len(kern), copies[0], len(kern)

    f_k, f_c, n = read(fetch_csv)
    w_k, w_c, _ = read(write_csv)
    f_scale, w_scale = copy_bytes / (f_c * 1024), copy_bytes / (w_c * 1024)
    fetch_b, write_b = f_k * 1024 * f_scale, w_k * 1024 * w_scale
    entry = dict(kernel_src_sha=kernel_source_hash(kernel_substr), kernel=kernel_substr, dispatches=n,
                 fetch_kib_raw=round(f_k, 3), write_kib_raw=round(w_k, 3),
                 copy_bytes=copy_bytes, copy_fetch_kib_raw=f_c, copy_write_kib_raw=w_c,
                 fetch_scale=round(f_scale, 5), write_scale=round(w_scale, 5),
                 fetch_bytes=int(fetch_b), write_bytes=int(write_b),
                 bytes_per_launch=int(fetch_b + write_b),
                 alg_bytes=alg_bytes(workloads()[workload]))
    data = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    data[workload] = entry
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(entry, indent=1))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-pmc":
        sp = argparse.ArgumentParser()
        sp.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
        sp.add_argument("--workload", default="long_decode")
        sp.add_argument("--kernel", default="fmha_decode_kernel")
        sp.add_argument("--copy-bytes", type=int, default=1 << 30)
        a = sp.parse_args()
        summarize_pmc(*a.summarize_pmc, a.workload, a.kernel, a.copy_bytes)
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_decode")
    ap.add_argument("--splits", type=int, default=0, help="0 = automatic")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="also run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the split-KV "
              "path here is single-GPU", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    W = workloads()
    w = W[args.workload]
    r = Runner(w, args.splits)
    ms_step, ms_kern, wall = time_eager(r, args.steps, args.warmup)

    if args.copy_calibration_gib > 0:
        n = int(args.copy_calibration_gib * (1 << 30))
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[calibration] copied {n} bytes", file=sys.stderr)

    nb, nf = alg_bytes(w), alg_flops(w)
    prefill = w["name"].startswith("varlen")
    if prefill:
        value, unit = nf / (ms_step * 1e-3) / 1e12, "TFLOP/s"
        achieved = nf / (ms_kern * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2),
                    peak=MFMA_PEAK_TFLOPS[w["dtype"]], unit="TFLOP/s")
    else:
        value, unit = nb / (ms_step * 1e-3) / 1e9, "GB/s"
        achieved = nb / (ms_kern * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s")
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = load_traffic(w["name"])
    roof["kernel_us"] = round(ms_kern * 1e3, 2)
    roof["kernel"] = kernel_name(r.plan.kernel_id) + (" (split partials)" if r.split else "")

    others = []
    if not args.no_others:
        for name in ("gqa_decode", "fp8_prefix_16384", "fp8_prefix_16384+in_kernel_combine",
                     "fp8_prefix_11008", "varlen_skewed",
                     "varlen_skewed_causal", "varlen_equal", "varlen_equal_causal",
                     "varlen_many_causal", "varlen_equal_d256", "varlen_equal_causal_d256"):
            if name == w["name"]:
                continue
            fused = name.endswith("+in_kernel_combine")
            o = W[name.split("+")[0]]
            ro = Runner(o, 0, combine_in_kernel=fused)
            med, sd = time_graph(ro)
            us = med * 1e3
            ent = dict(workload=o["desc"] + (" (split combine inside the attention launch)" if fused else ""),
                       us_per_call=round(us, 2), us_stdev=round(sd * 1e3, 2),
                       num_kv_splits=ro.plan.num_splits)
            if name.startswith("fp8"):
                # K/V (tens of MB) fit the 256 MB Infinity Cache: the headline
                # figure cycles through copies spanning 1 GiB (cold), the warm
                # one replays the same buffers
                us_warm = us
                med, sd = time_graph(ro, arg_sets=ro.rotated_args(1 << 30))
                us = med * 1e3
                one, _ = time_graph(ro, per_graph=1)
                ent.update(us_per_call=round(us, 2), us_stdev=round(sd * 1e3, 2),
                           us_per_call_warm=round(us_warm, 2),
                           us_per_call_warm_1fwd_graph=round(one * 1e3, 2))
            if name.startswith("varlen"):
                tf = alg_flops(o) / (us * 1e-6) / 1e12
                ent.update(tflops=round(tf, 1), frac_mfma_peak=round(tf / MFMA_PEAK_TFLOPS[o["dtype"]], 4))
            else:
                gbs = alg_bytes(o) / (us * 1e-6) / 1e9
                ent.update(gbs=round(gbs, 1), frac_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))
                if "us_per_call_warm" in ent:
                    gw = alg_bytes(o) / (ent["us_per_call_warm"] * 1e-6) / 1e9
                    ent.update(gbs_warm=round(gw, 1), frac_hbm_peak_warm=round(gw / HBM_PEAK_GBS, 4))
            others.append(ent)
            del ro
            torch.cuda.empty_cache()

    cpu = None if args.no_cpu_baseline else cpu_baseline(r)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic (seeded N(0,1))",
        "config": {"workload": w["desc"], "batch": len(w["lens_q"]),
                   "seqlen_q": max(w["lens_q"]), "seqlen_k": max(w["lens_k"]),
                   "heads_q": w["hq"], "heads_kv": w["hkv"], "head_dim_qk": w["dqk"],
                   "head_dim_v": w["dv"], "causal": w["causal"],
                   "num_kv_splits": r.plan.num_splits, "split_chunk": r.plan.split_chunk,
                   "alg_bytes": nb, "alg_flops": nf},
        "roofline": roof,
        "cpu_baseline": cpu,
        "others": others,
        "others_method": "per call: median (and stdev) of 7 rounds of ~100 forwards (attention + "
                         "combine) from replays of a HIP graph of 20 back-to-back forwards, after 5 "
                         "eager and 5 graph warmups; fp8 prefix cold = a graph of one forward per "
                         "K/V copy (copies spanning 1 GiB); us_per_call_warm_1fwd_graph = "
                         "100 replays of a one-forward graph (includes the host's replay cost)",
    }
    print(json.dumps(line, ensure_ascii=False))


if __name__ == "__main__":
    main()
