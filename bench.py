"""Prefill throughput of one Llama-3-8B-shape decoder layer on one MI355X.

A step is one tlp_prefill_layer call (the whole layer: RMSNorm, QKV GEMM,
QK-norm/RoPE/KV store, causal GQA attention, O GEMM + residual, FFN norm,
gate/up GEMM + SwiGLU, down GEMM + residual) over a 512-token micro-batch at
start position 0: hidden 4096, intermediate 14336, 32 q / 8 kv heads,
head_dim 128, bf16 weights N(0, 0.02) and inputs N(0, 1), fp32 accumulation.
Every step reads its own copy of the input rows (prepared before the timed
region), so every step does identical work; repeated calls at one start
position rewrite the same cache slots.

The K timed steps are captured once into a HIP graph and replayed (one
untimed replay, then the timed one): `value` and `ms_per_step` come from that
replay, `value_stream` / `ms_per_step_stream` from the same steps enqueued one
library call at a time on the stream (`--no-graph`: `value` from those).  The
32-layer chunk workload is timed as stream launches.

Prints one JSON line: tokens/s per layer, per-kernel HIP-event times from the
library's profiler, the roofline of the dominant kernel (the gate/up GEMM at
start 0, attention for the long-context workload) and the CPU float64 oracle
timed on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "prefill tokens/sec per layer + achieved MFMA TFLOP/s fraction, 8B shape"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def layer_flops(sh, n, start):
    """Algorithmic flops of one layer call: projections and causal attention."""
    H, I, hd, nq, nkv = sh.hidden, sh.inter, sh.head_dim, sh.nq, sh.nkv
    gemm = {
        "qkv_gemm": 2 * n * H * (nq + 2 * nkv) * hd,
        "o_gemm": 2 * n * nq * hd * H,
        "gate_up_gemm": 2 * n * H * 2 * I,
        "down_gemm": 2 * n * I * H,
    }
    keys = n * start + n * (n + 1) // 2
    return gemm, 4 * hd * nq * keys


def kernel_bytes(sh, n, start):
    """Algorithmic HBM bytes per launch: weights read once, activation rows in
    and out (bf16), and the K/V slots attention reads."""
    H, I, hd, nq, nkv = sh.hidden, sh.inter, sh.head_dim, sh.nq, sh.nkv
    qkv = (nq + 2 * nkv) * hd

    def gemm(n_out, k):
        return 2 * (n_out * k + n * k + n * n_out)
    return {
        "qkv_gemm": gemm(qkv, H),
        "o_gemm": gemm(H, nq * hd),
        "gate_up_gemm": 2 * (2 * I * H + n * H + n * I),
        "down_gemm": gemm(H, I),
        "attention": 2 * 2 * (start + n) * nkv * hd + 2 * 2 * n * nq * hd,
    }


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(sh, w, x, kc, vc, budget_s=20.0):
    """The float64 oracle on the host cores: whole layer calls, same inputs,
    with numpy's BLAS on all its threads and once more on one thread."""
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threadpool_limits = None
        blas = os.cpu_count() or 1
    w64 = synth.widen_layer(sh, w)
    x64 = synth.widen(x, sh.dtype)

    def timed_calls(max_calls, budget):
        times = []
        t_all = time.perf_counter()
        while True:
            kc64, vc64 = synth.widen(kc, sh.dtype), synth.widen(vc, sh.dtype)
            t0 = time.perf_counter()
            oracle.prefill_layer(sh, w64, 0, x64, sh.start, kc64, vc64)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_all > budget or len(times) >= max_calls:
                return float(np.mean(times)), len(times)

    t, n = timed_calls(5, budget_s / 2)
    out = {"value": sh.n_tokens / t, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
           "sample": f"{n} full float64 oracle layer call(s) of the same workload "
                     f"({sh.n_tokens} tokens at start {sh.start}), mean {t:.3f} s each",
           "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(), "blas_threads": int(blas)}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            t1, n1 = timed_calls(1, budget_s / 2)
        out["one_thread"] = {"value": sh.n_tokens / t1, "unit": "tokens/s", "cores": 1,
                             "sample": f"{n1} oracle layer call(s) on one BLAS thread, "
                                       f"{t1:.3f} s each"}
    return out


CSRC = os.path.join(ROOT, "transformer_layer_prefill_amd", "csrc")

# the sources that define each library kernel (its own file and the shared
# device header); stored counters of a kernel hold while these are unchanged
KERNEL_SOURCES = {
    "qkv_gemm": ("gemm.hip", "common.h"), "o_gemm": ("gemm.hip", "common.h"),
    "gate_up_gemm": ("gemm.hip", "common.h"), "down_gemm": ("gemm.hip", "common.h"),
    "attention": ("attention.hip", "common.h"),
}


def source_sha256() -> dict:
    """SHA-256 of every HIP source file; stored traffic counters apply to the
    kernels whose source files still hash the same."""
    import hashlib
    out = {}
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            out[f] = hashlib.sha256(fh.read()).hexdigest()
    return out


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes (scaled by the copy calibration), or None when they were
    taken on other sources of that kernel or are absent."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    now, then = source_sha256(), t.get("source_sha256", {})
    if not isinstance(then, dict):
        return None
    for name, v in t["kernels"].items():
        if name.split(" | ")[0] == kernel:
            # the files that define the kernel symbol the counters were taken on
            files = v.get("sources") or KERNEL_SOURCES.get(kernel, tuple(now))
            if any(now.get(f) != then.get(f) for f in files):
                return None
            return {"bytes": round(v["fetch_bytes"] + v["write_bytes"]),
                    "fetch_bytes": round(v["fetch_bytes"]), "write_bytes": round(v["write_bytes"]),
                    "source": f"profiles/traffic_{workload}.json"}
    return None


def copy_probe(mib: int) -> None:
    """Copy mib MiB device-to-device five times: a kernel that reads and writes
    exactly mib MiB each, against which FETCH_SIZE / WRITE_SIZE are scaled."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_mib": mib, "bytes_read": n * 4, "bytes_written": n * 4}))


def bench_verify_tail(args):
    """Speculative-verify tail of the Llama-3-8B head: final RMSNorm of 16 rows,
    LM-head projection to 128256 fp32 logits per row, per-row argmax.  HBM
    bound: the 1.05 GB head is read once per call."""
    import torch
    import transformer_layer_prefill_amd as tlp
    from transformer_layer_prefill_amd import tensors
    rows, H, V = 16, 4096, 128256
    sh = synth.Shape("llama3-8b-verify-tail", hidden=H, inter=14336, nq=32, nkv=8,
                     head_dim=128, qk_norm=False, eps=1e-5, theta=5e5, n_tokens=rows,
                     start=0, max_seq=4096, vocab=V, seed=1004)
    log("[bench] generating the 128256 x 4096 head")
    x = tensors.to_device(synth.hidden_input(sh))
    g = tensors.to_device(synth.final_norm(sh))
    W = tensors.to_device(synth.lm_head(sh, workers=16))
    cfg = tensors.config_of(sh)
    logits = torch.empty((rows, V), dtype=torch.float32, device="cuda")
    tokens = torch.empty(rows, dtype=torch.int32, device="cuda")
    ws = torch.empty(tlp.verify_workspace_bytes(cfg, rows), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        tlp.verify_tail(cfg, x, rows, g, W, V, sh.eps, logits, tokens, ws, stream=stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # the K steps captured into a HIP graph and replayed (the tail's inputs
    # are not overwritten, so replays repeat the same work)
    stream_ms = ms
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                tlp.verify_tail(cfg, x, rows, g, W, V, sh.eps, logits, tokens, ws)
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        graph.replay()
        g1.record()
        torch.cuda.synchronize()
        ms = g0.elapsed_time(g1) / args.steps
        del graph
    tlp.profile_begin()
    for _ in range(args.steps):
        step()
    prof = tlp.profile_end()
    prof.pop("not_timed", None)
    kernels = {k: {"launches": n, "avg_us": round(1e3 * t / n, 3)} for k, (n, t) in prof.items() if n}
    head_us = kernels["lm_head"]["avg_us"]
    head_bytes = 2 * V * H + 2 * rows * H + 4 * rows * V
    achieved = head_bytes / (head_us * 1e-6) / 1e9
    out = {
        "metric": "verify-tail rows/sec (final norm + LM head + argmax)", "value": round(rows / (ms * 1e-3), 1),
        "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": sh.name, "rows": rows, "hidden": H, "vocab": V,
                   "launch": "stream" if args.no_graph else "hip_graph",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "lm_head", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": None, "avg_us": head_us, "bytes_per_launch": head_bytes},
        "cpu_baseline": None,
        "kernels": kernels,
        "ms_per_step_stream": round(stream_ms, 4),
        "value_stream": round(rows / (stream_ms * 1e-3), 1),
    }
    print(json.dumps(out), flush=True)


def bench_stack(args):
    """The 32-layer chunked prefill: 4096 prompt tokens in micro-batches of
    512 through 32 Llama-3-8B-shape layers, then the final norm and the
    128256-row LM head on the last token.  One step is one tlp_prefill_chunk
    call; value = 4096 * 32 / step time (tokens/s per layer)."""
    import torch
    import transformer_layer_prefill_amd as tlp
    from transformer_layer_prefill_amd import tensors
    sh = synth.WORKLOADS["llama3-8b-stack32"]
    if args.kv_f16:
        sh = sh.replace(kv="f16")
    log(f"[bench] generating {sh.n_layers} layers and the head")
    layers = synth.stack_weights(sh, workers=16)
    dev = torch.device("cuda", 0)
    dls = [tensors.DeviceLayer(w, dev) for w in layers]
    del layers
    x0 = tensors.to_device(synth.hidden_input(sh), dev)
    kc, vc = synth.kv_caches(sh)
    kcd, vcd = tensors.to_device(kc, dev), tensors.to_device(vc, dev)
    del kc, vc
    fn = tensors.to_device(synth.final_norm(sh), dev)
    W = tensors.to_device(synth.lm_head(sh, workers=16), dev)
    cfg = tensors.config_of(sh)
    cos, sin = tlp.rope_table(sh.theta, sh.head_dim, sh.max_seq)
    cosd, sind = tensors.to_device(cos, dev), tensors.to_device(sin, dev)
    mb = sh.micro_batch
    # two workspaces: consecutive micro-batches run on two streams, one layer apart
    copies = 1 if args.no_pipeline else 2
    ws = torch.empty(copies * tlp.workspace_bytes(cfg, min(sh.n_tokens, mb)), dtype=torch.uint8,
                     device=dev)
    logits = torch.empty(sh.vocab, dtype=torch.float32, device=dev)
    pipeline = None if args.no_pipeline else tlp.Pipeline(sh.n_layers)
    structs = [d.struct for d in dls]
    # the profiled passes cover a few steps: one call makes ~2300 launches,
    # each bracketed by two events
    n_prof = min(args.steps, 2)
    n_buf = args.warmup + args.steps + n_prof
    hiddens = [x0.clone() for _ in range(n_buf)]
    stream = torch.cuda.current_stream(dev)

    one_ws = tlp.workspace_bytes(cfg, min(sh.n_tokens, mb))

    def step(i, one_stream=False):
        tlp.prefill_chunk(cfg, structs, hiddens[i], sh.n_tokens, sh.start, mb, kcd, vcd, cosd,
                          sind, ws, final_norm=fn, lm_head=W, vocab=sh.vocab, final_eps=sh.eps,
                          logits=logits, stream=stream, pipeline=None if one_stream else pipeline,
                          workspace_bytes=one_ws if one_stream else None)
    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    # per-kernel times from a one-stream pass (with two micro-batches in flight
    # a kernel's events would also span the other stream's kernels); the
    # profiler's events are all created by profile_begin, before the pass
    tlp.profile_begin(max_launches=4096 * n_prof)
    for i in range(n_prof):
        step(args.warmup + args.steps + i, one_stream=True)
    prof = tlp.profile_end()
    prof.pop("not_timed", None)

    # one chunk call captured into a HIP graph behind a copy that restores the
    # prompt rows (so every replay does the same work), replayed K times; a
    # captured call runs its micro-batches one at a time on the capture stream
    graph_ms = None
    if not args.no_graph:
        gh = hiddens[0]
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            gh.copy_(x0)
            tlp.prefill_chunk(cfg, structs, gh, sh.n_tokens, sh.start, mb, kcd, vcd, cosd, sind,
                              ws, final_norm=fn, lm_head=W, vocab=sh.vocab, final_eps=sh.eps,
                              logits=logits)
        graph.replay()
        torch.cuda.synchronize()
        log(f"[bench] timing {args.steps} graph replays")
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        del graph
    kernels = {k: {"launches": n, "avg_us": round(1e3 * t / n, 3)} for k, (n, t) in prof.items() if n}
    gemm_flops, _ = layer_flops(sh, mb, 0)
    for k, f in gemm_flops.items():
        kernels[k]["tflops"] = round(f / (kernels[k]["avg_us"] * 1e-6) / 1e12, 2)
    dom_us = kernels["gate_up_gemm"]["avg_us"]
    achieved = gemm_flops["gate_up_gemm"] / (dom_us * 1e-6) / 1e12
    tokens_layers = sh.n_tokens * sh.n_layers
    out = {
        "metric": "prefill tokens/sec per layer, 32-layer chunked prefill + head",
        "value": round(tokens_layers / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": sh.dtype,
        "data": "synthetic",
        "config": {"workload": sh.name, "tokens": sh.n_tokens, "layers": sh.n_layers,
                   "micro_batch": mb, "micro_batches_in_flight": copies, "vocab": sh.vocab,
                   "kv_cache": sh.kv_dtype,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "gate_up_gemm", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "avg_us": dom_us, "flops_per_launch": gemm_flops["gate_up_gemm"]},
        "cpu_baseline": None,
        "kernels": kernels,
        "wall_s_timed": round(wall, 3),
        "ms_per_step_graph_one_stream": None if graph_ms is None else round(graph_ms, 3),
        "kernels_timed_on": f"one stream (micro-batches one at a time), {n_prof} steps",
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3-8b-layer",
                    choices=["llama3-8b-layer", "qwen3-8b-sign1-layer", "llama3-8b-long-ctx",
                             "llama3-8b-decode", "llama3-8b-long-decode",
                             "llama3-8b-verify-tail", "llama3-8b-stack32", "tiny-f32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="layer workloads: time the steps as stream launches only (value from "
                         "them) instead of replaying them from a HIP graph")
    ap.add_argument("--no-pipeline", action="store_true",
                    help="32-layer chunk: one workspace, so one micro-batch at a time on one stream")
    ap.add_argument("--kv-f16", action="store_true",
                    help="keep the KV cache in IEEE fp16 (the cache type of metal_full_layer.rs)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, 5 times "
                         "(the calibration kernel for HBM traffic counters), then exit")
    args = ap.parse_args()
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); sharding the "
              "layer over several GPUs is not built, so there is no multi-GPU run",
              file=sys.stderr)
        sys.exit(2)

    if args.workload == "llama3-8b-verify-tail":
        bench_verify_tail(args)
        return
    if args.workload == "llama3-8b-stack32":
        bench_stack(args)
        return

    import torch
    import transformer_layer_prefill_amd as tlp
    from transformer_layer_prefill_amd import tensors

    sh = synth.WORKLOADS[args.workload]
    if args.kv_f16:
        sh = sh.replace(kv="f16")
    log(f"[bench] generating {sh.name}")
    w = synth.layer_weights(sh, 0)
    x = synth.hidden_input(sh)
    kc, vc = synth.kv_caches(sh)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cfg = tensors.config_of(sh)
    dl = tensors.DeviceLayer(w, dev)
    kcd, vcd = tensors.to_device(kc, dev), tensors.to_device(vc, dev)
    cos, sin = tlp.rope_table(sh.theta, sh.head_dim, sh.max_seq)
    cosd, sind = tensors.to_device(cos, dev), tensors.to_device(sin, dev)
    x0 = tensors.to_device(x, dev)
    ws = torch.empty(tlp.workspace_bytes(cfg, sh.n_tokens), dtype=torch.uint8, device=dev)
    n_buf = args.warmup + args.steps
    hiddens = [x0.clone() for _ in range(n_buf)]
    stream = torch.cuda.current_stream(dev)

    def step(i):
        tlp.prefill_layer(cfg, dl.struct, 0, hiddens[i], sh.n_tokens, sh.start, kcd, vcd, cosd,
                          sind, ws, stream=stream)

    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K steps bracketed by synchronisation, nothing else on the
    # stream; `value` comes from here
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    value = sh.n_tokens / (ms_step * 1e-3)

    # the same K steps again with the library's profiler on: HIP events on the
    # kernels' own stream around every launch give the per-kernel times (the
    # extra event packets lengthen the step a little: ms_per_step_profiled)
    tlp.profile_begin()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    prof = tlp.profile_end()
    prof.pop("not_timed", None)
    ms_step_prof = e0.elapsed_time(e1) / args.steps

    # the same K steps captured once into a HIP graph (each with its own input
    # copy, restored before the timed replay) and replayed: the step time
    # without the host's launch path between dependent kernels
    graph_ms = None
    if not args.no_graph:
        gh = [x0.clone() for _ in range(args.steps)]
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                tlp.prefill_layer(cfg, dl.struct, 0, gh[i], sh.n_tokens, sh.start, kcd, vcd,
                                  cosd, sind, ws)
        for rep_i in range(2):   # one untimed replay, then the timed one
            for h in gh:
                h.copy_(x0)
            torch.cuda.synchronize()
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g0.record()
            graph.replay()
            g1.record()
            torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        del graph, gh

    gemm_flops, attn_flops = layer_flops(sh, sh.n_tokens, sh.start)
    kernels = {}
    for k, (n, ms) in prof.items():
        if n:
            kernels[k] = {"launches": n, "avg_us": 1e3 * ms / n}
    gemm_us = sum(kernels[k]["avg_us"] for k in gemm_flops)
    proj_tflops = sum(gemm_flops.values()) / (gemm_us * 1e-6) / 1e12
    attn_us = kernels["attention"]["avg_us"]
    attn_tflops = attn_flops / (attn_us * 1e-6) / 1e12
    for k, f in gemm_flops.items():
        kernels[k]["tflops"] = f / (kernels[k]["avg_us"] * 1e-6) / 1e12
    kernels["attention"]["tflops"] = attn_tflops

    # the dominant kernel: the one with the longest launches among the
    # projections and attention (the gate/up GEMM at short context, attention
    # at long context).  Prefill micro-batches are MFMA-bound; decode steps
    # (a few rows) read every weight once per step and are HBM-bound.
    dom_flops = dict(gemm_flops, attention=attn_flops)
    dom = max(dom_flops, key=lambda k: kernels[k]["avg_us"])
    dom_us = kernels[dom]["avg_us"]
    if sh.n_tokens > 32:
        achieved = dom_flops[dom] / (dom_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": None,
                    "avg_us": round(dom_us, 2), "flops_per_launch": dom_flops[dom]}
    else:
        nbytes = kernel_bytes(sh, sh.n_tokens, sh.start)[dom]
        achieved = nbytes / (dom_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": None,
                    "avg_us": round(dom_us, 2), "bytes_per_launch": nbytes}
        for k, b in kernel_bytes(sh, sh.n_tokens, sh.start).items():
            kernels[k]["GBps"] = b / (kernels[k]["avg_us"] * 1e-6) / 1e9

    tr = stored_traffic(sh.name, dom)
    if tr is not None:
        roofline["traffic"] = tr["bytes"]
        roofline["traffic_detail"] = tr

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (float64 oracle on the host cores)")
        cpu = cpu_baseline(sh, w, x, kc, vc)

    # value: the K steps replayed from the HIP graph (the same kernels on the
    # same resident inputs, launched by the GPU's command processor without the
    # host's launch path between dependent kernels); --no-graph: enqueued one
    # call at a time on the stream
    eager_value, eager_ms = value, ms_step
    if graph_ms is not None:
        ms_step, value = graph_ms, sh.n_tokens / (graph_ms * 1e-3)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": sh.dtype,
        "data": "synthetic",
        "config": {"workload": sh.name, "tokens": sh.n_tokens, "start_position": sh.start,
                   "hidden": sh.hidden, "intermediate": sh.inter, "q_heads": sh.nq,
                   "kv_heads": sh.nkv, "head_dim": sh.head_dim, "weights": sh.wformat,
                   "kv_cache": sh.kv_dtype,
                   "launch": "hip_graph" if graph_ms is not None else "stream",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "mfma_frac": {"projections": round(proj_tflops / PEAK_BF16_TFLOPS, 4),
                      "attention": round(attn_tflops / PEAK_BF16_TFLOPS, 4)},
        "kernels": {k: {kk: round(vv, 3) if isinstance(vv, float) else vv
                        for kk, vv in v.items()} for k, v in kernels.items()},
        "wall_s_timed": round(wall, 4),
        "ms_per_step_profiled": round(ms_step_prof, 4),
        "ms_per_step_stream": round(eager_ms, 4),
        "value_stream": round(eager_value, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
