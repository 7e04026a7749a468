"""Throughput of the packed embedding pass on one MI355X.

A step is one pass of the whole path over one batch of synthetic input: for
the default workload, 64 packs of <= 2048 tokens (texts of log-uniform
length in [8, 512], greedy packing; full-size 25-layer 768-d encoder with
bf16 weights and matmul operands, fp32 accumulation), one tte_embed call per
pack.  Packs are dealt round-robin to --streams concurrent HIP streams (4),
one model (workspace) per stream over one shared copy of the weights and
one host thread per stream enqueueing its packs, the way a server answers
concurrent requests; the process asks the HIP runtime for two hardware
queues per stream.  Token ids and weights are resident in
HBM before timing starts; the timed region is bracketed by device
synchronisation and measured on the host clock.

Prints ONE JSON line: tokens/s (every token of every text, BOS/EOS included),
the roofline of the dominant kernel, and the CPU oracle timed on a bounded
sample of the same workload on the host's cores.  An untimed single-stream
step with an event pair around every launch gives each kernel class's time
and work rate ("kernels": TFLOP/s and fraction of peak for the GEMMs and
attention, GB/s for the row kernels); the dominant kernel is the one with
the most time there (the two residual products, Wo and Wo2, are one kernel).
Its roofline comes from a second timed pass of the same steps on a single
stream with a HIP event pair recorded in the dispatch of every launch of
that kernel (with several streams, kernels of different packs overlap and
per-launch durations would include the time they share the chip).
"configs" adds, from the same process, the other workloads: the fp32
957-token pack, the 4 x 4096-token bf16 pack, the int8 and 4-bit pack
streams (tokens/s and their own dominant kernel's fraction of peak).

--row-kernels prints a different line instead: the HBM-bound row kernels
(LayerNorm fp32 -> bf16 as in front of the bf16 products, and the per-row
7-bit quantisation of the integer paths) through the C ABI at one pack's
shape and at a 1 GiB fp32 input, as algorithmic bytes per launch over the
mean time of back-to-back launches (HIP events on the launching stream).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "encoded tokens/sec (25-layer 768-d encoder, ~2048-token packs) + % MFMA peak"
# the 4-bit path unpacks its codes to int8 and runs the int8 MFMA: int8 peak
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3, "int8": 5000.0, "int4": 5000.0}
DTYPE = {"bf16": "bf16", "fp32": "f32", "int8": "int8", "int4": "int8 (4-bit weights)"}
# flops per token of each GEMM class (H = 768, I = 3072): 2 * N * K
GEMM_CLASSES = {"gemm_qkv": lambda H, I: 2 * 3 * H * H, "gemm_o": lambda H, I: 2 * H * H,
                "gemm_geglu": lambda H, I: 2 * 2 * I * H, "gemm_o2": lambda H, I: 2 * H * I}


# kernels by name -> the classes of tte_profile whose launches they run; the
# residual products (Wo, Wo2) are one kernel template with the same tile
KERNEL_GROUPS = {"k_gemm residual (Wo + Wo2)": ["gemm_o", "gemm_o2"], "k_gemm geglu (Wi)": ["gemm_geglu"],
                 "k_gemm qkv": ["gemm_qkv"], "k_attn (global + local)": ["attn_global", "attn_local"],
                 "k_ln": ["norm"], "k_quant7": ["quant"], "k_pool": ["pool"], "k_embed_ln": ["embed"]}
GROUP_FILES = {"k_gemm residual (Wo + Wo2)": "kernels_gemm.hip", "k_gemm geglu (Wi)": "kernels_gemm.hip",
               "k_gemm qkv": "kernels_gemm.hip", "k_attn (global + local)": "kernels_attn.hip"}
GROUP_PROFILES = {"k_gemm residual (Wo + Wo2)": "traffic_gemm_resid_full_bf16_packs2048.json",
                  "k_gemm geglu (Wi)": "traffic_gemm_geglu_full_bf16_packs2048.json"}


def traffic_from_profile(kernel_source: str, profile: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None if the kernel source changed since it was taken."""
    import hashlib
    try:
        meta = json.load(open(profile))
        src = open(kernel_source, "rb").read()
    except OSError:
        return None
    if hashlib.sha256(src).hexdigest()[:16] != meta.get("source_sha256_16"):
        return None
    return meta["per_launch_mean"]["traffic_bytes"]


HBM_GBS = 8000.0


def row_kernels(torch, B, dev, reps=20):
    """Algorithmic GB/s of LayerNorm (fp32 in, bf16 out, gain read once) and
    7-bit quantisation (fp32 in, int8 codes and one fp32 scale per row out)
    at widths of 768, for 1913 rows (a mean pack) and 1 GiB of input."""
    H = 768
    s = torch.cuda.current_stream()
    res = []
    for rows in (1913, (1 << 30) // (4 * H)):
        g = torch.Generator(device=dev).manual_seed(7)
        x = torch.randn(rows, H, device=dev, generator=g)
        gamma = torch.ones(H, device=dev)
        out = torch.empty(rows, H, dtype=torch.bfloat16, device=dev)
        q = torch.empty(rows, H, dtype=torch.int8, device=dev)
        sc = torch.empty(rows, device=dev)
        kernels = (
            ("layernorm fp32 -> bf16", rows * H * (4 + 2) + H * 4,
             lambda: B.tte_op_layernorm(x.data_ptr(), gamma.data_ptr(), rows, H, 1e-5, B.TTE_OUT_BF16,
                                        out.data_ptr(), 0, s.cuda_stream)),
            ("quant7 fp32 -> int8", rows * H * (4 + 1) + rows * 4,
             lambda: B.tte_op_quant7(x.data_ptr(), rows, H, q.data_ptr(), sc.data_ptr(), s.cuda_stream)),
        )
        for name, nbytes, fn in kernels:
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(reps):
                fn()
            e1.record(s)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            gbs = nbytes / us / 1e3
            res.append({"kernel": name, "rows": rows, "width": H, "bytes": nbytes, "us": round(us, 2),
                        "GB/s": round(gbs, 1), "frac_of_hbm": round(gbs / HBM_GBS, 4)})
        del x, out, q, sc
    # the practical ceiling: a plain device copy of 1 GiB (torch), read + write
    src = torch.ones((1 << 30) // 4, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    res.append({"kernel": "device copy (torch), reference", "rows": None, "width": None, "bytes": 2 << 30,
                "us": round(us, 2), "GB/s": round((2 << 30) / us / 1e3, 1),
                "frac_of_hbm": round((2 << 30) / us / 1e3 / HBM_GBS, 4)})
    return res


def allowed_pairs(lengths, window):
    """(query, key) pairs attention computes: global layers see the whole
    text, local ones keys at most `window` positions away."""
    lengths = [int(L) for L in lengths]  # Python ints: the totals overflow int32
    g = sum(L * L for L in lengths)
    loc = 0
    for L in lengths:
        i = np.arange(L)
        loc += int(np.sum(np.minimum(L, i + window + 1) - np.maximum(0, i - window)))
    return g, loc


def class_work(cfg, packs):
    """Algorithmic work of one step per kernel class: (amount, unit, peak).
    GEMMs 2 N K flops per token; attention 4 * head_dim flops per allowed
    pair per head; the row kernels the bytes they must read and write."""
    H, I, Lyr = cfg.hidden, cfg.intermediate, cfg.layers
    T = sum(p.n_tokens for p in packs)
    gemm_peak = PEAK_TFLOPS[cfg.precision]
    attn_peak = PEAK_TFLOPS["bf16"] if cfg.precision == "bf16" else PEAK_TFLOPS["fp32"]
    n_glob = len([l for l in range(Lyr) if l % cfg.global_every == 0])
    pg = pl = 0
    for p in packs:
        g, loc = allowed_pairs(np.diff(p.offsets), cfg.window)
        pg, pl = pg + g, pl + loc
    per_pair = 4 * cfg.head_dim * cfg.heads
    out_b = {"bf16": 2, "fp32": 4, "int8": 1, "int4": 1}[cfg.precision]
    w = {k: (f(H, I) * T * Lyr, "TFLOP/s", gemm_peak) for k, f in GEMM_CLASSES.items()}
    w["attn_global"] = (pg * per_pair * n_glob, "TFLOP/s", attn_peak)
    w["attn_local"] = (pl * per_pair * (Lyr - n_glob), "TFLOP/s", attn_peak)
    x_b = 2 if cfg.precision == "bf16" else 4  # element bytes of the residual stream
    # 2 L - 1 norms (layer 0's attention input is the embedding norm's
    # output): read x rows, write the GEMM operand
    w["norm"] = ((2 * Lyr - 1) * T * H * (x_b + out_b), "GB/s", None)
    w["pool"] = (T * H * x_b, "GB/s", None)
    return w


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(name, cfg, w, packs, budget_tokens):
    """The oracle as it stands on the workload's first packs, one oracle call
    per pack, until at least budget_tokens tokens are covered."""
    import oracle
    import threadpoolctl
    n, used = 0, 0
    t0 = time.perf_counter()
    for p in packs:
        if n >= budget_tokens:
            break
        oracle.encode(cfg.as_dict(), w, p.ids, p.offsets)
        n += p.n_tokens
        used += 1
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    # the oracle computes in fp64 by design (it is the reference the GPU
    # paths are measured against); it is timed as it stands
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {used} packs ({n} tokens) of the workload, fp64 numpy oracle as it stands, {dt:.1f}s",
            "host_cpus": os.cpu_count(), "cpu_model": model, "blas_threads": threads}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="full_bf16_packs2048")
    ap.add_argument("--streams", type=int, default=4,
                    help="concurrent streams, one model each (4 measured best, with 8 hardware queues)")
    ap.add_argument("--output", choices=("pooled", "tokens"), default="pooled",
                    help="pooled unit vectors per text (tte_embed) or per-token states (tte_embed_tokens)")
    ap.add_argument("--split-k", action="store_true",
                    help="TTE_FLAG_SPLIT_K: split the down-projection of short packs (lower single-call latency)")
    ap.add_argument("--merged", action="store_true",
                    help="secondary number: all packs of a step concatenated into one call on one stream")
    ap.add_argument("--one-host-thread", dest="host_threads", action="store_false",
                    help="enqueue every stream's packs from the main thread (default: one host thread per stream, "
                         "as concurrent request handlers would)")
    ap.add_argument("--graph", action="store_true",
                    help="TTE_FLAG_GRAPH: replay each pack's captured HIP graph (needs --warmup >= 2)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=7000,
                    help="the CPU oracle times the first packs covering this many tokens (~15 s on 16 host threads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time the steps without the per-launch events of the dominant kernel")
    ap.add_argument("--no-breakdown", dest="breakdown", action="store_false",
                    help="leave the per-class kernel times of the untimed single-stream step out of the line")
    ap.add_argument("--no-configs", dest="configs", action="store_false",
                    help="skip the other workloads (fp32 957-token pack, 4 x 4096 bf16, int8 and 4-bit packs)")
    ap.add_argument("--row-kernels", action="store_true",
                    help="only measure the row kernels' HBM rate (LayerNorm, 7-bit quantisation) at two shapes")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized fp32 buffer 5 times with torch (known bytes, for HBM counter scaling)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    # Each concurrent stream needs a hardware queue of its own.  The HIP
    # runtime gives a process 4 by default; with 4 streams they collide
    # (measured on MI355X: 1.04M tokens/s on 4 queues against 1.30M on 8),
    # so the bench asks for twice the stream count (at most 32) before HIP
    # initialises.
    if a.streams > 1 and int(os.environ.get("GPU_MAX_HW_QUEUES", "4")) < 2 * a.streams:
        os.environ["GPU_MAX_HW_QUEUES"] = str(min(32, 2 * a.streams))

    import torch

    import tte_inputs as ti
    from transformer_text_embedding_amd import B, Model

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if a.copy_calibration:
        n = a.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "copies": 5}), flush=True)
        return
    if a.row_kernels:
        res = row_kernels(torch, B, dev)
        big = [r for r in res if r["kernel"].startswith("layernorm") and r["rows"] > 1913][0]
        print(json.dumps({"metric": "row kernels: algorithmic HBM GB/s (LayerNorm fp32 -> bf16 at 1 GiB)",
                          "value": big["GB/s"], "unit": "GB/s", "n_gpus": 1, "higher_is_better": True,
                          "peak": HBM_GBS, "data": "synthetic", "results": res}), flush=True)
        return
    runner = Runner(torch, ti, B, Model, a.workload, a.streams, merged=a.merged, per_token=a.output == "tokens",
                    split_k=a.split_k, graph=a.graph, host_threads=a.host_threads)
    runner.run_steps(a.warmup)
    torch.cuda.synchronize()
    log("warmup done")
    secs = runner.timed(a.steps)
    value = runner.tokens_per_step * a.steps / secs
    log(f"timed {a.steps} steps on {runner.S} streams: {secs * 1e3:.2f} ms")

    # per-class kernel time of one untimed single-stream step; the dominant
    # kernel is the one with the most time there
    breakdown = runner.breakdown()
    dominant = max((g for g in KERNEL_GROUPS if any(breakdown.get(c, {}).get("launches") for c in KERNEL_GROUPS[g])),
                   key=lambda g: sum(breakdown.get(c, {}).get("ms", 0.0) for c in KERNEL_GROUPS[g]))
    roofline, single_ms = None, None
    if not a.no_kernel_events:
        roofline, single_ms = runner.roofline(dominant, a.steps)
        if roofline is not None and not a.merged and a.workload == "full_bf16_packs2048" and dominant in GROUP_PROFILES:
            roofline["traffic"] = traffic_from_profile(
                os.path.join(ROOT, "transformer_text_embedding_amd", "csrc", GROUP_FILES[dominant]),
                os.path.join(ROOT, "profiles", GROUP_PROFILES[dominant]))
    torch.cuda.synchronize()
    cfg = runner.cfg
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(secs * 1e3 / a.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE[cfg.precision], "data": "synthetic",
        "config": {"workload": a.workload, "packs_per_step": len(runner.cpu_packs),
                   "tokens_per_step": runner.tokens_per_step, "pack_budget": runner.spec.get("pack_budget"),
                   "layers": cfg.layers, "hidden": cfg.hidden, "heads": cfg.heads, "intermediate": cfg.intermediate,
                   "calls_per_step": len(runner.packs), "streams": runner.S,
                   "hw_queues": int(os.environ.get("GPU_MAX_HW_QUEUES", "4")), "output": a.output,
                   "split_k": a.split_k, "graph": a.graph, "merged": a.merged, "host_threads": a.host_threads,
                   "single_stream_ms_per_step": round(single_ms, 3) if single_ms else None},
        "roofline": roofline,
    }
    if a.breakdown:
        line["kernels"] = public(breakdown)
    cpu_w, cpu_packs = runner.w, runner.cpu_packs
    runner.close()
    if a.configs and a.workload == "full_bf16_packs2048" and not a.merged and a.output == "pooled":
        line["configs"] = {}
        for key, name, steps, streams, split_k in SECONDARY:
            log(f"config {key}")
            r = Runner(torch, ti, B, Model, name, streams or a.streams, split_k=split_k, host_threads=a.host_threads)
            r.run_steps(2)
            torch.cuda.synchronize()
            sec = r.timed(steps)
            bd = r.breakdown()
            dom = max((g for g in KERNEL_GROUPS if any(bd.get(c, {}).get("launches") for c in KERNEL_GROUPS[g])),
                      key=lambda g: sum(bd.get(c, {}).get("ms", 0.0) for c in KERNEL_GROUPS[g]))
            line["configs"][key] = {
                "tokens_per_s": round(r.tokens_per_step * steps / sec, 1), "ms_per_step": round(sec * 1e3 / steps, 3),
                "steps": steps, "warmup": 2, "streams": r.S, "split_k": split_k, "calls_per_step": len(r.packs),
                "tokens_per_step": r.tokens_per_step,
                "dtype": DTYPE[r.cfg.precision], "dominant_kernel": dom, "dominant_frac_of_peak": group_frac(bd, dom),
                "residual_frac_of_peak": group_frac(bd, "k_gemm residual (Wo + Wo2)"),
                "kernels": public(bd)}
            r.close()
            torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        log("timing the CPU oracle sample")
        line["cpu_baseline"] = cpu_baseline(a.workload, cfg, cpu_w, cpu_packs, a.cpu_sample_tokens)
    print(json.dumps(line), flush=True)


# other lines measured in the default run: (key, workload, timed steps,
# streams (None: --streams), TTE_FLAG_SPLIT_K).  The last is the headline
# workload as a single caller would run it: one stream, the down-projection
# split over K so that a lone pack fills the CUs (lower latency per pack).
SECONDARY = [("full_fp32_957", "full_fp32_957", 30, None, False),
             # the same lone pack in the library's latency mode (one caller,
             # one call at a time: the residual products split over K)
             ("full_fp32_957_split_k", "full_fp32_957", 30, None, True),
             ("full_bf16_4x4096", "full_bf16_4x4096", 10, None, False),
             ("full_int8_packs2048", "full_int8_packs2048", 10, None, False),
             ("full_int4_packs2048", "full_int4_packs2048", 10, None, False),
             ("full_bf16_packs2048_one_stream_split_k", "full_bf16_packs2048", 5, 1, True)]


def public(bd):
    """A breakdown for the output line: the private work / peak fields
    dropped."""
    out = {k: {f: v for f, v in e.items() if not f.startswith("_")} for k, e in bd.items()}
    out["measured_in"] = "untimed single-stream step, events in each launch's dispatch (pool: around its 2 kernels)"
    return out


def group_frac(bd, group):
    """Fraction of peak of a kernel group from a breakdown: summed work over
    summed time of its classes."""
    present = [c for c in KERNEL_GROUPS[group] if c in bd and "_work" in bd[c]]
    if not present:
        return None
    work = sum(bd[c]["_work"] for c in present)
    ms = sum(bd[c]["ms"] for c in present)
    unit_scale = 1e12 if "TFLOP/s" in bd[present[0]] else 1e9
    return round(work / (ms / 1e3) / unit_scale / bd[present[0]]["_peak"], 4) if ms else None


_STREAMS = []


def shared_streams(torch, dev, n):
    """The first n of one list of streams that every Runner of the process
    shares.  HIP maps streams onto its hardware queues in creation order
    and reuses them round-robin, so fresh streams for each workload would
    land on queues that other (idle) streams already hold; reusing the
    same streams keeps every workload's packs on their own queues."""
    while len(_STREAMS) < n:
        _STREAMS.append(torch.cuda.Stream(device=dev))
    return _STREAMS[:n]


class Runner:
    """One workload on S concurrent streams: one model (workspace) per stream
    over one shared copy of the weights, packs dealt round-robin, one host
    thread per stream enqueueing its packs (or all from this thread)."""

    def __init__(self, torch, ti, B, Model, workload, streams, merged=False, per_token=False, split_k=False,
                 graph=False, host_threads=True):
        self.torch, self.B = torch, B
        dev = torch.device("cuda:0")
        self.spec = ti.workload(workload)
        self.cfg = cfg = self.spec["cfg"]
        t0 = time.perf_counter()
        self.w = ti.cached_storage_weights(cfg)
        packs = ti.make_packs(workload)
        self.cpu_packs = packs  # the CPU baseline always takes the workload's own packs
        if merged:
            # texts are independent: the whole step as one pack (one call)
            packs = [ti.pack_from_texts([p.text(b) for p in packs for b in range(p.n_texts)])]
            streams = 1
        self.packs = packs
        log(f"{workload}: inputs ready in {time.perf_counter() - t0:.1f}s: {len(packs)} packs, "
            f"{sum(p.n_tokens for p in packs)} tokens")
        max_tokens = max(p.n_tokens for p in packs)
        # a workload of one pack runs on one stream (its latency)
        self.S = S = max(1, min(streams, len(packs)))
        max_texts = max(1024, max(p.n_texts for p in packs))
        max_len = max(512, max(int(np.diff(p.offsets).max()) for p in packs))
        model = Model(cfg, self.w, max_tokens=max_tokens, max_text_len=max_len, max_texts=max_texts,
                      device="cuda:0", split_k=split_k, graph=graph)
        self.models = [model] + [Model(cfg, None, max_tokens=max_tokens, max_text_len=max_len, max_texts=max_texts,
                                       device="cuda:0", shared_from=model, split_k=split_k, graph=graph)
                                 for _ in range(S - 1)]
        self.streams = shared_streams(torch, dev, S)
        self.ids = [torch.from_numpy(p.ids).to(dev) for p in packs]
        self.outs = [torch.empty((p.n_tokens if per_token else p.n_texts, cfg.hidden), dtype=torch.float32,
                                 device=dev) for p in packs]
        self.offs = [B.int32_array(p.offsets) for p in packs]
        L = B.lib()
        self.embed = L.tte_embed_tokens if per_token else L.tte_embed
        self.host_threads = host_threads
        self.tokens_per_step = sum(p.n_tokens for p in packs)

    def call(self, i, k):
        p = self.packs[i]
        st = self.embed(self.models[k].handle, self.ids[i].data_ptr(), p.n_tokens, self.offs[i], p.n_texts,
                        self.outs[i].data_ptr(), self.streams[k].cuda_stream)
        if st != 0:
            self.B.check(st)

    def step(self, n_streams):
        for i in range(len(self.packs)):
            self.call(i, i % n_streams)

    def run_steps(self, n_steps):
        """n_steps steps on S streams, from one host thread per stream:
        thread k enqueues packs k, k + S, ... of every step on stream k (the
        library calls release the interpreter lock, so the launches are
        issued in parallel; from one thread, the ~200 launches of each of
        the 64 packs limit the step at ~1.44M tokens/s); with
        --one-host-thread from this thread."""
        S = self.S
        if not self.host_threads or S == 1:
            for _ in range(n_steps):
                self.step(S)
            return
        import threading
        errors = []

        def worker(k):
            try:
                for _ in range(n_steps):
                    for i in range(k, len(self.packs), S):
                        self.call(i, k)
            except Exception as e:  # reported on the main thread
                errors.append(e)

        threads = [threading.Thread(target=worker, args=(k,)) for k in range(S)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        if errors:
            raise errors[0]

    def timed(self, n_steps):
        """Host seconds of n_steps steps between two device synchronisations."""
        torch = self.torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.run_steps(n_steps)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def breakdown(self):
        """One untimed single-stream step with an event pair around every
        launch: per class ms, launches and work rate (work and peak kept
        under _work / _peak for group fractions, dropped from the output)."""
        B = self.B
        h = self.models[0].handle
        B.tte_profile_start(h, (1 << B.TTE_K_COUNT) - 1, (10 * self.cfg.layers + 4) * len(self.packs) + 16)
        self.step(1)
        prof = B.tte_profile_stop(h)
        work = class_work(self.cfg, self.packs)
        out = {}
        for k, (ms, n) in prof.items():
            if n == 0:
                continue
            entry = {"ms": round(ms, 3), "launches": int(n)}
            if k in work:
                amount, unit, peak = work[k]
                rate = amount / (ms / 1e3)
                if unit == "TFLOP/s":
                    entry["TFLOP/s"] = round(rate / 1e12, 1)
                    entry["frac_of_peak"] = round(rate / 1e12 / peak, 4)
                else:
                    entry["GB/s"] = round(rate / 1e9, 1)
                    entry["frac_of_hbm"] = round(rate / 1e9 / HBM_GBS, 4)
                    peak = HBM_GBS
                entry["_work"], entry["_peak"] = amount, peak
            out[k] = entry
        return out

    def roofline(self, group, n_steps):
        """n_steps single-stream steps with an event pair in the dispatch of
        every launch of the group's classes: its achieved rate against the
        peak of its bound, and the step time on one stream."""
        B, torch = self.B, self.torch
        classes = KERNEL_GROUPS[group]
        mask = 0
        for c in classes:
            mask |= 1 << B.KERNEL_CLASSES.index(c)
        h = self.models[0].handle
        B.tte_profile_start(h, mask, (len(classes) * self.cfg.layers + 4) * len(self.packs) * n_steps + 16)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n_steps):
            self.step(1)
        torch.cuda.synchronize()
        single_ms = (time.perf_counter() - t0) * 1e3 / n_steps
        prof = B.tte_profile_stop(h)
        work = class_work(self.cfg, self.packs)
        ms = sum(prof[c][0] for c in classes)
        n = sum(prof[c][1] for c in classes)
        amount = sum(work[c][0] for c in classes if c in work) * n_steps
        unit = work[classes[0]][1] if classes[0] in work else None
        if not ms or unit is None:
            return None, single_ms
        if unit == "TFLOP/s":
            achieved, peak, bound = amount / (ms / 1e3) / 1e12, work[classes[0]][2], "mfma"
            per = {"flops_per_launch_avg": int(amount / max(n, 1))}
        else:
            achieved, peak, bound, unit = amount / (ms / 1e3) / 1e9, HBM_GBS, "hbm", "GB/s"
            per = {"bytes_per_launch_avg": int(amount / max(n, 1))}
        return ({"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                 "frac": round(achieved / peak, 4), "traffic": None, "kernel": group, "classes": classes,
                 "launches": int(n), "avg_launch_us": round(ms * 1e3 / max(n, 1), 2), **per,
                 "measured_in": "single-stream pass, events in each launch's dispatch"}, single_ms)

    def close(self):
        for m in self.models:
            m.close()
        self.models = []


if __name__ == "__main__":
    main()
