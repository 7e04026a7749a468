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
sample of the same workload on the host's cores.  The roofline comes from a
second timed pass of the same steps on a single stream with a HIP event pair
around every launch of the dominant kernel on that stream (with several
streams, kernels of different packs overlap and per-launch durations would
include the time they share the chip).  An untimed single-stream step with
event pairs around every launch adds the work rate of each kernel class
("kernels": TFLOP/s and fraction of peak for the GEMMs and attention, GB/s
for the row kernels).

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
    w["norm"] = (2 * Lyr * T * H * (4 + out_b), "GB/s", None)  # read fp32 rows, write the GEMM operand
    w["pool"] = (T * H * 4, "GB/s", None)
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
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {used} packs ({n} tokens) of the workload, fp64 numpy, {dt:.1f}s"}


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
    ap.add_argument("--cpu-sample-tokens", type=int, default=3000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time the steps without the per-launch events of the dominant kernel")
    ap.add_argument("--no-breakdown", dest="breakdown", action="store_false",
                    help="skip the untimed single-stream step that times every kernel class")
    ap.add_argument("--row-kernels", action="store_true",
                    help="only measure the row kernels' HBM rate (LayerNorm, 7-bit quantisation) at two shapes")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized fp32 buffer 5 times with torch (known bytes, for HBM counter scaling)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {a.gpus}).",
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
    spec = ti.workload(a.workload)
    cfg = spec["cfg"]
    t0 = time.perf_counter()
    w = ti.cached_storage_weights(cfg)
    packs = ti.make_packs(a.workload)
    cpu_packs = packs  # the CPU baseline always takes the workload's own packs
    if a.merged:
        # texts are independent: the whole step as one pack (one call)
        packs = [ti.pack_from_texts([p.text(b) for p in packs for b in range(p.n_texts)])]
        a.streams = 1
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s: {len(packs)} packs, "
        f"{sum(p.n_tokens for p in packs)} tokens")
    max_tokens = max(p.n_tokens for p in packs)
    S = max(1, a.streams)
    max_texts = max(1024, max(p.n_texts for p in packs))
    max_len = max(512, max(int(np.diff(p.offsets).max()) for p in packs))
    model = Model(cfg, w, max_tokens=max_tokens, max_text_len=max_len, max_texts=max_texts, device="cuda:0",
                  split_k=a.split_k, graph=a.graph)
    models = [model] + [Model(cfg, None, max_tokens=max_tokens, max_text_len=max_len, max_texts=max_texts,
                              device="cuda:0", shared_from=model, split_k=a.split_k, graph=a.graph)
                        for _ in range(S - 1)]
    streams = [torch.cuda.Stream(device=dev) for _ in range(S)]
    ids = [torch.from_numpy(p.ids).to(dev) for p in packs]
    per_token = a.output == "tokens"
    outs = [torch.empty((p.n_tokens if per_token else p.n_texts, cfg.hidden), dtype=torch.float32, device=dev)
            for p in packs]
    offs = [B.int32_array(p.offsets) for p in packs]
    L = B.lib()
    embed = L.tte_embed_tokens if per_token else L.tte_embed

    def step(n_streams):
        for i, p in enumerate(packs):
            k = i % n_streams
            st = embed(models[k].handle, ids[i].data_ptr(), p.n_tokens, offs[i], p.n_texts, outs[i].data_ptr(),
                       streams[k].cuda_stream)
            if st != 0:
                B.check(st)

    def run_steps(n_steps):
        """n_steps steps on S streams, from one host thread per stream:
        thread k enqueues packs k, k + S, ... of every step on stream k (the
        library calls release the interpreter lock, so the launches are
        issued in parallel; from one thread, the ~200 launches of each of
        the 64 packs limit the step at ~1.44M tokens/s); with
        --one-host-thread from this thread."""
        if not a.host_threads or S == 1:
            for _ in range(n_steps):
                step(S)
            return
        import threading
        errors = []

        def worker(k):
            try:
                for _ in range(n_steps):
                    for i in range(k, len(packs), S):
                        p = packs[i]
                        st = embed(models[k].handle, ids[i].data_ptr(), p.n_tokens, offs[i], p.n_texts,
                                   outs[i].data_ptr(), streams[k].cuda_stream)
                        if st != 0:
                            B.check(st)
            except Exception as e:  # reported on the main thread
                errors.append(e)

        threads = [threading.Thread(target=worker, args=(k,)) for k in range(S)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        if errors:
            raise errors[0]

    torch.cuda.synchronize()
    run_steps(a.warmup)
    torch.cuda.synchronize()
    log("warmup done")

    tokens_per_step = sum(p.n_tokens for p in packs)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(a.steps)
    torch.cuda.synchronize()
    secs = time.perf_counter() - t0
    value = tokens_per_step * a.steps / secs
    log(f"timed {a.steps} steps on {S} streams: {secs * 1e3:.2f} ms")

    # single-stream pass: per-launch events around the dominant kernel
    roofline = None
    H, I = cfg.hidden, cfg.intermediate
    dominant = "gemm_geglu"
    single_ms = None
    if not a.no_kernel_events:
        h = models[0].handle
        B.tte_profile_start(h, 1 << B.KERNEL_CLASSES.index(dominant), cfg.layers * len(packs) * a.steps + 16)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(a.steps):
            step(1)
        torch.cuda.synchronize()
        single_ms = (time.perf_counter() - t0) * 1e3 / a.steps
        prof = B.tte_profile_stop(h)
        ms_dom, n_dom = prof[dominant]
        flops = GEMM_CLASSES[dominant](H, I) * tokens_per_step * cfg.layers * a.steps
        achieved = flops / (ms_dom / 1e3) / 1e12
        peak = PEAK_TFLOPS[cfg.precision]
        traffic = None
        if a.workload == "full_bf16_packs2048" and not a.merged:  # the counters' launch shapes
            traffic = traffic_from_profile(
                os.path.join(ROOT, "transformer_text_embedding_amd", "csrc", "kernels_gemm.hip"),
                os.path.join(ROOT, "profiles", "traffic_gemm_geglu_full_bf16_packs2048.json"))
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": f"k_gemm ({dominant})",
                    "launches": int(n_dom), "avg_launch_us": round(ms_dom * 1e3 / max(n_dom, 1), 2),
                    "flops_per_launch_avg": int(flops / max(n_dom, 1)), "measured_in": "single-stream pass"}

    breakdown = None
    if a.breakdown:
        h = models[0].handle
        B.tte_profile_start(h, (1 << B.TTE_K_COUNT) - 1, (10 * cfg.layers + 4) * len(packs) + 16)
        step(1)
        prof = B.tte_profile_stop(h)
        breakdown = {}
        work = class_work(cfg, packs)
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
            breakdown[k] = entry

    torch.cuda.synchronize()
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(secs * 1e3 / a.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE[cfg.precision], "data": "synthetic",
        "config": {"workload": a.workload, "packs_per_step": len(cpu_packs), "tokens_per_step": tokens_per_step,
                   "pack_budget": spec.get("pack_budget"), "layers": cfg.layers, "hidden": cfg.hidden,
                   "heads": cfg.heads, "intermediate": cfg.intermediate, "calls_per_step": len(packs),
                   "streams": S, "hw_queues": int(os.environ.get("GPU_MAX_HW_QUEUES", "4")), "output": a.output,
                   "split_k": a.split_k, "graph": a.graph, "merged": a.merged, "host_threads": a.host_threads,
                   "single_stream_ms_per_step": round(single_ms, 3) if single_ms else None},
        "roofline": roofline,
    }
    if breakdown is not None:
        # one pack at a time: the residual products' tiles are sized for
        # packs on concurrent streams, so their lone rate here is low
        breakdown["measured_in"] = "untimed single-stream step"
        line["kernels"] = breakdown
    if not a.no_cpu_baseline:
        log("timing the CPU oracle sample")
        line["cpu_baseline"] = cpu_baseline(a.workload, cfg, w, cpu_packs, a.cpu_sample_tokens)
    for m in models:
        m.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
