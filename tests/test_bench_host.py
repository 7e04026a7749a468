"""Host-side logic of bench.py (no GPU): the algorithmic work it divides by."""
import importlib.util
import os

import numpy as np

import tte_inputs as ti

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _brute_pairs(lengths, window):
    g = loc = 0
    for L in lengths:
        i, j = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
        g += L * L
        loc += int(np.sum(np.abs(i - j) <= window))
    return g, loc


def test_allowed_pairs_brute_force():
    b = _bench()
    for lengths in ([8, 40, 130], [1], [65, 66, 200], [957], [3, 4096]):
        assert b.allowed_pairs(lengths, 64) == _brute_pairs(lengths, 64)
        # text lengths as the packs hold them (int32 offsets)
        assert b.allowed_pairs(np.array(lengths, np.int32), 64) == _brute_pairs(lengths, 64)


def test_class_work_no_int32_overflow_on_the_full_workload():
    b = _bench()
    cfg = ti.workload("full_bf16_packs2048")["cfg"]
    packs = ti.make_packs("full_bf16_packs2048")
    w = b.class_work(cfg, packs)
    g = sum(_brute_pairs([int(x) for x in np.diff(p.offsets)], 64)[0] for p in packs[:2])
    assert g > 0 and w["attn_global"][0] > 2 ** 31 and w["attn_local"][0] > 2 ** 31


def test_class_work_gemm_flops_per_token():
    """471.86 MFLOP of weight products per token at full size."""
    b = _bench()
    cfg = ti.workload("full_bf16_packs2048")["cfg"]
    pack = ti.random_pack(np.random.default_rng(0), [10, 20], cfg.vocab)
    w = b.class_work(cfg, [pack])
    gemm = sum(w[k][0] for k in b.GEMM_CLASSES)
    assert gemm / pack.n_tokens == 2 * 25 * (3 * 768 * 768 + 768 * 768 + 2 * 3072 * 768 + 768 * 3072)
    assert abs(gemm / pack.n_tokens / 1e6 - 471.86) < 0.01
    # attention: 9 global layers of 25, 4 * 64 * 12 flops per pair and layer
    g, loc = _brute_pairs([10, 20], 64)
    assert w["attn_global"][0] == g * 3072 * 9 and w["attn_local"][0] == loc * 3072 * 16


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: asked for more it exits with status 2 and a
    message, before anything touches a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU" in r.stderr and r.stdout == ""
