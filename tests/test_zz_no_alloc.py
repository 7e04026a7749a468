"""tte_op_pool_static (the pooling entry point with its scratch in a static
device array) against tte_op_pool, through the C ABI: two calls in a row,
the second with a smaller pack, each bit-identical to tte_op_pool's output
and within the oracle's tolerance; and the size limit refused cleanly."""
import numpy as np
import pytest

import oracle
import tte_inputs as ti
from gpu_util import dev, empty, host, say, stream, torch
from transformer_text_embedding_amd import B, Model

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny_fp32", "full_bf16_packs2048"])
def test_pool_static_matches_pool(name):
    t = torch()
    cfg = ti.workload(name)["cfg"]
    H = cfg.hidden
    rng = np.random.default_rng(77)
    gamma = (1 + rng.normal(0, 0.1, size=H)).astype(np.float32)
    m = Model(cfg.as_dict(), _weights(cfg, gamma), max_tokens=8192, max_text_len=4096, max_texts=256)
    try:
        # two calls in a row, the second with a smaller pack
        for lengths in ([700, 1, 33, 2000, 64, 31, 96, 4096], [5, 40, 129]):
            T = sum(lengths)
            off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
            x = (rng.normal(size=(T, H)) * 2 + 0.3).astype(np.float32)
            dx = dev(x)
            a = empty((len(lengths), H), t.float32)
            b = empty((len(lengths), H), t.float32)
            say(f"  {name}: pool_static on T={T} B={len(lengths)}")
            B.tte_op_pool(m.handle, dx.data_ptr(), T, off, a.data_ptr(), stream())
            B.tte_op_pool_static(m.handle, dx.data_ptr(), T, off, b.data_ptr(), stream())
            ga, gb = host(a), host(b)
            assert np.array_equal(ga, gb)
            ref = oracle.mean_pool_l2(oracle.layer_norm(x, gamma, cfg.ln_eps), off)
            np.testing.assert_allclose(gb, ref, atol=2e-6, rtol=0)
    finally:
        m.close()


def _weights(cfg, gamma):
    w = ti.storage_weights(cfg) if cfg.hidden <= 128 else ti.cached_storage_weights(cfg)
    w = dict(w)
    w["final_norm"] = gamma
    return w


def test_pool_static_refuses_packs_beyond_its_scratch():
    t = torch()
    cfg = ti.workload("full_bf16_packs2048")["cfg"]
    m = Model(cfg.as_dict(), ti.cached_storage_weights(cfg), max_tokens=100000, max_text_len=100000, max_texts=4)
    try:
        T = 90000  # 2813 partial rows of 768 fp32: above 8 MiB
        off = np.array([0, T], np.int32)
        dx = t.zeros((T, cfg.hidden), dtype=t.float32, device="cuda:0")
        out = empty((1, cfg.hidden), t.float32)
        with pytest.raises(B.TteError) as e:
            B.tte_op_pool_static(m.handle, dx.data_ptr(), T, off, out.data_ptr(), stream())
        assert e.value.status == B.TTE_E_UNSUPPORTED and "scratch" in str(e.value)
        # a pack that fits still works after the refusal
        T2 = 64
        off2 = np.array([0, T2], np.int32)
        B.tte_op_pool_static(m.handle, dx.data_ptr(), T2, off2, out.data_ptr(), stream())
        host(out)
    finally:
        m.close()
