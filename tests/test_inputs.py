"""The seeded input generator: determinism and the workload shapes."""
import numpy as np

import tte_inputs as ti


def test_fixed_length_workloads():
    p = ti.make_packs("tiny_fp32")
    assert len(p) == 1 and p[0].n_tokens == 178 and list(np.diff(p[0].offsets)) == [8, 40, 130]
    p = ti.make_packs("full_fp32_957")
    assert p[0].n_tokens == 957 and p[0].n_texts == 7
    p = ti.make_packs("full_bf16_4x4096")
    assert p[0].n_tokens == 16384 and p[0].n_texts == 4
    t = p[0].text(0)
    assert t[0] == ti.BOS and t[-1] == ti.EOS
    assert np.all(t[1:-1] >= ti.FIRST_ORDINARY_ID) and np.all(t[1:-1] < 102400)


def test_pack_streams():
    for name in ("full_bf16_packs2048", "full_int8_packs2048"):
        packs = ti.make_packs(name)
        assert len(packs) == 64
        for p in packs:
            lens = np.diff(p.offsets)
            assert p.n_tokens <= 2048 and np.all(lens >= 8) and np.all(lens <= 512)
        mean = np.mean([p.n_tokens for p in packs])
        assert 1700 < mean <= 2048


def test_determinism():
    a = ti.make_packs("full_bf16_packs2048")
    b = ti.make_packs("full_bf16_packs2048")
    for x, y in zip(a, b):
        assert np.array_equal(x.ids, y.ids) and np.array_equal(x.offsets, y.offsets)
    cfg = ti.workload("tiny_fp32")["cfg"]
    w1, w2 = ti.make_fp32_weights(cfg), ti.make_fp32_weights(cfg)
    assert np.array_equal(w1["tok_emb"], w2["tok_emb"])
    assert np.array_equal(w1["layers"][1]["wo2"], w2["layers"][1]["wo2"])


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38], np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties to even gives 1
    bits = ti.bf16_bits(x)
    back = ti.bf16_to_f32(bits)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.015625)
    assert back[3] == -2.5


def test_weight_blocks():
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.02, size=(6, 96)).astype(np.float32)
    w[2, 32:64] = 0
    q, s = ti.quantize_weight_blocks(w)
    assert q.shape == (6, 96) and s.shape == (6, 3)
    assert s[2, 1] == 0 and np.all(q[2, 32:64] == 0)
    assert np.all(np.abs(q) <= 127)
    err = np.abs(ti.dequant_blocks(q, s) - w)
    assert np.all(err <= np.repeat(s, 32, axis=1) * 0.5 + 1e-9)
