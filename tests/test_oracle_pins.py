"""Pins for the CPU oracle: each check ties an oracle function to something
other than itself -- a closed form, an invariant, brute force on a tiny input,
an independent library routine (torch functional ops, transformers'
ModernBERT), or a value the tensai "テキスト埋め込み" page prints.

A plausible mistake in the oracle (a dropped term, a wrong sign or index, a
transposed operand, the wrong RoPE pairing or GeGLU half, an off-by-one in the
window) fails at least one of these.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import tte_inputs as ti

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny_cfg(precision="fp32"):
    spec = ti.workload("tiny_fp32")["cfg"]
    d = spec.as_dict()
    d["precision"] = precision
    return d


# --------------------------------------------------------------------------
# LayerNorm
# --------------------------------------------------------------------------

def test_layer_norm_closed_form():
    rng = np.random.default_rng(10)
    x = rng.normal(3.0, 2.0, size=(37, 128))
    y = oracle.layer_norm(x, np.ones(128), 1e-5)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-12)
    # with gain 1 the output variance is var / (var + eps)
    np.testing.assert_allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-12)


def test_layer_norm_matches_torch_functional():
    rng = np.random.default_rng(11)
    x = rng.normal(size=(19, 96)) * 5
    g = 1 + rng.normal(0, 0.02, size=96)
    ref = F.layer_norm(torch.from_numpy(x), (96,), weight=torch.from_numpy(g), bias=None, eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.layer_norm(x, g, 1e-5), ref, rtol=1e-12, atol=1e-12)


def test_layer_norm_has_no_bias_term():
    # a constant row normalises to exactly zero whatever the gain: no beta
    y = oracle.layer_norm(np.full((2, 64), 7.0), np.linspace(0.5, 2, 64), 1e-5)
    assert np.all(y == 0)


# --------------------------------------------------------------------------
# GELU / GeGLU
# --------------------------------------------------------------------------

def _golden_phi():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "normal_cdf.txt")) if l.strip() and not l.startswith("#")]
    return np.array([[float(a), float(b)] for a, b in rows])


def test_gelu_is_x_times_normal_cdf():
    tab = _golden_phi()
    np.testing.assert_allclose(oracle.gelu(tab[:, 0]), tab[:, 0] * tab[:, 1], rtol=1e-14, atol=1e-16)


def test_gelu_matches_torch_exact_gelu_not_tanh():
    z = np.linspace(-6, 6, 1001)
    ref = F.gelu(torch.from_numpy(z), approximate="none").numpy()
    np.testing.assert_allclose(oracle.gelu(z), ref, rtol=1e-13, atol=1e-15)
    tanh_form = F.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    assert np.max(np.abs(oracle.gelu(z) - tanh_form)) > 1e-4


def test_geglu_first_half_activated_second_half_gates():
    a = np.array([[1.0, -2.0, 0.5]])
    g = np.array([[3.0, 5.0, -1.0]])
    out = oracle.geglu(np.concatenate([a, g], axis=1))
    np.testing.assert_allclose(out, a * _golden_phi_at(a) * g, rtol=1e-12)
    # a zero gate kills the output whatever the activated half holds
    assert np.all(oracle.geglu(np.concatenate([a, np.zeros_like(g)], axis=1)) == 0)


def _golden_phi_at(a):
    tab = dict((round(x, 6), p) for x, p in _golden_phi())
    out = np.empty_like(a)
    for idx, v in np.ndenumerate(a):
        if round(v, 6) in tab:
            out[idx] = tab[round(v, 6)]
        else:
            out[idx] = 0.5 * (1 + math.erf(v / math.sqrt(2)))
    return out


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------

def test_rope_position_zero_is_identity_and_norm_preserved():
    rng = np.random.default_rng(12)
    u = rng.normal(size=(50, 64))
    pos = np.arange(50)
    r = oracle.rope(u, pos, 10000.0)
    np.testing.assert_allclose(r[0], u[0], rtol=0, atol=0)
    np.testing.assert_allclose(np.linalg.norm(r, axis=1), np.linalg.norm(u, axis=1), rtol=1e-13)


def test_rope_depends_only_on_relative_position():
    rng = np.random.default_rng(13)
    q, k = rng.normal(size=(1, 64)), rng.normal(size=(1, 64))
    for base in (10000.0, 160000.0):
        dots = []
        for p, r in [(3, 10), (103, 110), (4000, 4007)]:
            dots.append(float((oracle.rope(q, np.array([p]), base) @ oracle.rope(k, np.array([r]), base).T)[0, 0]))
        np.testing.assert_allclose(dots, dots[0], rtol=1e-9)


def test_rope_rotate_half_equals_complex_rotation():
    # independent formulation: z_c = u_c + i u_{c+32}, rotated by exp(i p base^(-c/32))
    rng = np.random.default_rng(14)
    u = rng.normal(size=(9, 64))
    pos = np.array([0, 1, 2, 7, 64, 65, 500, 2047, 4095])
    for base in (10000.0, 160000.0):
        z = u[:, :32] + 1j * u[:, 32:]
        theta = np.array([base ** (-c / 32.0) for c in range(32)])
        zr = z * np.exp(1j * pos[:, None] * theta[None, :])
        ref = np.concatenate([zr.real, zr.imag], axis=1)
        np.testing.assert_allclose(oracle.rope(u, pos, base), ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# attention and masks
# --------------------------------------------------------------------------

def _complex_rope(u, pos, base):
    d = u.shape[-1]
    z = u[..., : d // 2] + 1j * u[..., d // 2:]
    theta = base ** (-np.arange(d // 2) / (d // 2))
    zr = z * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    return np.concatenate([zr.real, zr.imag], axis=-1)


def _dense_attention_sdpa(qkv, offsets, nh, d, is_global, window, base):
    """Brute force over the whole pack: a dense T x T boolean mask
    (same text and, on local layers, |pos_i - pos_j| <= window) fed to torch's
    scaled_dot_product_attention in fp64; RoPE by complex rotation."""
    T = qkv.shape[0]
    H = nh * d
    off = np.asarray(offsets)
    tid = np.searchsorted(off, np.arange(T), side="right") - 1
    pos = np.arange(T) - off[tid]
    q = _complex_rope(qkv[:, :H].reshape(T, nh, d), pos, base)
    k = _complex_rope(qkv[:, H:2 * H].reshape(T, nh, d), pos, base)
    v = qkv[:, 2 * H:].reshape(T, nh, d)
    mask = tid[:, None] == tid[None, :]
    if not is_global:
        mask &= np.abs(np.arange(T)[:, None] - np.arange(T)[None, :]) <= window
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).permute(1, 0, 2)
    tv = torch.from_numpy(v).permute(1, 0, 2)
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask))
    return o.permute(1, 0, 2).reshape(T, H).numpy()


@pytest.mark.parametrize("is_global", [True, False])
@pytest.mark.parametrize("sharpen", [1.0, 10.0])
def test_attention_matches_dense_mask_brute_force(is_global, sharpen):
    rng = np.random.default_rng(15)
    lengths = [5, 70, 130, 1, 64]
    off = np.concatenate([[0], np.cumsum(lengths)])
    T, nh, d = off[-1], 2, 64
    qkv = rng.normal(size=(T, 3 * nh * d)) * sharpen
    for base in (10000.0, 160000.0):
        got = oracle.attention(qkv, off, nh, d, is_global, 64, base)
        ref = _dense_attention_sdpa(qkv, off, nh, d, is_global, 64, base)
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


def test_local_equals_global_up_to_65_tokens_and_differs_beyond():
    rng = np.random.default_rng(16)
    nh, d = 2, 64
    for n in (1, 8, 64, 65):
        qkv = rng.normal(size=(n, 3 * nh * d)) * 3
        off = [0, n]
        a = oracle.attention(qkv, off, nh, d, True, 64, 10000.0)
        b = oracle.attention(qkv, off, nh, d, False, 64, 10000.0)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    qkv = rng.normal(size=(66, 3 * nh * d)) * 0.3
    a = oracle.attention(qkv, [0, 66], nh, d, True, 64, 10000.0)
    b = oracle.attention(qkv, [0, 66], nh, d, False, 64, 10000.0)
    # only the first and last rows lose a key at 66 tokens
    diff = np.abs(a - b).max(axis=1)
    assert diff[0] > 1e-6 and diff[65] > 1e-6 and np.all(diff[1:65] < 1e-13)


def test_attention_packed_equals_alone_and_permutes():
    rng = np.random.default_rng(17)
    nh, d = 2, 64
    lengths = [9, 100, 33]
    texts = [rng.normal(size=(n, 3 * nh * d)) for n in lengths]
    off = np.concatenate([[0], np.cumsum(lengths)])
    for g in (True, False):
        packed = oracle.attention(np.concatenate(texts), off, nh, d, g, 64, 160000.0)
        for b, t in enumerate(texts):
            alone = oracle.attention(t, [0, len(t)], nh, d, g, 64, 160000.0)
            np.testing.assert_allclose(packed[off[b]:off[b + 1]], alone, rtol=0, atol=1e-14)
        perm = [2, 0, 1]
        off_p = np.concatenate([[0], np.cumsum([lengths[i] for i in perm])])
        packed_p = oracle.attention(np.concatenate([texts[i] for i in perm]), off_p, nh, d, g, 64, 160000.0)
        for j, i in enumerate(perm):
            np.testing.assert_allclose(packed_p[off_p[j]:off_p[j + 1]], packed[off[i]:off[i + 1]], atol=1e-14)


def test_offsets_validation():
    with pytest.raises(ValueError):
        oracle.validate_offsets([1, 3], 3)
    with pytest.raises(ValueError):
        oracle.validate_offsets([0, 2, 2, 5], 5)
    with pytest.raises(ValueError):
        oracle.validate_offsets([0, 4], 5)
    with pytest.raises(ValueError):
        oracle.validate_offsets([0, 3, 9], 9, max_text_len=5)
    assert list(oracle.positions([0, 3, 5])) == [0, 1, 2, 0, 1]
    assert list(oracle.text_index([0, 3, 5])) == [0, 0, 0, 1, 1]


# --------------------------------------------------------------------------
# pooling and normalisation
# --------------------------------------------------------------------------

def test_pool_unit_norm_and_identical_rows():
    rng = np.random.default_rng(18)
    x = rng.normal(size=(20, 32))
    e = oracle.mean_pool_l2(x, [0, 3, 20])
    np.testing.assert_allclose(np.linalg.norm(e, axis=1), 1.0, rtol=1e-15)
    row = rng.normal(size=32)
    e2 = oracle.mean_pool_l2(np.tile(row, (7, 1)), [0, 7])
    np.testing.assert_allclose(e2[0], row / np.linalg.norm(row), rtol=1e-14)
    # every token counts, the first and last ones included
    x3 = np.zeros((4, 2))
    x3[0] = [4.0, 0.0]
    x3[3] = [0.0, 4.0]
    np.testing.assert_allclose(oracle.mean_pool_l2(x3, [0, 4])[0], [math.sqrt(0.5)] * 2, rtol=1e-15)


def test_cosine_matrix_structure_matches_printed_example():
    printed = np.loadtxt(os.path.join(GOLDEN, "tensai_sim_matrix.txt"))
    # the printed matrix: symmetric, unit diagonal, entries below 1
    np.testing.assert_array_equal(printed, printed.T)
    np.testing.assert_array_equal(np.diag(printed), 1.0)
    assert np.all(printed[~np.eye(5, dtype=bool)] < 1.0)
    # the oracle's vectors give the same structure
    rng = np.random.default_rng(19)
    e = oracle.mean_pool_l2(rng.normal(size=(40, 16)), [0, 4, 9, 20, 33, 40])
    c = oracle.cosine_matrix(e)
    np.testing.assert_allclose(c, c.T, atol=1e-15)
    np.testing.assert_allclose(np.diag(c), 1.0, atol=1e-15)
    assert np.all(np.abs(c[~np.eye(5, dtype=bool)]) < 1.0)


# --------------------------------------------------------------------------
# 7-bit activations and the block-scaled integer product
# --------------------------------------------------------------------------

def test_quantize_rows_closed_form_ties_to_even():
    x = np.array([[63.0, 0.5, 1.5, 2.5, -0.5, -2.5, -63.0, 31.49]])
    q, s = oracle.quantize_rows_7bit(x)
    assert s[0] == np.float32(1.0)
    assert list(q[0]) == [63, 0, 2, 2, 0, -2, -63, 31]


def test_quantize_rows_properties():
    rng = np.random.default_rng(20)
    x = rng.normal(size=(64, 768)).astype(np.float32) * rng.uniform(0.01, 100, size=(64, 1)).astype(np.float32)
    x[5] = 0.0
    q, s = oracle.quantize_rows_7bit(x)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert np.all(np.abs(q) <= 63)
    assert s[5] == 0 and np.all(q[5] == 0)
    rows = [r for r in range(64) if r != 5]
    amax_idx = np.argmax(np.abs(x[rows]), axis=1)
    assert np.all(np.abs(q[rows, amax_idx]) == 63)
    err = np.abs(x[rows].astype(np.float64) - s[rows, None].astype(np.float64) * q[rows])
    assert np.all(err <= s[rows, None] * (0.5 + 1e-5))


def test_block_matmul_matches_int64_brute_force():
    rng = np.random.default_rng(21)
    M, N, K = 7, 5, 96
    qx = rng.integers(-63, 64, size=(M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    sx = rng.uniform(0.001, 0.1, size=M).astype(np.float32)
    sw = rng.uniform(0.001, 0.1, size=(N, K // 32)).astype(np.float32)
    ref = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for b in range(K // 32):
                p = int(sum(int(qx[m, k]) * int(qw[n, k]) for k in range(32 * b, 32 * b + 32)))
                acc += float(sw[n, b]) * p
            ref[m, n] = float(sx[m]) * acc
    np.testing.assert_allclose(oracle.block_matmul_int8(qx, sx, qw, sw), ref, rtol=1e-13)


# --------------------------------------------------------------------------
# the whole pass
# --------------------------------------------------------------------------

def _tiny_inputs():
    spec = ti.workload("tiny_fp32")
    cfg = spec["cfg"]
    w32 = ti.make_fp32_weights(cfg)
    pack = ti.make_packs("tiny_fp32")[0]
    return cfg, w32, pack


def test_encode_matches_transformers_modernbert():
    """transformers' ModernBERT (the architecture the page names; tensai is
    compared against it) with the same weights, fp64, one text at a time."""
    from transformers import ModernBertConfig, ModernBertModel
    import transformers
    transformers.logging.set_verbosity_error()
    cfg, w32, pack = _tiny_inputs()
    hf_cfg = ModernBertConfig(
        vocab_size=cfg.vocab, hidden_size=cfg.hidden, intermediate_size=cfg.intermediate,
        num_hidden_layers=3, num_attention_heads=cfg.heads, global_attn_every_n_layers=3,
        local_attention=2 * cfg.window, global_rope_theta=cfg.rope_base_global,
        local_rope_theta=cfg.rope_base_local, norm_eps=cfg.ln_eps, norm_bias=False,
        attention_bias=False, mlp_bias=False, hidden_activation="gelu",
        max_position_embeddings=8192, pad_token_id=0, bos_token_id=1, eos_token_id=2,
        cls_token_id=1, sep_token_id=2)
    hf_cfg._attn_implementation = "eager"
    # three layers (global, local, local) so the local base and window both show
    rng = np.random.default_rng(22)
    layers = w32["layers"] + [{k: (None if v is None else rng.normal(0, 0.02, size=v.shape).astype(np.float32))
                               for k, v in w32["layers"][1].items()}]
    layers[2]["attn_norm"] = (1 + rng.normal(0, 0.1, size=cfg.hidden)).astype(np.float32)
    layers[2]["mlp_norm"] = (1 + rng.normal(0, 0.1, size=cfg.hidden)).astype(np.float32)
    w = dict(w32, layers=layers)
    w["emb_norm"] = (1 + rng.normal(0, 0.1, size=cfg.hidden)).astype(np.float32)
    w["final_norm"] = (1 + rng.normal(0, 0.1, size=cfg.hidden)).astype(np.float32)
    model = ModernBertModel(hf_cfg).double().eval()
    sd = {"embeddings.tok_embeddings.weight": w["tok_emb"], "embeddings.norm.weight": w["emb_norm"],
          "final_norm.weight": w["final_norm"]}
    for l, L in enumerate(layers):
        if l > 0:
            sd[f"layers.{l}.attn_norm.weight"] = L["attn_norm"]
        sd[f"layers.{l}.attn.Wqkv.weight"] = L["wqkv"]
        sd[f"layers.{l}.attn.Wo.weight"] = L["wo"]
        sd[f"layers.{l}.mlp_norm.weight"] = L["mlp_norm"]
        sd[f"layers.{l}.mlp.Wi.weight"] = L["wi"]
        sd[f"layers.{l}.mlp.Wo.weight"] = L["wo2"]
    model.load_state_dict({k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in sd.items()}, strict=True)
    ocfg = dict(cfg.as_dict(), layers=3)
    # weights scaled up so that attention is sharp and mask errors show
    for L in layers:
        L["wqkv"] = L["wqkv"] * 8
    model.load_state_dict({f"layers.{l}.attn.Wqkv.weight": torch.from_numpy(np.asarray(L["wqkv"], np.float64))
                           for l, L in enumerate(layers)}, strict=False)
    emb = oracle.encode(ocfg, w, pack.ids, pack.offsets)
    for b in range(pack.n_texts):
        ids = torch.from_numpy(pack.text(b).astype(np.int64))[None]
        with torch.no_grad():
            hs = model(input_ids=ids, attention_mask=torch.ones_like(ids)).last_hidden_state[0].numpy()
        e = hs.mean(axis=0)
        e = e / np.linalg.norm(e)
        # transformers forms the RoPE angles in fp32 (its rotary module casts
        # the inverse frequencies to float), which alone moves the result by
        # ~1e-8; a structural mistake (RoPE pairing, GeGLU half, norm
        # placement, window bound, QKV layout) moves it by more than 1e-3.
        np.testing.assert_allclose(emb[b], e, rtol=0, atol=1e-7)
        # the per-token states agree too (before pooling)
        own = oracle.encode_tokens(ocfg, w, pack.text(b), [0, pack.offsets[b + 1] - pack.offsets[b]])
        np.testing.assert_allclose(own, hs, rtol=0, atol=2e-5)


def test_encode_packed_equals_alone_unit_norm():
    cfg, w32, pack = _tiny_inputs()
    c = cfg.as_dict()
    emb = oracle.encode(c, w32, pack.ids, pack.offsets)
    np.testing.assert_allclose(np.linalg.norm(emb, axis=1), 1.0, rtol=1e-14)
    for b in range(pack.n_texts):
        t = pack.text(b)
        alone = oracle.encode(c, w32, t, [0, len(t)])
        np.testing.assert_allclose(emb[b], alone[0], rtol=0, atol=1e-13)


def test_encode_int8_and_bf16_storage_stay_close_to_fp32():
    cfg, w32, pack = _tiny_inputs()
    ref = oracle.encode(cfg.as_dict(), w32, pack.ids, pack.offsets)
    for prec in ("bf16", "int8"):
        c = dict(cfg.as_dict(), precision=prec)
        w = ti.storage_weights(ti.EncoderConfig(**{**cfg.as_dict(), "precision": prec}), w32)
        e = oracle.encode(c, w, pack.ids, pack.offsets)
        cos = np.sum(e * ref, axis=1)
        assert np.all(cos > 0.999), (prec, cos)
        assert np.all(cos < 1 - 1e-9), (prec, cos)  # the formats really differ


def test_encode_rejects_bad_ids():
    cfg, w32, pack = _tiny_inputs()
    with pytest.raises(ValueError):
        oracle.encode(cfg.as_dict(), w32, np.array([1, 5000, 2]), [0, 3])


# --------------------------------------------------------------------------
# the 4-bit weight path (section 精度と量子化, -q4)
# --------------------------------------------------------------------------

def test_q4_decode_hand_computed():
    """One 128-input group, values worked by hand: w = d*sc*q - dmin*mn."""
    import struct
    codes = np.zeros((1, 128), np.uint8)
    codes[0, 0] = 0x21            # inputs 0, 1: q = 1, 2
    codes[0, 16] = 0xF0           # inputs 32, 33 (block 1): q = 0, 15
    meta = np.zeros((1, 2, 16), np.uint8)  # K = 256: two groups of 128
    for g in range(2):
        meta[0, g, 0:4] = [3, 1, 0, 63]    # sc of blocks 0..3
        meta[0, g, 4:8] = [5, 2, 0, 1]     # mn
        meta[0, g, 8:16] = np.frombuffer(struct.pack("<ff", 0.5, 0.25), np.uint8)
    w = oracle.decode_matrix({"m_q4": codes, "m_q4m": meta}, "m", "int4")
    assert w.shape == (1, 256)
    assert w[0, 0] == 0.5 * 3 * 1 - 0.25 * 5 == 0.25
    assert w[0, 1] == 0.5 * 3 * 2 - 1.25 == 1.75
    assert w[0, 2] == -1.25                 # q = 0 in block 0
    assert w[0, 32] == -0.5 and w[0, 33] == 0.5 * 1 * 15 - 0.5 == 7.0
    assert w[0, 64] == 0.0                  # sc = mn = 0
    assert w[0, 96] == -0.25                # block 3: q = 0, offset 0.25
    assert w[0, 128] == -1.25               # second group: same metadata, codes 0


def test_q4_quantizer_rounds_to_the_nearest_code():
    """Quantising N(0, 0.02) weights: every unclipped weight decodes to
    within half a step es/2 of itself, and clipping is rare."""
    rng = np.random.default_rng(7)
    w = rng.normal(0, 0.02, size=(64, 512)).astype(np.float32)
    codes, meta = ti.quantize_weight_q4(w)
    back = oracle.decode_matrix({"m_q4": codes, "m_q4m": meta}, "m", "int4")
    es, eo = oracle.q4_block_params(meta)
    step = np.repeat(es.astype(np.float64), 32, axis=1)
    q = oracle.q4_codes(codes)
    err = np.abs(back - w)
    inside = (q > 0) & (q < 15)
    assert np.all(err[inside] <= step[inside] / 2 * (1 + 1e-6))
    assert np.mean(err <= step / 2 * (1 + 1e-6)) > 0.99
    cos = np.sum(back * w) / np.linalg.norm(back) / np.linalg.norm(w)
    assert cos > 0.99


def test_block_matmul_q4_exact_block_sums():
    """The product against its definition with integer block sums P and S
    and exact rational arithmetic (Fraction of every fp32 scale)."""
    from fractions import Fraction
    rng = np.random.default_rng(9)
    M, N, K = 3, 4, 256
    x = rng.normal(size=(M, K)).astype(np.float32)
    qx, sx = oracle.quantize_rows_7bit(x)
    codes, meta = ti.quantize_weight_q4(rng.normal(0, 0.05, size=(N, K)).astype(np.float32))
    q = oracle.q4_codes(codes)
    es, eo = oracle.q4_block_params(meta)
    got = oracle.block_matmul_q4(qx, sx, codes, meta)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for b in range(K // 32):
                ks = slice(32 * b, 32 * b + 32)
                P = int(np.dot(qx[m, ks].astype(np.int64), q[n, ks]))
                S = int(qx[m, ks].astype(np.int64).sum())
                tot += Fraction(float(es[n, b])) * P - Fraction(float(eo[n, b])) * S
            exact = float(Fraction(float(sx[m])) * tot)
            assert abs(got[m, n] - exact) <= 1e-12 * max(1.0, abs(exact))


def test_encode_int4_stays_close_to_fp32():
    """The whole pass with 4-bit layer weights keeps every text's direction
    (quantisation noise only)."""
    base = ti.EncoderConfig("small_q4", precision="fp32", seed=3, **ti.SMALL_Q4)
    w32 = ti.make_fp32_weights(base)
    q4 = ti.EncoderConfig("small_q4", precision="int4", seed=3, **ti.SMALL_Q4)
    w4 = ti.storage_weights(q4, w32)
    pack = ti.random_pack(np.random.default_rng(1), [5, 40, 90], base.vocab)
    e32 = oracle.encode(base.as_dict(), ti.storage_weights(base, w32), pack.ids, pack.offsets)
    e4 = oracle.encode(q4.as_dict(), w4, pack.ids, pack.offsets)
    cos = np.sum(e32 * e4, axis=1)
    assert cos.min() > 0.95, cos
