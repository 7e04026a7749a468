"""The parity tolerances, checked on the CPU (no GPU, no HIP library):

* bf16 attention: the per-element bound derived from the kernel's bf16
  roundings holds for a NumPy replay of exactly those roundings, is far
  tighter than the values' scale, and is exceeded by planted mistakes
  (a window one position short, K without RoPE);
* integer paths: rounding the oracle's intermediates to fp32 -- a change of
  at most half an fp32 ulp per value -- moves the 7-bit pass's vectors by
  1 - cos of order 1e-4 .. 1e-3 (the codes amplify it), while the fp32 pass
  moves by ~1e-13; the stored full-size spreads back the end-to-end gate
  min cos >= 0.998 of the int8 and 4-bit paths.
"""
import os

import numpy as np
import pytest

import oracle
import tte_inputs as ti
from parity_bounds import (attention_bf16_bound, attention_bf16_emulated, cos_rows, encode_layers_bf16_emulated,
                           encode_layers_fp32_rounded, pooled_spread, rounding_spread)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _qkv(lengths, layer, heads):
    rng = np.random.default_rng(sum(lengths) + layer)
    T, H = sum(lengths), 64 * heads
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    qkv = (rng.normal(size=(T, 3 * H)) * 1.5).astype(np.float32)
    return ti.bf16_to_f32(ti.bf16_bits(qkv)).astype(np.float64), off


@pytest.mark.parametrize("lengths,layer,heads", [([8, 40, 130], 0, 12), ([8, 40, 130], 1, 12),
                                                 ([1, 64, 65, 200, 3, 129], 1, 4), ([957], 0, 2)])
def test_attention_bf16_bound_holds_for_the_kernels_roundings(lengths, layer, heads):
    qv, off = _qkv(lengths, layer, heads)
    g = layer % 3 == 0
    base = 160000.0 if g else 10000.0
    ref = oracle.attention(qv, off, heads, 64, g, 64, base)
    emu = attention_bf16_emulated(qv, off, heads, 64, g, 64, base)
    bound, sd = attention_bf16_bound(qv, off, heads, 64, g, 64, base)
    err = np.abs(emu - ref)
    assert np.all(err <= bound), (err / bound).max()
    # informative: the bound is a small fraction of the outputs' scale
    assert bound.mean() < 0.025 and bound.mean() < 0.1 * np.abs(ref).mean()
    assert err.mean() > 0.1 * bound.mean() / 6  # the emulation really rounds


def test_attention_bf16_bound_catches_planted_mistakes():
    lengths, heads = [8, 40, 130], 4
    for layer, mistake in ((1, "window"), (1, "no_rope_k"), (0, "no_rope_k")):
        qv, off = _qkv(lengths, layer, heads)
        g = layer % 3 == 0
        base = 160000.0 if g else 10000.0
        bound, _ = attention_bf16_bound(qv, off, heads, 64, g, 64, base)
        if mistake == "window":
            wrong = attention_bf16_emulated(qv, off, heads, 64, g, 63, base)
        else:
            # K columns un-rotated: undo the rotation the emulation applies
            H = 64 * heads
            pos = oracle.positions(off)
            k = qv[:, H:2 * H].reshape(len(qv), heads, 64)
            k_inv = oracle.rope(k, -pos, base).reshape(len(qv), H)
            wrong = attention_bf16_emulated(np.concatenate([qv[:, :H], k_inv, qv[:, 2 * H:]], axis=1),
                                            off, heads, 64, g, 64, base)
        ref = oracle.attention(qv, off, heads, 64, g, 64, base)
        assert np.any(np.abs(wrong - ref) > bound), mistake


def _subpack(name, pack_index, texts):
    pack = ti.make_packs(name)[pack_index]
    return ti.pack_from_texts([pack.text(b) for b in texts])


def _decoded_fp32(cfg, w):
    """The same model in fp32: every stored int8 matrix decoded (q * s)."""
    out = {k: v for k, v in w.items() if k != "layers" and not k.startswith("tok_emb")}
    out["tok_emb"] = oracle.decode_matrix(w, "tok_emb", "int8").astype(np.float32)
    out["layers"] = []
    for L in w["layers"]:
        d = {k: v for k, v in L.items() if k.endswith("norm")}
        for name in ("wqkv", "wo", "wi", "wo2"):
            d[name] = oracle.decode_matrix(L, name, "int8").astype(np.float32)
        out["layers"].append(d)
    return out


def test_fp32_rounding_is_amplified_by_the_7bit_codes_at_full_size():
    """Seven texts (492 tokens) of the full-size int8 workload's first pack,
    25 layers: 1 - cos between the oracle's pass and its fp32-rounded twin
    rises layer after layer into the range the end-to-end gate allows for;
    the same weights run in fp32 (no 7-bit codes) barely move."""
    cfg = ti.workload("full_int8_packs2048")["cfg"]
    w = ti.cached_storage_weights(cfg)
    pack = _subpack("full_int8_packs2048", 0, range(3, 10))
    a = oracle.encode_layers(cfg.as_dict(), w, pack.ids, pack.offsets)
    b = encode_layers_fp32_rounded(cfg.as_dict(), w, pack.ids, pack.offsets)
    spread = np.array([1 - cos_rows(x, y).min() for x, y in zip(a, b)])
    assert spread[0] < 1e-12  # the embedding norm has no 7-bit codes ahead of it
    assert spread[-1] > 1e-5 and spread[-1] > 10 * spread[1]
    assert spread[-1] < 2e-2
    cfg32 = ti.EncoderConfig(**{**cfg.as_dict(), "precision": "fp32"})
    w32 = _decoded_fp32(cfg, w)
    _, _, fin32, _ = rounding_spread(cfg32.as_dict(), w32, pack.ids, pack.offsets)
    assert fin32 < 1e-10
    assert spread[-1] > 1e4 * fin32


@pytest.mark.parametrize("name", ["full_int8_packs2048", "full_int4_packs2048"])
def test_stored_spreads_back_the_integer_gate(name):
    """tests/golden/rounding_spread.npz (written by make_oracle_golden.py
    from the oracle alone): over a whole ~1.9k-token pack the fp32-rounded
    pass ends at pooled 1 - cos of order 1e-3, so the end-to-end gate
    (min cos >= 0.998, mean >= 0.999) allows about twice what rounding
    alone produces, and no more."""
    z = np.load(os.path.join(GOLDEN, "rounding_spread.npz"), allow_pickle=False)
    fin_min, fin_mean = z[f"{name}_pack0_final"]
    per_min = z[f"{name}_pack0_min"]
    assert len(per_min) == 26
    assert 3e-4 < fin_min < 1.3e-3 and fin_mean < 1e-3
    assert 1 - 0.998 >= 1.5 * fin_min and 1 - 0.999 >= 1.5 * fin_mean
    # the spread only grows with depth (up to small wiggles)
    assert np.all(np.diff(per_min[1:]) > -0.1 * per_min[1:-1])


def test_bf16_stream_rounding_sits_well_inside_the_bf16_gate():
    """Three texts (491 tokens) of the full-size bf16 workload's first pack,
    25 layers, on the CPU: the kernels' bf16 operand roundings with the
    residual stream also held in bf16 end at pooled 1 - cos of order 1e-4
    at most, a tenth of what the end-to-end gate (min cos >= 0.999) allows;
    holding the stream in bf16 really moves the result (several times the
    spread of the operand roundings alone)."""
    cfg = ti.workload("full_bf16_packs2048")["cfg"]
    w = ti.cached_storage_weights(cfg)
    pack = _subpack("full_bf16_packs2048", 0, range(3))
    c = cfg.as_dict()
    ops_only = pooled_spread(c, w, pack.ids, pack.offsets,
                             encode_layers_bf16_emulated(c, w, pack.ids, pack.offsets, stream_bf16=False))
    stream = pooled_spread(c, w, pack.ids, pack.offsets, encode_layers_bf16_emulated(c, w, pack.ids, pack.offsets))
    print(f"bf16 operands: 1 - cos min {ops_only[0]:.2e} mean {ops_only[1]:.2e}; "
          f"+ bf16 stream: {stream[0]:.2e} / {stream[1]:.2e}")
    assert stream[0] < 0.1 * (1 - 0.999)
    assert stream[0] > 2 * ops_only[0]
