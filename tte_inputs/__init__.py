"""Seeded synthetic inputs for the packed text-embedding encoder.

This module is shared data, not method: it draws weights, token ids and pack
layouts from fixed seeds, and converts weights into the storage formats the
encoder reads (fp32, bf16 bit patterns, int8 blocks with fp32 scales).  None of
the encoder's arithmetic (norms, projections, attention, pooling, activation
quantisation) lives here; the oracle and the HIP library each implement that
on their own.

Workload shapes follow the tensai "テキスト埋め込み" page: a 25-layer, 12-head
ModernBERT encoder (section 何が動くか, encoder paragraph), texts packed up to
about 2048 tokens with positions restarting per text (same section, packing
paragraph), and 7 texts of 8 to 382 tokens for the accuracy comparison
(section 精度と量子化).  Dimensions the page does not give (hidden 768,
intermediate 3072, vocab 102400) are the stated full-size dims.
"""
from __future__ import annotations

import dataclasses
import math
import os
from typing import Dict, List, Optional

import numpy as np

BOS = 1
EOS = 2
FIRST_ORDINARY_ID = 4


@dataclasses.dataclass(frozen=True)
class EncoderConfig:
    name: str
    vocab: int
    hidden: int
    heads: int
    head_dim: int
    intermediate: int
    layers: int
    precision: str  # "fp32" | "bf16" | "int8" | "int4"
    seed: int
    global_every: int = 3
    window: int = 64
    rope_base_global: float = 160000.0
    rope_base_local: float = 10000.0
    ln_eps: float = 1e-5
    init_std: float = 0.02

    def as_dict(self) -> dict:
        return dataclasses.asdict(self)


TINY = dict(vocab=1000, hidden=128, heads=2, head_dim=64, intermediate=256, layers=2)
FULL = dict(vocab=102400, hidden=768, heads=12, head_dim=64, intermediate=3072, layers=25)

# The five workloads.  Text lengths include the BOS/EOS wrappers, so the
# 3-text tiny pack is 8 + 40 + 130 = 178 tokens and the 7-text pack is 957.
WORKLOADS = {
    "tiny_fp32": dict(cfg=EncoderConfig("tiny_fp32", precision="fp32", seed=0, **TINY),
                      lengths=[8, 40, 130]),
    "full_fp32_957": dict(cfg=EncoderConfig("full_fp32_957", precision="fp32", seed=1, **FULL),
                          lengths=[8, 24, 57, 96, 150, 240, 382]),
    "full_bf16_packs2048": dict(cfg=EncoderConfig("full_bf16_packs2048", precision="bf16", seed=2, **FULL),
                                n_packs=64, pack_budget=2048, len_lo=8, len_hi=512),
    "full_bf16_4x4096": dict(cfg=EncoderConfig("full_bf16_4x4096", precision="bf16", seed=3, **FULL),
                             lengths=[4096, 4096, 4096, 4096]),
    "full_int8_packs2048": dict(cfg=EncoderConfig("full_int8_packs2048", precision="int8", seed=4, **FULL),
                                n_packs=64, pack_budget=2048, len_lo=8, len_hi=512),
    # the 4-bit weight path (the page's -q4): same packs as the int8 one
    "full_int4_packs2048": dict(cfg=EncoderConfig("full_int4_packs2048", precision="int4", seed=5, **FULL),
                                n_packs=64, pack_budget=2048, len_lo=8, len_hi=512),
}
# A small config whose widths hold whole 256-input super-blocks (the 4-bit
# format needs K % 256 == 0, which the tiny config's hidden 128 is not).
SMALL_Q4 = dict(vocab=1000, hidden=256, heads=4, head_dim=64, intermediate=512, layers=3)
WORKLOAD_ORDER = list(WORKLOADS)


def workload(name: str) -> dict:
    return WORKLOADS[name]


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------

def matrix_shapes(cfg: EncoderConfig) -> Dict[str, tuple]:
    H, I = cfg.hidden, cfg.intermediate
    return {"wqkv": (3 * H, H), "wo": (H, H), "wi": (2 * I, H), "wo2": (H, I)}


def make_fp32_weights(cfg: EncoderConfig) -> dict:
    """fp32 master weights, drawn N(0, init_std) in fp64 and cast to fp32.

    Draw order: token embedding, then per layer Wqkv, Wo, Wi, Wo2.  Every
    LayerNorm gain is 1 (the standard init; only matrices are drawn).
    Matrices are [out, in] row-major, so each projection is x @ W.T.
    """
    rng = np.random.default_rng([cfg.seed, 0])
    H = cfg.hidden

    def draw(shape):
        return rng.normal(0.0, cfg.init_std, size=shape).astype(np.float32)

    w = {"tok_emb": draw((cfg.vocab, H)), "emb_norm": np.ones(H, np.float32),
         "final_norm": np.ones(H, np.float32), "layers": []}
    shapes = matrix_shapes(cfg)
    for l in range(cfg.layers):
        layer = {name: draw(shape) for name, shape in shapes.items()}
        layer["attn_norm"] = None if l == 0 else np.ones(H, np.float32)
        layer["mlp_norm"] = np.ones(H, np.float32)
        w["layers"].append(layer)
    return w


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def quantize_weight_blocks(w: np.ndarray, block: int = 32):
    """Storage format of the int8 model: per row, per `block` consecutive
    input elements, one fp32 scale s = amax/127 and codes
    q = clamp(rint(w/s), -127, 127) (ties to even); an all-zero block stores
    s = 0 and q = 0.  Returns (q int8 [N,K], s fp32 [N,K/block])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % block == 0
    wb = w.reshape(N, K // block, block)
    amax = np.abs(wb).max(axis=2)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint(wb / safe[:, :, None]).astype(np.float32)
    q = np.clip(q, -127, 127)
    q = np.where(s[:, :, None] > 0, q, 0).astype(np.int8)
    return q.reshape(N, K), s


def quantize_weight_q4(w: np.ndarray):
    """Storage format of the 4-bit model, in the style of the Q4_K blocks the
    page's -q4 repacks (asymmetric 4-bit codes, two-level scales):

    per row, per 32 inputs (a block): codes q in [0, 15]; per 256 inputs (a
    super-block of 8 blocks): fp32 d and dmin, and per block 6-bit indices
    sc, mn in [0, 63].  The block's scale is es = fp32(d * sc), its offset
    eo = fp32(dmin * mn), and the weight w = es * q - eo.

    Construction: a block's range [min(lo, 0), hi] gives a = (hi - lo') / 15
    and m = -lo'; d = max a / 63 and dmin = max m / 63 over the super-block;
    sc = rint(a / d), mn = rint(m / dmin) (0 when d or dmin is 0); then
    q = clamp(rint((w + eo) / es), 0, 15) (0 when es = 0).

    Returns (codes uint8 [N, K/2], two per byte, the even input in the low
    nibble; meta uint8 [N, K/128, 16]: per 128 inputs sc[4], mn[4] (one byte
    each), then d and dmin of their super-block as fp32)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % 256 == 0
    nb = K // 32
    wb = w.reshape(N, nb, 32)
    lo = np.minimum(wb.min(axis=2), np.float32(0))
    hi = wb.max(axis=2)
    a = ((hi - lo) / np.float32(15)).astype(np.float32)
    m = (-lo).astype(np.float32)
    sa, sm = a.reshape(N, nb // 8, 8), m.reshape(N, nb // 8, 8)
    d = (sa.max(axis=2) / np.float32(63)).astype(np.float32)
    dmin = (sm.max(axis=2) / np.float32(63)).astype(np.float32)
    sd = np.where(d > 0, d, np.float32(1))[:, :, None]
    sdm = np.where(dmin > 0, dmin, np.float32(1))[:, :, None]
    sc = np.where(d[:, :, None] > 0, np.clip(np.rint(sa / sd), 0, 63), 0).astype(np.uint8)
    mn = np.where(dmin[:, :, None] > 0, np.clip(np.rint(sm / sdm), 0, 63), 0).astype(np.uint8)
    es = (d[:, :, None] * sc.astype(np.float32)).astype(np.float32).reshape(N, nb)
    eo = (dmin[:, :, None] * mn.astype(np.float32)).astype(np.float32).reshape(N, nb)
    safe = np.where(es > 0, es, np.float32(1))[:, :, None]
    q = np.where(es[:, :, None] > 0, np.clip(np.rint((wb + eo[:, :, None]) / safe), 0, 15), 0)
    q = q.astype(np.uint8).reshape(N, K)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    meta = np.zeros((N, K // 128, 16), np.uint8)
    sc2, mn2 = sc.reshape(N, K // 128, 4), mn.reshape(N, K // 128, 4)
    meta[:, :, 0:4] = sc2
    meta[:, :, 4:8] = mn2
    d2 = np.repeat(d, 2, axis=1)  # each super-block spans two 128-input groups
    dm2 = np.repeat(dmin, 2, axis=1)
    meta[:, :, 8:12] = d2.astype("<f4").view(np.uint8).reshape(N, K // 128, 4)
    meta[:, :, 12:16] = dm2.astype("<f4").view(np.uint8).reshape(N, K // 128, 4)
    return codes, meta


def dequant_blocks(q: np.ndarray, s: np.ndarray, block: int = 32) -> np.ndarray:
    """fp64 values of a block-quantised matrix (exact: int8 times fp32 fits fp64)."""
    N, K = q.shape
    return (q.astype(np.float64).reshape(N, K // block, block) * s.astype(np.float64)[:, :, None]).reshape(N, K)


def storage_weights(cfg: EncoderConfig, w32: Optional[dict] = None) -> dict:
    """Weights in the storage format of cfg.precision.

    fp32: the fp32 arrays.  bf16: every matrix (embedding included) as uint16
    bf16 bits (key suffix _bf16).  int8: every matrix as (q int8, s fp32)
    blocks of 32 along the input dimension (suffixes _q, _s).  int4: the
    layer matrices as quantize_weight_q4 (suffixes _q4, _q4m), the token
    table as int8 blocks.  LayerNorm gains stay fp32 in every format.
    """
    if w32 is None:
        w32 = make_fp32_weights(cfg)
    mats = ["wqkv", "wo", "wi", "wo2"]
    out = {"emb_norm": w32["emb_norm"], "final_norm": w32["final_norm"], "layers": [],
           "precision": cfg.precision}
    if cfg.precision == "fp32":
        out["tok_emb"] = w32["tok_emb"]
        for L in w32["layers"]:
            out["layers"].append({k: L[k] for k in mats + ["attn_norm", "mlp_norm"]})
    elif cfg.precision == "bf16":
        out["tok_emb_bf16"] = bf16_bits(w32["tok_emb"])
        for L in w32["layers"]:
            d = {k + "_bf16": bf16_bits(L[k]) for k in mats}
            d["attn_norm"], d["mlp_norm"] = L["attn_norm"], L["mlp_norm"]
            out["layers"].append(d)
    elif cfg.precision == "int8":
        out["tok_emb_q"], out["tok_emb_s"] = quantize_weight_blocks(w32["tok_emb"])
        for L in w32["layers"]:
            d = {}
            for k in mats:
                d[k + "_q"], d[k + "_s"] = quantize_weight_blocks(L[k])
            d["attn_norm"], d["mlp_norm"] = L["attn_norm"], L["mlp_norm"]
            out["layers"].append(d)
    elif cfg.precision == "int4":
        # the layer matrices in 4-bit blocks; the token table in the int8
        # blocks (the page's Q4_K_M file keeps some tensors at more bits)
        out["tok_emb_q"], out["tok_emb_s"] = quantize_weight_blocks(w32["tok_emb"])
        for L in w32["layers"]:
            d = {}
            for k in mats:
                d[k + "_q4"], d[k + "_q4m"] = quantize_weight_q4(L[k])
            d["attn_norm"], d["mlp_norm"] = L["attn_norm"], L["mlp_norm"]
            out["layers"].append(d)
    else:
        raise ValueError(cfg.precision)
    return out


_CACHE_DIR = os.environ.get("TTE_INPUT_CACHE", "/tmp/tte_inputs_cache")


def cached_storage_weights(cfg: EncoderConfig) -> dict:
    """storage_weights(cfg), memoised on disk as .npy files (allow_pickle=False).

    Full-size weights take several seconds to draw; the cache is keyed by the
    workload name and seed, and is regenerated if absent."""
    key = f"{cfg.name}_s{cfg.seed}_v{cfg.vocab}_h{cfg.hidden}_l{cfg.layers}_{cfg.precision}"
    d = os.path.join(_CACHE_DIR, key)
    names = _flat_names(cfg)
    if all(os.path.exists(os.path.join(d, n + ".npy")) for n in names):
        try:
            flat = {n: np.load(os.path.join(d, n + ".npy"), allow_pickle=False) for n in names}
            return _unflatten(cfg, flat)
        except Exception:
            pass
    w = storage_weights(cfg)
    try:
        os.makedirs(d, exist_ok=True)
        for n, a in _flatten(w).items():
            tmp = os.path.join(d, f".{n}.{os.getpid()}.npy")
            np.save(tmp, a, allow_pickle=False)
            os.replace(tmp, os.path.join(d, n + ".npy"))
    except OSError:
        pass
    return w


def _flat_names(cfg: EncoderConfig) -> List[str]:
    mats = ["wqkv", "wo", "wi", "wo2"]
    suf = {"fp32": [""], "bf16": ["_bf16"], "int8": ["_q", "_s"], "int4": ["_q4", "_q4m"]}[cfg.precision]
    emb_suf = ["_q", "_s"] if cfg.precision == "int4" else suf
    names = ["emb_norm", "final_norm"] + ["tok_emb" + s for s in emb_suf]
    for l in range(cfg.layers):
        names += [f"l{l}_{m}{s}" for m in mats for s in suf]
        names += [f"l{l}_mlp_norm"] + ([f"l{l}_attn_norm"] if l > 0 else [])
    return names


def _flatten(w: dict) -> Dict[str, np.ndarray]:
    flat = {k: v for k, v in w.items() if isinstance(v, np.ndarray)}
    for l, L in enumerate(w["layers"]):
        for k, v in L.items():
            if v is not None:
                flat[f"l{l}_{k}"] = v
    return flat


def _unflatten(cfg: EncoderConfig, flat: Dict[str, np.ndarray]) -> dict:
    w = {"precision": cfg.precision, "layers": []}
    for k, v in flat.items():
        if not k.startswith("l") or k[1] not in "0123456789":
            w[k] = v
    for l in range(cfg.layers):
        pre = f"l{l}_"
        L = {k[len(pre):]: v for k, v in flat.items() if k.startswith(pre)}
        L.setdefault("attn_norm", None)
        w["layers"].append(L)
    return w


# --------------------------------------------------------------------------
# token ids and packs
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Pack:
    ids: np.ndarray      # int32 [T], texts concatenated
    offsets: np.ndarray  # int32 [B+1], offsets[0] = 0, offsets[B] = T

    @property
    def n_tokens(self) -> int:
        return int(self.offsets[-1])

    @property
    def n_texts(self) -> int:
        return len(self.offsets) - 1

    def text(self, b: int) -> np.ndarray:
        return self.ids[self.offsets[b]:self.offsets[b + 1]]


def text_ids(rng: np.random.Generator, n: int, vocab: int) -> np.ndarray:
    """One text of n tokens: BOS, n-2 ids uniform in [4, vocab), EOS
    (a 1-token text is BOS alone)."""
    assert n >= 1
    if n == 1:
        return np.array([BOS], np.int32)
    mid = rng.integers(FIRST_ORDINARY_ID, vocab, size=n - 2)
    return np.concatenate([[BOS], mid, [EOS]]).astype(np.int32)


def pack_from_texts(texts: List[np.ndarray]) -> Pack:
    lens = [len(t) for t in texts]
    offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ids = np.concatenate(texts).astype(np.int32) if texts else np.zeros(0, np.int32)
    return Pack(ids=ids, offsets=offsets)


def make_packs(name: str) -> List[Pack]:
    """The packs of a workload, from rng = default_rng([seed, 1]).

    Fixed-length workloads give one pack.  Pack-stream workloads draw text
    lengths round(exp(U(ln lo, ln hi))) one at a time and pack greedily: a pack
    is closed when the next text would push it past the budget; drawing stops
    once n_packs packs are closed."""
    spec = WORKLOADS[name]
    cfg = spec["cfg"]
    rng = np.random.default_rng([cfg.seed, 1])
    if "lengths" in spec:
        return [pack_from_texts([text_ids(rng, n, cfg.vocab) for n in spec["lengths"]])]
    packs, cur, cur_len = [], [], 0
    lo, hi = math.log(spec["len_lo"]), math.log(spec["len_hi"])
    while len(packs) < spec["n_packs"]:
        n = int(round(math.exp(rng.uniform(lo, hi))))
        if cur and cur_len + n > spec["pack_budget"]:
            packs.append(pack_from_texts(cur))
            cur, cur_len = [], 0
            if len(packs) == spec["n_packs"]:
                break
        cur.append(text_ids(rng, n, cfg.vocab))
        cur_len += n
    return packs


def random_pack(rng: np.random.Generator, lengths: List[int], vocab: int) -> Pack:
    return pack_from_texts([text_ids(rng, n, vocab) for n in lengths])
