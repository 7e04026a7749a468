"""Oracle: a plain, slow CPU implementation of the packed embedding pass.

TEST INFRASTRUCTURE ONLY.  Tests, the smoke check and the bench's CPU-baseline
leg call this module; the product path never does.

It follows the tensai "テキスト埋め込み" page (mattn.github.io/tensai/ja/embeddings):

* section 何が動くか, encoder paragraph: 25 layers, each a bias-free
  LayerNorm, 12-head attention with RoPE, and a GeGLU feed-forward; the first
  layer and every third layer after it attend over the whole text with RoPE
  base 160000, the others see only the 64 tokens on either side with base
  10000;
* section 何が動くか, pooling paragraph: the last layer's output is averaged
  over the text and scaled to length 1;
* section 何が動くか, packing paragraph: texts are processed together, with
  positions counted from zero in every text and attention kept inside each
  text, so a packed batch gives the same vectors as one text at a time;
* section 精度と量子化: the integer matmul rounds the activations of every
  row to 7 bits with a single scale per row, while the stored weight blocks
  are used unchanged.

Where the page leaves a step open, the reading taken is the ModernBERT layout
the page names (the model is a ModernBERT and matches transformers' output):
an embedding LayerNorm, pre-norm sub-layers whose attention norm is absent on
layer 0, a final LayerNorm before pooling, rotate-half RoPE with
theta_c = base^(-2c/d), the erf form of GELU with the first half of the
up-projection activated and the second half the gate, a fused QKV weight laid
out [Q; K; V] with heads contiguous, scale 1/sqrt(d), the window bound
|i - j| <= 64 inclusive, and mean pooling over every token of the text
(BOS/EOS included).

Arithmetic is fp64 (numpy).  In the int8 mode, the one place where floating
point decides an integer -- the 7-bit activation code -- is decided in fp32,
the precision the kernel uses.  Parity pins: every function here is checked in
the CPU test suite against closed forms, invariants, brute force or an
independent library (torch functional ops, transformers' ModernBERT).
"""
from __future__ import annotations

import math
from typing import List, Optional

import numpy as np
from numpy.lib.stride_tricks import sliding_window_view
from scipy.special import erf


# --------------------------------------------------------------------------
# pack bookkeeping (packing paragraph)
# --------------------------------------------------------------------------

def validate_offsets(offsets, n_tokens: int, max_text_len: Optional[int] = None) -> np.ndarray:
    """Offsets are B+1 exclusive prefix sums: 0 first, strictly increasing
    (no empty text), last equal to the token count."""
    off = np.asarray(offsets, dtype=np.int64)
    if off.ndim != 1 or len(off) < 2:
        raise ValueError("offsets must hold at least two entries")
    if off[0] != 0:
        raise ValueError("offsets[0] must be 0")
    if np.any(np.diff(off) <= 0):
        raise ValueError("offsets must be strictly increasing")
    if off[-1] != n_tokens:
        raise ValueError("offsets[-1] must equal the number of tokens")
    if max_text_len is not None and np.max(np.diff(off)) > max_text_len:
        raise ValueError("a text is longer than max_text_len")
    return off


def text_index(offsets) -> np.ndarray:
    """b(t): the text that token t belongs to."""
    off = np.asarray(offsets, dtype=np.int64)
    return np.repeat(np.arange(len(off) - 1), np.diff(off))


def positions(offsets) -> np.ndarray:
    """pos[t] = t - offsets[b(t)]: positions restart at 0 in every text."""
    off = np.asarray(offsets, dtype=np.int64)
    t = np.arange(off[-1])
    return t - off[text_index(off)]


# --------------------------------------------------------------------------
# building blocks
# --------------------------------------------------------------------------

def layer_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """Bias-free LayerNorm over the last axis: (x - mean) / sqrt(var + eps) * gamma,
    with the biased (1/H) variance and no additive term."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(gamma, dtype=np.float64)


def gelu(z: np.ndarray) -> np.ndarray:
    """GELU, erf form: z * Phi(z) = 0.5 * z * (1 + erf(z / sqrt(2)))."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def geglu(u: np.ndarray) -> np.ndarray:
    """GeGLU: split the up-projection in two halves [a | g]; GELU(a) * g."""
    half = u.shape[-1] // 2
    return gelu(u[..., :half]) * u[..., half:]


def rope_inverse_frequencies(base: float, d: int) -> np.ndarray:
    """theta_c = base^(-2c/d) for c = 0 .. d/2 - 1."""
    c = np.arange(d // 2, dtype=np.float64)
    return base ** (-2.0 * c / d)


def rope(u: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half RoPE on the last axis (size d): the pair (u_c, u_{c+d/2})
    is rotated by the angle pos * theta_c."""
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[:, None] * rope_inverse_frequencies(base, d)[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    if u.ndim == 3:  # [n, heads, d]
        cos, sin = cos[:, None, :], sin[:, None, :]
    a, b = u[..., : d // 2], u[..., d // 2:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def _window_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, window: int, scale: float) -> np.ndarray:
    """One text, one head, local layer: row i attends to keys i-window ..
    i+window that exist in the text.  Key rows are read through a sliding
    window view of the zero-padded K and V, so row i holds exactly its own
    2*window+1 candidate keys; candidates outside the text get -inf."""
    n, d = q.shape
    pad = np.zeros((window, d))
    kw = sliding_window_view(np.concatenate([pad, k, pad]), (2 * window + 1, d))[:, 0]  # [n, 2w+1, d]
    vw = sliding_window_view(np.concatenate([pad, v, pad]), (2 * window + 1, d))[:, 0]
    s = np.einsum("nd,nwd->nw", q, kw) * scale
    j = np.arange(n)[:, None] + np.arange(-window, window + 1)[None, :]
    s = np.where((j >= 0) & (j < n), s, -np.inf)
    return np.einsum("nw,nwd->nd", _softmax_rows(s), vw)


def attention(qkv: np.ndarray, offsets, n_heads: int, head_dim: int, is_global: bool,
              window: int, rope_base: float) -> np.ndarray:
    """Attention of one layer over a pack.

    qkv is [T, 3*H] laid out [Q | K | V], head j at columns j*d .. j*d+d-1 of
    each block.  RoPE (positions restarting per text) is applied to Q and K.
    Each text attends only to itself; on a local layer token i also needs
    |i - j| <= window.  Scores are q.k / sqrt(d), softmax over the allowed keys.
    Returns O [T, H] with head j at columns j*d .. j*d+d-1.
    """
    qkv = np.asarray(qkv, dtype=np.float64)
    T = qkv.shape[0]
    H = n_heads * head_dim
    off = np.asarray(offsets, dtype=np.int64)
    q = qkv[:, :H].reshape(T, n_heads, head_dim)
    k = qkv[:, H:2 * H].reshape(T, n_heads, head_dim)
    v = qkv[:, 2 * H:].reshape(T, n_heads, head_dim)
    pos = positions(off)
    q = rope(q, pos, rope_base)
    k = rope(k, pos, rope_base)
    out = np.zeros((T, n_heads, head_dim))
    scale = 1.0 / math.sqrt(head_dim)
    for b in range(len(off) - 1):
        lo, hi = off[b], off[b + 1]
        for h in range(n_heads):
            qt, kt, vt = q[lo:hi, h, :], k[lo:hi, h, :], v[lo:hi, h, :]
            if is_global:
                out[lo:hi, h, :] = _softmax_rows((qt @ kt.T) * scale) @ vt
            else:
                out[lo:hi, h, :] = _window_attention(qt, kt, vt, window, scale)
    return out.reshape(T, H)


def mean_pool_l2(x: np.ndarray, offsets) -> np.ndarray:
    """Per text: mean of its rows (every token, BOS and EOS included), then
    divided by max(||e||_2, 1e-12) so every vector has length 1."""
    x = np.asarray(x, dtype=np.float64)
    off = np.asarray(offsets, dtype=np.int64)
    e = np.stack([x[off[b]:off[b + 1]].mean(axis=0) for b in range(len(off) - 1)])
    return e / np.maximum(np.linalg.norm(e, axis=1, keepdims=True), 1e-12)


def cosine_matrix(e: np.ndarray) -> np.ndarray:
    """Cosine similarities of unit vectors: their dot products."""
    e = np.asarray(e, dtype=np.float64)
    return e @ e.T


# --------------------------------------------------------------------------
# integer path (section 精度と量子化)
# --------------------------------------------------------------------------

def quantize_rows_7bit(x: np.ndarray):
    """Per-row 7-bit activation codes, decided in fp32.

    amax = max |x| over the row; inv = 63 / amax; q = clamp(rint(x * inv), -63, 63)
    with ties to even; scale s = amax / 63 (every operation rounded to fp32).
    A row of zeros gives q = 0 and s = 0.  Returns (q int8 [M,K], s fp32 [M]).
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(x32), axis=1).astype(np.float32)
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1.0)).astype(np.float32)
    inv = (np.float32(63.0) / safe).astype(np.float32)
    q = np.rint((x32 * inv[:, None]).astype(np.float32))
    q = np.clip(q, -63, 63)
    q = np.where(nz[:, None], q, 0).astype(np.int8)
    s = np.where(nz, (amax / np.float32(63.0)).astype(np.float32), np.float32(0.0)).astype(np.float32)
    return q, s


def block_matmul_int8(qx: np.ndarray, sx: np.ndarray, qw: np.ndarray, sw: np.ndarray,
                      block: int = 32) -> np.ndarray:
    """y[m,n] = sx[m] * sum_b sw[n,b] * sum_{k in block b} qx[m,k] * qw[n,k].

    Evaluated in fp64 as sx * (qx @ (qw * sw)^T): each product of an int8, an
    int8 and an fp32 scale is exact in fp64, so this is the definition up to
    fp64 summation order.
    """
    N, K = qw.shape
    wdeq = (qw.astype(np.float64).reshape(N, K // block, block)
            * np.asarray(sw, np.float64)[:, :, None]).reshape(N, K)
    return np.asarray(sx, np.float64)[:, None] * (qx.astype(np.float64) @ wdeq.T)


def q4_codes(codes: np.ndarray) -> np.ndarray:
    """4-bit codes [N, K] from their packed bytes [N, K/2] (two per byte, the
    even input in the low nibble)."""
    c = np.asarray(codes, np.uint8)
    q = np.empty((c.shape[0], 2 * c.shape[1]), np.int64)
    q[:, 0::2] = c & 15
    q[:, 1::2] = c >> 4
    return q


def q4_block_params(meta: np.ndarray):
    """Per 32-input block of a 4-bit matrix: its scale es = fp32(d * sc) and
    offset eo = fp32(dmin * mn).  meta is uint8 [N, K/128, 16]: per 128
    inputs the four blocks' 6-bit sc and mn (a byte each), then the fp32 d
    and dmin of their 256-input super-block.  Returns (es, eo) fp32
    [N, K/32]."""
    m = np.ascontiguousarray(meta, np.uint8)
    N, G, _ = m.shape
    sc = m[:, :, 0:4].astype(np.float32).reshape(N, 4 * G)
    mn = m[:, :, 4:8].astype(np.float32).reshape(N, 4 * G)
    d = np.ascontiguousarray(m[:, :, 8:12]).view("<f4").reshape(N, G)
    dmin = np.ascontiguousarray(m[:, :, 12:16]).view("<f4").reshape(N, G)
    es = (np.repeat(d, 4, axis=1) * sc).astype(np.float32)
    eo = (np.repeat(dmin, 4, axis=1) * mn).astype(np.float32)
    return es, eo


def block_matmul_q4(qx: np.ndarray, sx: np.ndarray, codes: np.ndarray, meta: np.ndarray,
                    block: int = 32) -> np.ndarray:
    """The -q4 integer product (section 精度と量子化): 7-bit activation codes
    against 4-bit weight codes, per block b
        y[m,n] = sx[m] * sum_b (es[n,b] * P[m,n,b] - eo[n,b] * S[m,b]),
    P = sum_{k in b} qx[m,k] q[n,k] and S = sum_{k in b} qx[m,k].
    Evaluated in fp64 as sx * (qx @ W^T) with W = es * q - eo (each term
    exact in fp64), i.e. the definition up to fp64 summation order."""
    q = q4_codes(codes)
    N, K = q.shape
    es, eo = q4_block_params(meta)
    wdeq = (q.astype(np.float64).reshape(N, K // block, block) * es.astype(np.float64)[:, :, None]
            - eo.astype(np.float64)[:, :, None]).reshape(N, K)
    return np.asarray(sx, np.float64)[:, None] * (qx.astype(np.float64) @ wdeq.T)


# --------------------------------------------------------------------------
# weights in their storage formats
# --------------------------------------------------------------------------

def decode_matrix(w: dict, name: str, precision: str) -> np.ndarray:
    """The fp64 values of a stored matrix.  bf16 values are the upper 16 bits
    of an fp32; int8 blocks are q * s with one fp32 scale per 32 inputs."""
    if precision == "fp32":
        return np.asarray(w[name], dtype=np.float64)
    if precision == "bf16":
        bits = np.asarray(w[name + "_bf16"], dtype=np.uint16)
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if precision == "int8":
        q, s = w[name + "_q"], w[name + "_s"]
        N, K = q.shape
        return (q.astype(np.float64).reshape(N, K // 32, 32)
                * np.asarray(s, np.float64)[:, :, None]).reshape(N, K)
    if precision == "int4":
        if name == "tok_emb":  # the token table stays in int8 blocks
            return decode_matrix(w, name, "int8")
        q = q4_codes(w[name + "_q4"])
        N, K = q.shape
        es, eo = q4_block_params(w[name + "_q4m"])
        return (q.astype(np.float64).reshape(N, K // 32, 32) * es.astype(np.float64)[:, :, None]
                - eo.astype(np.float64)[:, :, None]).reshape(N, K)
    raise ValueError(precision)


def _project(x: np.ndarray, layer: dict, name: str, precision: str) -> np.ndarray:
    """x @ W^T for one stored weight.  In int8 and int4 modes x is first
    rounded per row to 7 bits and the block-scaled integer product is
    taken."""
    if precision == "int8":
        qx, sx = quantize_rows_7bit(x)
        return block_matmul_int8(qx, sx, layer[name + "_q"], layer[name + "_s"])
    if precision == "int4":
        qx, sx = quantize_rows_7bit(x)
        return block_matmul_q4(qx, sx, layer[name + "_q4"], layer[name + "_q4m"])
    return np.asarray(x, np.float64) @ decode_matrix(layer, name, precision).T


# --------------------------------------------------------------------------
# the whole pass
# --------------------------------------------------------------------------

def encoder_layer(cfg: dict, w: dict, l: int, x: np.ndarray, offsets) -> np.ndarray:
    """Layer l applied to the residual stream x [T, H] of a pack (section
    何が動くか, encoder paragraph): pre-norm attention (no norm on layer 0;
    global with RoPE base 160000 when l is a multiple of global_every, else
    the +-window local form with base 10000), its output projection added
    to x; then pre-norm GeGLU feed-forward added to x."""
    H, nh, d = cfg["hidden"], cfg["heads"], cfg["head_dim"]
    prec = cfg["precision"]
    off = np.asarray(offsets, dtype=np.int64)
    x = np.asarray(x, dtype=np.float64)
    layer = w["layers"][l]
    is_global = (l % cfg["global_every"]) == 0
    base = cfg["rope_base_global"] if is_global else cfg["rope_base_local"]
    a = x if l == 0 else layer_norm(x, layer["attn_norm"], cfg["ln_eps"])
    qkv = _project(a, layer, "wqkv", prec)
    o = attention(qkv, off, nh, d, is_global, cfg["window"], base)
    x = x + _project(o, layer, "wo", prec)
    m = layer_norm(x, layer["mlp_norm"], cfg["ln_eps"])
    y = geglu(_project(m, layer, "wi", prec))
    return x + _project(y, layer, "wo2", prec)


def encode_layers(cfg: dict, w: dict, ids, offsets, n_layers: Optional[int] = None) -> List[np.ndarray]:
    """Hidden states of the residual stream: after the embedding LayerNorm and
    after each layer (fp64 [T, H] each).  n_layers limits the depth."""
    prec = cfg["precision"]
    ids = np.asarray(ids, dtype=np.int64)
    off = validate_offsets(offsets, len(ids))
    if np.any(ids < 0) or np.any(ids >= cfg["vocab"]):
        raise ValueError("token id out of range")
    emb = decode_matrix(w, "tok_emb", prec)
    x = layer_norm(emb[ids], w["emb_norm"], cfg["ln_eps"])
    states = [x]
    L = cfg["layers"] if n_layers is None else n_layers
    for l in range(L):
        x = encoder_layer(cfg, w, l, x, off)
        states.append(x)
    return states


def encode_tokens(cfg: dict, w: dict, ids, offsets) -> np.ndarray:
    """Per-token output states [T, H]: the layers and the final LayerNorm,
    before any pooling (the encoder's own per-token output, which the
    pooling paragraph of section 何が動くか then averages)."""
    x = encode_layers(cfg, w, ids, offsets)[-1]
    return layer_norm(x, w["final_norm"], cfg["ln_eps"])


def encode(cfg: dict, w: dict, ids, offsets) -> np.ndarray:
    """Unit-norm embeddings [B, H] of the texts of a pack: the per-token
    states, mean pooling per text and L2 normalisation."""
    return mean_pool_l2(encode_tokens(cfg, w, ids, offsets), offsets)
