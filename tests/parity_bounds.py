"""Tolerances of the parity tests, derived from the arithmetic rather than
fitted to results.

bf16 attention (tensai "テキスト埋め込み" page, section 何が動くか: each token
attends to its own text, on local layers within 64 positions).  The kernel
rounds to bf16 (ties to even, unit roundoff u = 2^-8) at three places: Q and
K after RoPE, the softmax numerators P, and the output O; it accumulates in
fp32.  V arrives in bf16 and is used as it is, so it carries no new error.
The oracle keeps fp64 after reading the same bf16 Q, K, V.  With w_ij the
exact softmax weights and O_i = sum_j w_ij v_j:

* a rounding error e of a value x is modelled as uniform in +-ulp/2, which
  is at most u |x|: variance <= (u x)^2 / 3, independent between values;
* a score error ds_ij moves the output by sum_j w_ij (ds_ij - mean) v_j =
  sum_j w_ij ds_ij (v_j - O_i) (the weights stay normalised);
  - Q errors: ds_ij = (1/8) sum_d dq_id k_jd, shared by every key j of query
    i: variance (1/64) sum_d (u q_id)^2/3 * C_idd'^2 with
    C_idd' = sum_j w_ij k_jd (v_jd' - O_id');
  - K errors: (1/8) sum_d q_id dk_jd, independent over j and d: variance
    (u^2/192) sum_j w_ij^2 (v_jd' - O_id')^2 sum_d q_id^2 k_jd^2;
* P errors: P_j (1 + eta_j) (P taken against any reference max: the
  rounding is relative), and the kernel divides by the sum of the same
  rounded P, so O moves by sum_j w_ij eta_j (v_j - O_i): variance
  (u^2/3) sum_j w_ij^2 (v_jd' - O_id')^2;
* the final rounding of O adds at most u |O|; fp32 sums over n keys add at
  most 2 n 2^-24 (sum_j w_ij |v_j| + |O|).

The element bound is 6 standard deviations of the first three terms (the
sum of many independent roundings is close to normal; 6 sigma is exceeded
with probability ~2e-9 per element) plus the last two.  A CPU test checks it
against a NumPy emulation of exactly these roundings.
"""
import numpy as np

import oracle

U_BF16 = 2.0 ** -8
U_F32 = 2.0 ** -24


def bf16_round(x):
    """Round to bf16 (ties to even), returned as fp64."""
    f = np.asarray(x, np.float64).astype(np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _heads(qkv, offsets, n_heads, head_dim, rope_base):
    """Q, K rotated (the oracle's RoPE, positions restarting per text) and V,
    each [T, heads, d], fp64."""
    qkv = np.asarray(qkv, np.float64)
    T = qkv.shape[0]
    H = n_heads * head_dim
    pos = oracle.positions(offsets)
    q = oracle.rope(qkv[:, :H].reshape(T, n_heads, head_dim), pos, rope_base)
    k = oracle.rope(qkv[:, H:2 * H].reshape(T, n_heads, head_dim), pos, rope_base)
    v = qkv[:, 2 * H:].reshape(T, n_heads, head_dim)
    return q, k, v


def _allowed(n, is_global, window):
    i = np.arange(n)
    return np.ones((n, n), bool) if is_global else np.abs(i[:, None] - i[None, :]) <= window


def attention_bf16_bound(qkv, offsets, n_heads, head_dim, is_global, window, rope_base, sigmas=6.0):
    """Per-element bound [T, H] on |bf16 kernel - fp64 oracle| of one
    attention layer, and the standard deviation part alone."""
    q, k, v = _heads(qkv, offsets, n_heads, head_dim, rope_base)
    T = q.shape[0]
    off = np.asarray(offsets, np.int64)
    u = U_BF16
    bound = np.zeros((T, n_heads, head_dim))
    sd = np.zeros((T, n_heads, head_dim))
    scale = 1.0 / np.sqrt(head_dim)
    for b in range(len(off) - 1):
        lo, hi = off[b], off[b + 1]
        n = hi - lo
        mask = _allowed(n, is_global, window)
        for h in range(n_heads):
            Q, K, V = q[lo:hi, h], k[lo:hi, h], v[lo:hi, h]
            s = np.where(mask, (Q @ K.T) * scale, -np.inf)
            w = np.exp(s - s.max(axis=1, keepdims=True))
            w /= w.sum(axis=1, keepdims=True)
            O = w @ V
            # Q errors: C[i, d, d'] = sum_j w_ij k_jd (v_jd' - O_id')
            kbar = w @ K
            C = (w @ (K[:, :, None] * V[:, None, :]).reshape(n, -1)).reshape(n, head_dim, head_dim)
            C -= kbar[:, :, None] * O[:, None, :]
            var_q = np.einsum("id,ide->ie", (u * Q) ** 2 / 3.0, C ** 2) * scale ** 2
            # K errors and P errors: sum_j B_ij (v_jd' - O_id')^2
            def spread(Bm):
                return Bm @ V ** 2 - 2 * O * (Bm @ V) + O ** 2 * Bm.sum(axis=1, keepdims=True)
            A = (Q ** 2) @ (K ** 2).T
            var_k = (u ** 2 / 3.0) * scale ** 2 * spread(w ** 2 * A)
            var_p = (u ** 2 / 3.0) * spread(w ** 2)
            sigma = np.sqrt(np.maximum(var_q + var_k + var_p, 0.0))
            keys = mask.sum(axis=1, keepdims=True)
            fp32 = 2 * keys * U_F32 * (w @ np.abs(V) + np.abs(O))
            sd[lo:hi, h] = sigma
            bound[lo:hi, h] = sigmas * sigma + u * np.abs(O) + fp32 + 1e-7
    H = n_heads * head_dim
    return bound.reshape(T, H), sd.reshape(T, H)


def attention_bf16_emulated(qkv, offsets, n_heads, head_dim, is_global, window, rope_base):
    """The bf16 kernel's roundings replayed in NumPy (for checking the bound
    on the CPU): Q, K after RoPE to bf16, scores and sums in fp32, P to bf16
    with the row sum taken over the rounded P, O to bf16.  P is taken here
    against the row max; the kernel takes it against a reference that lags
    the running max by less than 2^8 (P <= 256), which scales P by a
    factor the softmax divides out again and leaves each rounding of P
    within the same relative u, the only property of P's rounding the
    bound uses."""
    q, k, v = _heads(qkv, offsets, n_heads, head_dim, rope_base)
    q, k = bf16_round(q), bf16_round(k)
    T = q.shape[0]
    off = np.asarray(offsets, np.int64)
    out = np.zeros((T, n_heads, head_dim))
    scale = 1.0 / np.sqrt(head_dim)
    for b in range(len(off) - 1):
        lo, hi = off[b], off[b + 1]
        mask = _allowed(hi - lo, is_global, window)
        for h in range(n_heads):
            Q, K, V = q[lo:hi, h], k[lo:hi, h], v[lo:hi, h]
            s = ((Q @ K.T).astype(np.float32) * np.float32(scale)).astype(np.float64)
            s = np.where(mask, s, -np.inf)
            p = bf16_round(np.exp(s - s.max(axis=1, keepdims=True)).astype(np.float32))
            l = p.sum(axis=1, keepdims=True).astype(np.float32).astype(np.float64)
            o = (p @ V).astype(np.float32).astype(np.float64)
            out[lo:hi, h] = bf16_round((o / l).astype(np.float32))
    return out.reshape(T, n_heads * head_dim)


# --------------------------------------------------------------------------
# integer paths: how far fp32 rounding alone moves the 7-bit pass
# --------------------------------------------------------------------------

def round_f32(a):
    """fp64 values rounded to the nearest fp32 (ties to even)."""
    return np.asarray(a, np.float64).astype(np.float32).astype(np.float64)


def encode_layers_fp32_rounded(cfg, w, ids, offsets):
    """The oracle's pass (tensai page, section 何が動くか, encoder paragraph;
    section 精度と量子化 for the 7-bit codes) composed from its own
    functions, with every intermediate -- norm outputs, projections,
    attention output, GeGLU, residual stream -- rounded to fp32 between
    steps, as a pass that stores fp32 activations does.  Each rounding moves
    a value by at most half an fp32 ulp; in the integer modes the 7-bit codes
    then amplify that (a value near a rounding boundary takes the
    neighbouring code, an error of amax/63), which is the spread the
    integer-path parity gates must allow.  Returns the residual states after
    the embedding norm and after each layer."""
    from oracle import encoder as E
    H, nh, d = cfg["hidden"], cfg["heads"], cfg["head_dim"]
    prec = cfg["precision"]
    emb = E.decode_matrix(w, "tok_emb", prec)
    off = E.validate_offsets(offsets, len(ids))
    x = round_f32(E.layer_norm(emb[np.asarray(ids, np.int64)], w["emb_norm"], cfg["ln_eps"]))
    states = [x]
    for l in range(cfg["layers"]):
        layer = w["layers"][l]
        g = (l % cfg["global_every"]) == 0
        base = cfg["rope_base_global"] if g else cfg["rope_base_local"]
        a = x if l == 0 else round_f32(E.layer_norm(x, layer["attn_norm"], cfg["ln_eps"]))
        qkv = round_f32(E._project(a, layer, "wqkv", prec))
        o = round_f32(E.attention(qkv, off, nh, d, g, cfg["window"], base))
        x = round_f32(x + round_f32(E._project(o, layer, "wo", prec)))
        m = round_f32(E.layer_norm(x, layer["mlp_norm"], cfg["ln_eps"]))
        y = round_f32(E.geglu(round_f32(E._project(m, layer, "wi", prec))))
        x = round_f32(x + round_f32(E._project(y, layer, "wo2", prec)))
        states.append(x)
    return states


def encode_layers_bf16_emulated(cfg, w, ids, offsets, stream_bf16=True):
    """The oracle's bf16 pass (tensai page, section 何が動くか, encoder
    paragraph) composed from its own functions, with the bf16 roundings of
    the kernels' data flow applied between steps: every weight-product and
    attention operand rounded to bf16 (norm outputs, Q/K/V, attention output,
    GeGLU output) and, with stream_bf16, the residual stream rounded to bf16
    after the embedding norm and after each of its updates (the update
    itself added exactly, as the kernels add it in fp32 and round once).
    Attention's internal roundings are left out (their own bound is
    attention_bf16_bound).  Returns the residual states after the embedding
    norm and after each layer."""
    from oracle import encoder as E
    nh, d, prec = cfg["heads"], cfg["head_dim"], cfg["precision"]
    rx = bf16_round if stream_bf16 else (lambda v: np.asarray(v, np.float64))
    emb = E.decode_matrix(w, "tok_emb", prec)
    off = E.validate_offsets(offsets, len(ids))
    x = rx(E.layer_norm(emb[np.asarray(ids, np.int64)], w["emb_norm"], cfg["ln_eps"]))
    states = [x]
    for l in range(cfg["layers"]):
        layer = w["layers"][l]
        g = (l % cfg["global_every"]) == 0
        base = cfg["rope_base_global"] if g else cfg["rope_base_local"]
        a = x if l == 0 else E.layer_norm(x, layer["attn_norm"], cfg["ln_eps"])
        qkv = bf16_round(E._project(bf16_round(a), layer, "wqkv", prec))
        o = E.attention(qkv, off, nh, d, g, cfg["window"], base)
        x = rx(x + E._project(bf16_round(o), layer, "wo", prec))
        m = E.layer_norm(x, layer["mlp_norm"], cfg["ln_eps"])
        y = E.geglu(E._project(bf16_round(m), layer, "wi", prec))
        x = rx(x + E._project(bf16_round(y), layer, "wo2", prec))
        states.append(x)
    return states


def pooled_spread(cfg, w, ids, offsets, states):
    """1 - min and 1 - mean over texts of the cosine between the oracle's
    pooled vectors and those pooled from `states[-1]`."""
    from oracle import encoder as E
    ref = oracle.encode(cfg, w, ids, offsets)
    got = E.mean_pool_l2(E.layer_norm(states[-1], w["final_norm"], cfg["ln_eps"]), offsets)
    c = cos_rows(ref, got)
    return 1 - c.min(), 1 - c.mean()


def cos_rows(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.sum(a * b, axis=1) / (np.linalg.norm(a, axis=1) * np.linalg.norm(b, axis=1))


def rounding_spread(cfg, w, ids, offsets):
    """Per state (embedding norm, then each layer): 1 - min and 1 - mean of
    the per-token cosine between the oracle's pass and the same pass with
    fp32 roundings between steps; and of the final pooled vectors."""
    from oracle import encoder as E
    a = E.encode_layers(cfg, w, ids, offsets)
    b = encode_layers_fp32_rounded(cfg, w, ids, offsets)
    per_min, per_mean = [], []
    for sa, sb in zip(a, b):
        c = cos_rows(sa, sb)
        per_min.append(1 - c.min())
        per_mean.append(1 - c.mean())
    ea = E.mean_pool_l2(E.layer_norm(a[-1], w["final_norm"], cfg["ln_eps"]), offsets)
    eb = E.mean_pool_l2(E.layer_norm(b[-1], w["final_norm"], cfg["ln_eps"]), offsets)
    c = cos_rows(ea, eb)
    return np.array(per_min), np.array(per_mean), 1 - c.min(), 1 - c.mean()
