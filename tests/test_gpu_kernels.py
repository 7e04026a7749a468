"""Per-kernel parity: each production HIP kernel, called through the C ABI on
seeded inputs, against the oracle's function for the same step.  Sizes span
several tiles and a ragged tail."""
import numpy as np
import pytest

import oracle
import tte_inputs as ti
from parity_bounds import attention_bf16_bound
from gpu_util import DEV, dev, empty, host, row_cosines, say, stream, sync, torch
from transformer_text_embedding_amd import B, Model

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------------------
# LayerNorm / quantisation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("width", [128, 768, 3072])
@pytest.mark.parametrize("rows", [1, 357])
def test_layernorm_fp32_bf16(width, rows):
    t = torch()
    rng = np.random.default_rng(100 + width + rows)
    x = (rng.normal(size=(rows, width)) * 3 + 1).astype(np.float32)
    g = (1 + rng.normal(0, 0.1, size=width)).astype(np.float32)
    dx, dg = dev(x), dev(g)
    out = empty((rows, width), t.float32)
    outb = empty((rows, width), t.int16)
    B.tte_op_layernorm(dx.data_ptr(), dg.data_ptr(), rows, width, 1e-5, B.TTE_OUT_F32, out.data_ptr(), 0, stream())
    B.tte_op_layernorm(dx.data_ptr(), dg.data_ptr(), rows, width, 1e-5, B.TTE_OUT_BF16, outb.data_ptr(), 0, stream())
    ref = oracle.layer_norm(x, g, 1e-5)
    np.testing.assert_allclose(host(out), ref, atol=2e-5, rtol=0)
    got_b = ti.bf16_to_f32(host(outb).view(np.uint16)).astype(np.float64)
    np.testing.assert_allclose(got_b, ref, rtol=2.0 ** -8, atol=1e-6)


@pytest.mark.parametrize("width", [768, 3072])
def test_quant7_bit_exact(width):
    t = torch()
    rng = np.random.default_rng(7 + width)
    rows = 301
    x = (rng.normal(size=(rows, width)) * rng.uniform(0.01, 50, size=(rows, 1))).astype(np.float32)
    x[3] = 0.0
    x[4, :8] = [63.0, 0.5, 1.5, 2.5, -0.5, -2.5, -63.0, 31.5]
    x[4, 8:] = 0.25
    x[5, :] = -1.0
    dx = dev(x)
    q = empty((rows, width), t.int8)
    s = empty((rows,), t.float32)
    B.tte_op_quant7(dx.data_ptr(), rows, width, q.data_ptr(), s.data_ptr(), stream())
    qr, sr = oracle.quantize_rows_7bit(x)
    np.testing.assert_array_equal(host(q), qr)
    np.testing.assert_array_equal(host(s), sr)


def test_layernorm_to_int8_codes():
    t = torch()
    rng = np.random.default_rng(5)
    rows, width = 257, 768
    x = rng.normal(size=(rows, width)).astype(np.float32)
    g = np.ones(width, np.float32)
    dx, dg = dev(x), dev(g)
    q = empty((rows, width), t.int8)
    s = empty((rows,), t.float32)
    B.tte_op_layernorm(dx.data_ptr(), dg.data_ptr(), rows, width, 1e-5, B.TTE_OUT_I8, q.data_ptr(), s.data_ptr(),
                       stream())
    qr, sr = oracle.quantize_rows_7bit(oracle.layer_norm(x, g, 1e-5))
    qg = host(q).astype(np.int64)
    # the LayerNorm itself is fp32 on the GPU and fp64 in the oracle: a value
    # within an ulp of a rounding boundary may land on the neighbouring code
    diff = np.abs(qg - qr)
    assert diff.max() <= 1 and np.mean(diff) < 1e-3
    np.testing.assert_allclose(host(s), sr, rtol=1e-5)


# --------------------------------------------------------------------------
# GEMMs
# --------------------------------------------------------------------------

# tile configurations: 4-wave 32x128 (few narrow tiles), 64x128, 64x128 with
# 3 stages (K > 1024), 128x128 (int8, >= 1024 tiles); 8-wave 128x128 (wide
# fp32 / bf16 products) and 256x256 (>= 512 such tiles, or residual
# products of >= 8k rows)
SHAPES = [(178, 384, 128), (957, 2304, 768), (300, 768, 3072), (130, 512, 256), (1, 128, 128), (4100, 4096, 128),
          (8200, 768, 3072), (1913, 2304, 768)]
# GeGLU (bf16) at 2001 rows takes the 128 x 192 tiles (512 blocks, where
# 192 x 128 tiles would make 528), with a ragged last row tile
GEGLU_SHAPES = [(178, 256, 128), (957, 3072, 768), (65, 64, 256), (2100, 4096, 128), (8192, 3072, 768),
                (1913, 3072, 768), (2001, 3072, 768)]


def _run_gemm(prec, epi, a, a_s, w, w_s, M, N, K, c, out_kind):
    B.tte_op_gemm(prec, epi, a.data_ptr(), a_s.data_ptr() if a_s is not None else 0, w.data_ptr(),
                  w_s.data_ptr() if w_s is not None else 0, M, N, K, c.data_ptr(), out_kind, stream())


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_fp32_store_and_residual(M, N, K):
    t = torch()
    say(f"gemm fp32 {M}x{N}x{K}")
    rng = np.random.default_rng(M + N + K)
    a = rng.normal(size=(M, K)).astype(np.float32)
    w = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    r = rng.normal(size=(M, N)).astype(np.float32)
    da, dw = dev(a), dev(w)
    c = empty((M, N), t.float32)
    _run_gemm(B.TTE_FP32, B.TTE_EPI_STORE, da, None, dw, None, M, N, K, c, B.TTE_OUT_F32)
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    np.testing.assert_allclose(host(c), ref, atol=2e-5, rtol=1e-5)
    cr = dev(r)
    _run_gemm(B.TTE_FP32, B.TTE_EPI_RESIDUAL, da, None, dw, None, M, N, K, cr, B.TTE_OUT_F32)
    np.testing.assert_allclose(host(cr), r + ref, atol=2e-5, rtol=1e-5)


@pytest.mark.parametrize("M,N,K", GEGLU_SHAPES)
@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_gemm_geglu(M, N, K, prec):
    t = torch()
    say(f"gemm geglu {prec} {M}x{N}x{K}")
    rng = np.random.default_rng(11 * M + N + K)
    a = rng.normal(size=(M, K)).astype(np.float32)
    w = rng.normal(0, 0.05, size=(2 * N, K)).astype(np.float32)
    if prec == "bf16":
        ab, wb = ti.bf16_bits(a), ti.bf16_bits(w)
        av, wv = ti.bf16_to_f32(ab).astype(np.float64), ti.bf16_to_f32(wb).astype(np.float64)
        da, dw = dev(ab), dev(wb)
        p = B.TTE_BF16
    else:
        av, wv = a.astype(np.float64), w.astype(np.float64)
        da, dw = dev(a), dev(w)
        p = B.TTE_FP32
    ref = oracle.geglu(av @ wv.T)
    c = empty((M, N), t.float32)
    _run_gemm(p, B.TTE_EPI_GEGLU, da, None, dw, None, M, N, K, c, B.TTE_OUT_F32)
    np.testing.assert_allclose(host(c), ref, atol=5e-5, rtol=1e-4)
    cb = empty((M, N), t.int16)
    _run_gemm(p, B.TTE_EPI_GEGLU, da, None, dw, None, M, N, K, cb, B.TTE_OUT_BF16)
    got = ti.bf16_to_f32(host(cb).view(np.uint16)).astype(np.float64)
    np.testing.assert_allclose(got, ref, atol=1e-4, rtol=2.0 ** -8)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_bf16(M, N, K):
    t = torch()
    say(f"gemm bf16 {M}x{N}x{K}")
    rng = np.random.default_rng(3 * M + N + K)
    ab = ti.bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    wb = ti.bf16_bits(rng.normal(0, 0.02, size=(N, K)).astype(np.float32))
    ref = ti.bf16_to_f32(ab).astype(np.float64) @ ti.bf16_to_f32(wb).astype(np.float64).T
    da, dw = dev(ab), dev(wb)
    c = empty((M, N), t.float32)
    _run_gemm(B.TTE_BF16, B.TTE_EPI_STORE, da, None, dw, None, M, N, K, c, B.TTE_OUT_F32)
    np.testing.assert_allclose(host(c), ref, atol=2e-5, rtol=1e-5)
    cb = empty((M, N), t.int16)
    _run_gemm(B.TTE_BF16, B.TTE_EPI_STORE, da, None, dw, None, M, N, K, cb, B.TTE_OUT_BF16)
    got = ti.bf16_to_f32(host(cb).view(np.uint16)).astype(np.float64)
    np.testing.assert_allclose(got, ref, atol=1e-6, rtol=2.0 ** -8)
    r = rng.normal(size=(M, N)).astype(np.float32)
    cr = dev(r)
    _run_gemm(B.TTE_BF16, B.TTE_EPI_RESIDUAL, da, None, dw, None, M, N, K, cr, B.TTE_OUT_F32)
    np.testing.assert_allclose(host(cr), r + ref, atol=2e-5, rtol=1e-5)
    # bf16 residual stream: x + A W^T summed in fp32 and rounded once to
    # bf16, so within half a bf16 ulp (at most 2^-8 of the value: 8
    # significant bits) of the exact sum plus
    # the fp32 product's error, and equal to the exact sum's rounding except
    # where that error crosses a rounding boundary
    rb = ti.bf16_bits(r)
    want = ti.bf16_to_f32(rb).astype(np.float64) + ref
    crb = dev(rb)
    _run_gemm(B.TTE_BF16, B.TTE_EPI_RESIDUAL, da, None, dw, None, M, N, K, crb, B.TTE_OUT_BF16)
    got = ti.bf16_to_f32(host(crb).view(np.uint16)).astype(np.float64)
    np.testing.assert_allclose(got, want, atol=2e-5, rtol=2.0 ** -8)
    same = got == ti.bf16_to_f32(ti.bf16_bits(want.astype(np.float32))).astype(np.float64)
    say(f"  bf16 residual: {same.mean():.5f} of elements equal the exact sum's rounding")
    assert same.mean() > 0.99


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_int8_bit_exact_int32_accumulation(M, N, K):
    """With every scale 1 the output is the exact integer sum: each 32-block
    sum is < 2^18 and the running fp32 sum stays below 2^24."""
    t = torch()
    say(f"gemm int8 exact {M}x{N}x{K}")
    rng = np.random.default_rng(5 * M + N + K)
    wmax = 127 if K <= 1024 else 63
    qx = rng.integers(-63, 64, size=(M, K)).astype(np.int8)
    qw = rng.integers(-wmax, wmax + 1, size=(N, K)).astype(np.int8)
    sx = np.ones(M, np.float32)
    sw = np.ones((N, K // 32), np.float32)
    exact = qx.astype(np.int64) @ qw.astype(np.int64).T
    assert np.abs(exact).max() < 2 ** 24
    dqx, dsx, dqw, dsw = dev(qx), dev(sx), dev(qw), dev(sw)
    c = empty((M, N), t.float32)
    _run_gemm(B.TTE_INT8, B.TTE_EPI_STORE, dqx, dsx, dqw, dsw, M, N, K, c, B.TTE_OUT_F32)
    got = host(c)
    assert np.array_equal(got.astype(np.int64), exact) and np.all(got == exact.astype(np.float32))


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_int8_scaled(M, N, K):
    t = torch()
    rng = np.random.default_rng(9 * M + N + K)
    x = rng.normal(size=(M, K)).astype(np.float32)
    x[0] = 0.0  # a zero row: scale 0
    qx, sx = oracle.quantize_rows_7bit(x)
    qw, sw = ti.quantize_weight_blocks(rng.normal(0, 0.02, size=(N, K)).astype(np.float32))
    sw[0, 0] = 0.0
    qw[0, :32] = 0
    ref = oracle.block_matmul_int8(qx, sx, qw, sw)
    dqx, dsx, dqw, dsw = dev(qx), dev(sx), dev(qw), dev(sw)
    c = empty((M, N), t.float32)
    _run_gemm(B.TTE_INT8, B.TTE_EPI_STORE, dqx, dsx, dqw, dsw, M, N, K, c, B.TTE_OUT_F32)
    got = host(c)
    scale = np.abs(ref).max()
    np.testing.assert_allclose(got, ref, atol=2e-6 * scale, rtol=1e-5)
    assert np.all(got[0] == 0)
    # residual and GeGLU epilogues on the same operands
    r = rng.normal(size=(M, N)).astype(np.float32)
    cr = dev(r)
    _run_gemm(B.TTE_INT8, B.TTE_EPI_RESIDUAL, dqx, dsx, dqw, dsw, M, N, K, cr, B.TTE_OUT_F32)
    np.testing.assert_allclose(host(cr), r + ref, atol=2e-6 * scale + 1e-6, rtol=1e-5)
    if N % 128 == 0:
        half = N // 2
        cg = empty((M, half), t.float32)
        _run_gemm(B.TTE_INT8, B.TTE_EPI_GEGLU, dqx, dsx, dqw, dsw, M, half, K, cg, B.TTE_OUT_F32)
        np.testing.assert_allclose(host(cg), oracle.geglu(ref), atol=4e-6 * scale * scale + 1e-6, rtol=1e-4)


# 4-bit weights: K a multiple of 256; 4-wave 32/64-row tiles and 128x128
# (>= 1024 tiles), 2 and 3 stages
Q4_SHAPES = [(178, 384, 256), (957, 2304, 768), (300, 768, 3072), (130, 512, 256), (1, 128, 256),
             (4100, 4096, 256), (1913, 2304, 768), (8200, 768, 3072)]


def _q4_pack(q, sc, mn, d, dmin):
    """Packed codes and per-128 records from codes q [N, K] in [0, 15],
    per-32 sc, mn [N, K/32] and per-128 fp32 d, dmin [N, K/128]."""
    N, K = q.shape
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    meta = np.zeros((N, K // 128, 16), np.uint8)
    meta[:, :, 0:4] = sc.reshape(N, K // 128, 4)
    meta[:, :, 4:8] = mn.reshape(N, K // 128, 4)
    meta[:, :, 8:12] = np.asarray(d, "<f4").view(np.uint8).reshape(N, K // 128, 4)
    meta[:, :, 12:16] = np.asarray(dmin, "<f4").view(np.uint8).reshape(N, K // 128, 4)
    return codes, meta


def _q4_exact_operands(M, N, K, rng):
    """Operands whose product every fp32 step represents exactly: codes and
    indices small integers, d and dmin powers of two >= 1/4, and
    sum |terms| < 2^22 in units of 1/4."""
    amax = 63 if K <= 1024 else 15
    qx = rng.integers(-amax, amax + 1, size=(M, K)).astype(np.int8)
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    sc = rng.integers(1, 4, size=(N, K // 32)).astype(np.uint8)
    mn = rng.integers(0, 9, size=(N, K // 32)).astype(np.uint8)
    d = rng.choice(np.array([0.25, 0.5, 1.0], np.float32), size=(N, K // 128))
    dmin = rng.choice(np.array([0.5, 1.0], np.float32), size=(N, K // 128))
    codes, meta = _q4_pack(q, sc, mn, d, dmin)
    bound = (K // 32) * 32 * amax * (3 * 15 + 8) * 4
    assert bound < 2 ** 24
    return qx, codes, meta


@pytest.mark.parametrize("M,N,K", Q4_SHAPES)
def test_gemm_int4_exact(M, N, K):
    """Every block scale, offset and partial sum representable: the output
    equals the fp64 definition exactly, so a wrong nibble order, record
    field or block index shows as a mismatch, not as a small error."""
    t = torch()
    say(f"gemm int4 exact {M}x{N}x{K}")
    rng = np.random.default_rng(19 * M + N + K)
    qx, codes, meta = _q4_exact_operands(M, N, K, rng)
    sx = np.ones(M, np.float32)
    exact = oracle.block_matmul_q4(qx, sx, codes, meta)
    dqx, dsx, dqw, dsw = dev(qx), dev(sx), dev(codes), dev(meta)
    c = empty((M, N), t.float32)
    _run_gemm(B.TTE_INT4, B.TTE_EPI_STORE, dqx, dsx, dqw, dsw, M, N, K, c, B.TTE_OUT_F32)
    got = host(c)
    bad = np.argwhere(got != exact)
    assert bad.size == 0, (bad[:5], got[tuple(bad[0])], exact[tuple(bad[0])])


def _q4_bound(qx, sx, codes, meta):
    """A bound on the fp32 evaluation error of block_matmul_q4: every partial
    sum is at most sx * sum |qx| (|es q| + |eo|) in magnitude, and each of
    the 2 K/32 + 2 fused steps rounds once."""
    q = oracle.q4_codes(codes)
    N, K = q.shape
    es, eo = oracle.q4_block_params(meta)
    mag = (np.abs(q.astype(np.float64)).reshape(N, K // 32, 32) * es.astype(np.float64)[:, :, None]
           + eo.astype(np.float64)[:, :, None]).reshape(N, K)
    total = np.abs(np.asarray(sx, np.float64))[:, None] * (np.abs(qx.astype(np.float64)) @ mag.T)
    return (2 * K // 32 + 2) * 2.0 ** -24 * total


@pytest.mark.parametrize("M,N,K", Q4_SHAPES)
def test_gemm_int4_scaled(M, N, K):
    """Quantised weights and 7-bit activations against the oracle's
    block_matmul_q4, in the store, residual and GeGLU epilogues."""
    t = torch()
    say(f"gemm int4 scaled {M}x{N}x{K}")
    rng = np.random.default_rng(23 * M + N + K)
    x = rng.normal(size=(M, K)).astype(np.float32)
    x[0] = 0.0  # a zero row: scale 0
    qx, sx = oracle.quantize_rows_7bit(x)
    codes, meta = ti.quantize_weight_q4(rng.normal(0, 0.02, size=(N, K)).astype(np.float32))
    meta[0, 0, :] = 0  # a zero record: es = eo = 0 for its 128 inputs
    ref = oracle.block_matmul_q4(qx, sx, codes, meta)
    tol = _q4_bound(qx, sx, codes, meta) + 1e-30
    dqx, dsx, dqw, dsw = dev(qx), dev(sx), dev(codes), dev(meta)
    c = empty((M, N), t.float32)
    _run_gemm(B.TTE_INT4, B.TTE_EPI_STORE, dqx, dsx, dqw, dsw, M, N, K, c, B.TTE_OUT_F32)
    got = host(c)
    assert np.all(np.abs(got - ref) <= tol), np.abs(got - ref).max()
    assert np.all(got[0] == 0)
    r = rng.normal(size=(M, N)).astype(np.float32)
    cr = dev(r)
    _run_gemm(B.TTE_INT4, B.TTE_EPI_RESIDUAL, dqx, dsx, dqw, dsw, M, N, K, cr, B.TTE_OUT_F32)
    assert np.all(np.abs(host(cr) - (r + ref)) <= tol + 2.0 ** -23 * np.abs(r + ref))
    if N % 128 == 0:
        half = N // 2
        cg = empty((M, half), t.float32)
        _run_gemm(B.TTE_INT4, B.TTE_EPI_GEGLU, dqx, dsx, dqw, dsw, M, half, K, cg, B.TTE_OUT_F32)
        scale = np.abs(ref).max()
        np.testing.assert_allclose(host(cg), oracle.geglu(ref), atol=1e-5 * scale * scale + 1e-6, rtol=1e-4)
        cb = empty((M, half), t.int16)
        _run_gemm(B.TTE_INT4, B.TTE_EPI_GEGLU, dqx, dsx, dqw, dsw, M, half, K, cb, B.TTE_OUT_BF16)
        got_b = ti.bf16_to_f32(host(cb).view(np.uint16)).astype(np.float64)
        np.testing.assert_allclose(got_b, oracle.geglu(ref), atol=1e-5 * scale * scale + 1e-6, rtol=2.0 ** -8)


# split-K residual projection: (M, N, K, splits); 2 or 3 stages per part
SPLIT_SHAPES = [(957, 768, 3072, 2), (1913, 768, 3072, 4), (178, 384, 256, 2), (65, 256, 1536, 3), (1, 128, 512, 2)]


def _split_operands(prec, M, N, K, rng):
    """Device operands and fp64 per-part references of the split product."""
    if prec == "int8":
        x = rng.normal(size=(M, K)).astype(np.float32)
        qx, sx = oracle.quantize_rows_7bit(x)
        qw, sw = ti.quantize_weight_blocks(rng.normal(0, 0.02, size=(N, K)).astype(np.float32))
        return (B.TTE_INT8, dev(qx), dev(sx), dev(qw), dev(sw),
                lambda k0, k1: oracle.block_matmul_int8(qx[:, k0:k1], sx, qw[:, k0:k1], sw[:, k0 // 32:k1 // 32]))
    if prec == "int4":
        x = rng.normal(size=(M, K)).astype(np.float32)
        qx, sx = oracle.quantize_rows_7bit(x)
        codes, meta = ti.quantize_weight_q4(rng.normal(0, 0.02, size=(N, K)).astype(np.float32))
        return (B.TTE_INT4, dev(qx), dev(sx), dev(codes), dev(meta),
                lambda k0, k1: oracle.block_matmul_q4(qx[:, k0:k1], sx, codes[:, k0 // 2:k1 // 2],
                                                      meta[:, k0 // 128:k1 // 128]))
    a = rng.normal(size=(M, K)).astype(np.float32)
    w = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    if prec == "bf16":
        ab, wb = ti.bf16_bits(a), ti.bf16_bits(w)
        av, wv = ti.bf16_to_f32(ab).astype(np.float64), ti.bf16_to_f32(wb).astype(np.float64)
        return B.TTE_BF16, dev(ab), None, dev(wb), None, lambda k0, k1: av[:, k0:k1] @ wv[:, k0:k1].T
    av, wv = a.astype(np.float64), w.astype(np.float64)
    return B.TTE_FP32, dev(a), None, dev(w), None, lambda k0, k1: av[:, k0:k1] @ wv[:, k0:k1].T


@pytest.mark.parametrize("M,N,K,splits", SPLIT_SHAPES)
@pytest.mark.parametrize("prec", ["fp32", "bf16", "int8", "int4"])
def test_gemm_splitk_partials(M, N, K, splits, prec):
    t = torch()
    say(f"gemm split-K {prec} {M}x{N}x{K} / {splits}")
    rng = np.random.default_rng(13 * M + N + K + splits)
    p, da, das, dw, dws, part_ref = _split_operands(prec, M, N, K, rng)
    c = empty((splits, M, N), t.float32)
    B.tte_op_gemm_splitk(p, da.data_ptr(), das.data_ptr() if das is not None else 0, dw.data_ptr(),
                         dws.data_ptr() if dws is not None else 0, M, N, K, splits, c.data_ptr(), stream())
    got = host(c)
    kp = K // splits
    for s in range(splits):
        ref = part_ref(s * kp, (s + 1) * kp)
        np.testing.assert_allclose(got[s], ref, atol=2e-5 * max(1.0, np.abs(ref).max()), rtol=1e-5)


@pytest.mark.parametrize("M,N,K,splits", [(300, 256, 1024, 2), (64, 128, 768, 3)])
def test_gemm_splitk_int8_bit_exact(M, N, K, splits):
    """Scales 1: every partial is its exact integer sum."""
    t = torch()
    rng = np.random.default_rng(17 * M + K)
    qx = rng.integers(-63, 64, size=(M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    # device operands stay referenced until the kernel has run
    dqx, dsx, dqw, dsw = dev(qx), dev(np.ones(M, np.float32)), dev(qw), dev(np.ones((N, K // 32), np.float32))
    c = empty((splits, M, N), t.float32)
    B.tte_op_gemm_splitk(B.TTE_INT8, dqx.data_ptr(), dsx.data_ptr(), dqw.data_ptr(), dsw.data_ptr(), M, N, K, splits,
                         c.data_ptr(), stream())
    got = host(c)
    kp = K // splits
    for s in range(splits):
        exact = qx[:, s * kp:(s + 1) * kp].astype(np.int64) @ qw[:, s * kp:(s + 1) * kp].astype(np.int64).T
        assert np.array_equal(got[s].astype(np.int64), exact) and np.all(got[s] == exact.astype(np.float32))


@pytest.mark.parametrize("width,rows,splits", [(768, 357, 2), (768, 1, 4), (3072, 65, 1), (768, 100, 0)])
def test_resid_ln(width, rows, splits):
    """x += sum of partials, then LayerNorm / conversion / 7-bit codes."""
    t = torch()
    rng = np.random.default_rng(31 * width + rows + splits)
    x = (rng.normal(size=(rows, width)) * 2).astype(np.float32)
    parts = rng.normal(size=(max(splits, 1), rows, width)).astype(np.float32)
    g = (1 + rng.normal(0, 0.1, size=width)).astype(np.float32)
    new_x = x.copy()
    for s in range(splits):
        new_x = new_x + parts[s]  # fp32, in split order, as the kernel adds
    ref = oracle.layer_norm(new_x, g, 1e-5)
    dp, dg = dev(parts), dev(g)
    for kind in (B.TTE_OUT_F32, B.TTE_OUT_BF16, B.TTE_OUT_I8, -1):
        dx = dev(x)
        out = empty((rows, width), {B.TTE_OUT_F32: t.float32, B.TTE_OUT_BF16: t.int16}.get(kind, t.int8))
        sc = empty((rows,), t.float32)
        B.tte_op_resid_ln(dx.data_ptr(), dp.data_ptr(), splits, dg.data_ptr(), rows, width, 1e-5, kind,
                          out.data_ptr() if kind >= 0 else 0, sc.data_ptr() if kind == B.TTE_OUT_I8 else 0, stream())
        np.testing.assert_array_equal(host(dx), new_x)
        if kind == B.TTE_OUT_F32:
            np.testing.assert_allclose(host(out), ref, atol=2e-5, rtol=0)
        elif kind == B.TTE_OUT_BF16:
            got_b = ti.bf16_to_f32(host(out).view(np.uint16)).astype(np.float64)
            np.testing.assert_allclose(got_b, ref, rtol=2.0 ** -8, atol=1e-6)
        elif kind == B.TTE_OUT_I8:
            qr, sr = oracle.quantize_rows_7bit(ref)
            diff = np.abs(host(out).astype(np.int64) - qr)
            assert diff.max() <= 1 and np.mean(diff) < 1e-3
            np.testing.assert_allclose(host(sc), sr, rtol=1e-5)
    # no norm: plain conversion of the updated rows
    dx = dev(x)
    out = empty((rows, width), t.float32)
    B.tte_op_resid_ln(dx.data_ptr(), dp.data_ptr(), splits, 0, rows, width, 1e-5, B.TTE_OUT_F32, out.data_ptr(), 0,
                      stream())
    np.testing.assert_array_equal(host(out), new_x)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def _attn_model(precision, hidden, heads):
    spec = dict(vocab=64, hidden=hidden, heads=heads, head_dim=64, intermediate=2 * hidden, layers=3,
                precision=precision, global_every=3, window=64, rope_base_global=160000.0,
                rope_base_local=10000.0, ln_eps=1e-5)
    cfg = ti.EncoderConfig(name="attn", seed=9, **spec)
    w = ti.storage_weights(cfg)
    return Model(spec, w, max_tokens=4096, max_text_len=4096, max_texts=64)


# bf16 global layers take 128-query blocks when the texts average >= 1024
# tokens ([2048], [1100, 1037], [3000, 7]: the last two with ragged tails,
# and a short text inside the last block), 64-query blocks otherwise
ATTN_PACKS = [[8, 40, 130], [1, 64, 65, 200, 3, 129], [957], [2048], [5, 3000, 2], [1100, 1037], [3000, 7]]


@pytest.mark.parametrize("lengths", ATTN_PACKS)
@pytest.mark.parametrize("precision", ["fp32", "bf16"])
@pytest.mark.parametrize("layer", [0, 1])
def test_attention(precision, lengths, layer):
    t = torch()
    heads = 2 if sum(lengths) > 1000 else 12
    say(f"attention {precision} layer {layer} lengths {lengths} heads {heads}")
    m = _attn_model(precision, 64 * heads, heads)
    rng = np.random.default_rng(sum(lengths) + layer)
    T, H = sum(lengths), 64 * heads
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    qkv = (rng.normal(size=(T, 3 * H)) * 1.5).astype(np.float32)
    if precision == "bf16":
        bits = ti.bf16_bits(qkv)
        qv = ti.bf16_to_f32(bits).astype(np.float64)
        dq = dev(bits)
        o = empty((T, H), t.int16)
    else:
        qv = qkv.astype(np.float64)
        dq = dev(qkv)
        o = empty((T, H), t.float32)
    B.tte_op_attention(m.handle, layer, dq.data_ptr(), T, off, o.data_ptr(), stream())
    is_global = layer % 3 == 0
    ref = oracle.attention(qv, off, heads, 64, is_global, 64, 160000.0 if is_global else 10000.0)
    got = host(o)
    if precision == "bf16":
        got = ti.bf16_to_f32(got.view(np.uint16)).astype(np.float64)
        cos = row_cosines(got.reshape(T * heads, 64), ref.reshape(T * heads, 64))
        assert cos.min() > 0.999, cos.min()
        # per-element bound from the kernel's bf16 roundings (Q and K after
        # RoPE, P, O) and fp32 sums, at this input's scale
        bound, _ = attention_bf16_bound(qv, off, heads, 64, is_global, 64, 160000.0 if is_global else 10000.0)
        err = np.abs(got - ref)
        say(f"  max |err| {err.max():.4f}, max |err| / bound {(err / bound).max():.3f}")
        assert np.all(err <= bound), (err / bound).max()
        assert err.mean() < 5e-3
    else:
        np.testing.assert_allclose(got, ref, atol=2e-5, rtol=0)
    m.close()


# --------------------------------------------------------------------------
# similarity matrix
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,dim", [(1, 768), (5, 768), (16, 128), (17, 768), (130, 768), (64, 16)])
def test_similarity_matrix(n, dim):
    t = torch()
    rng = np.random.default_rng(41 * n + dim)
    e = rng.normal(size=(n, dim))
    e = (e / np.linalg.norm(e, axis=1, keepdims=True)).astype(np.float32)
    de = dev(e)
    sim = empty((n, n), t.float32)
    B.tte_similarity(de.data_ptr(), n, dim, sim.data_ptr(), stream())
    got = host(sim)
    ref = oracle.cosine_matrix(e)
    # fp32 products and sums of dim terms of size <= 1
    np.testing.assert_allclose(got, ref, atol=2e-6, rtol=0)
    np.testing.assert_allclose(np.diag(got), 1.0, atol=2e-6)
    np.testing.assert_array_equal(got, got.T)  # same products, same order


# --------------------------------------------------------------------------
# pooling
# --------------------------------------------------------------------------

@pytest.mark.parametrize("lengths", [[8, 40, 130], [1], [33, 32, 31, 1, 64, 100, 2000]])
def test_pool(lengths):
    t = torch()
    spec = ti.workload("tiny_fp32")["cfg"]
    w = ti.storage_weights(spec)
    rng = np.random.default_rng(len(lengths))
    w["final_norm"] = (1 + rng.normal(0, 0.1, size=spec.hidden)).astype(np.float32)
    m = Model(spec, w, max_tokens=4096, max_text_len=4096, max_texts=16)
    T = sum(lengths)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x = (rng.normal(size=(T, spec.hidden)) * 2 + 0.3).astype(np.float32)
    dx = dev(x)
    out = empty((len(lengths), spec.hidden), t.float32)
    B.tte_op_pool(m.handle, dx.data_ptr(), T, off, out.data_ptr(), stream())
    ref = oracle.mean_pool_l2(oracle.layer_norm(x, w["final_norm"], 1e-5), off)
    np.testing.assert_allclose(host(out), ref, atol=2e-6, rtol=0)
    m.close()


# --------------------------------------------------------------------------
# QKV projection with the fused RoPE / transposed-V epilogue
# --------------------------------------------------------------------------

@pytest.mark.parametrize("precision", ["fp32", "bf16", "int8", "int4"])
# 178 and 433 tokens take the 128-row tiles, 1913 the 192-row ones (bf16)
@pytest.mark.parametrize("lengths", [[8, 40, 130], [1, 64, 65, 300, 3], [500, 700, 713]])
@pytest.mark.parametrize("layer", [0, 1])
def test_qkv_rope_epilogue(precision, lengths, layer):
    t = torch()
    heads = 12
    m = _attn_model(precision, 64 * heads, heads)
    cfg = m.spec
    w = ti.storage_weights(ti.EncoderConfig(name="attn", seed=9, **{k: cfg[k] for k in (
        "vocab", "hidden", "heads", "head_dim", "intermediate", "layers", "precision", "global_every", "window",
        "rope_base_global", "rope_base_local", "ln_eps")}))
    L = w["layers"][layer]
    T, H = sum(lengths), 64 * heads
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rng = np.random.default_rng(T + layer)
    x = rng.normal(size=(T, H)).astype(np.float32)
    if precision == "int8":
        qx, sx = oracle.quantize_rows_7bit(x)
        da, ds = dev(qx), dev(sx)
        raw = oracle.block_matmul_int8(qx, sx, L["wqkv_q"], L["wqkv_s"])
    elif precision == "int4":
        qx, sx = oracle.quantize_rows_7bit(x)
        da, ds = dev(qx), dev(sx)
        raw = oracle.block_matmul_q4(qx, sx, L["wqkv_q4"], L["wqkv_q4m"])
    elif precision == "bf16":
        xb = ti.bf16_bits(x)
        da, ds = dev(xb), None
        raw = ti.bf16_to_f32(xb).astype(np.float64) @ oracle.decode_matrix(L, "wqkv", "bf16").T
    else:
        da, ds = dev(x), None
        raw = x.astype(np.float64) @ oracle.decode_matrix(L, "wqkv", "fp32").T
    is_global = layer % 3 == 0
    base = 160000.0 if is_global else 10000.0
    pos = oracle.positions(off)
    q = oracle.rope(raw[:, :H].reshape(T, heads, 64), pos, base).reshape(T, H)
    k = oracle.rope(raw[:, H:2 * H].reshape(T, heads, 64), pos, base).reshape(T, H)
    vT = raw[:, 2 * H:].T
    dt = t.int16 if precision == "bf16" else t.float32
    # zero-filled: the kernel leaves columns 2H.. (V) of qk untouched
    qk = torch().zeros((T, 3 * H), dtype=dt, device=DEV)
    vt = empty((H, T), dt)
    B.tte_op_qkv(m.handle, layer, da.data_ptr(), ds.data_ptr() if ds is not None else 0, T, off, qk.data_ptr(),
                 vt.data_ptr(), stream())
    got_qk, got_vt = host(qk), host(vt)
    if precision == "bf16":
        got_qk = ti.bf16_to_f32(got_qk.view(np.uint16)).astype(np.float64)
        got_vt = ti.bf16_to_f32(got_vt.view(np.uint16)).astype(np.float64)
        tol = dict(rtol=2.0 ** -8, atol=1e-5)
    else:
        tol = dict(rtol=1e-5, atol=2e-5 * np.abs(raw).max())
    np.testing.assert_allclose(got_qk[:, :H], q, **tol)
    np.testing.assert_allclose(got_qk[:, H:2 * H], k, **tol)
    np.testing.assert_allclose(got_vt, vT, **tol)
    m.close()
