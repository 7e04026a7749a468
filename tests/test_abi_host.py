"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/tte.h declares, sizes workspaces, and rejects bad
configs and packs before anything would be enqueued."""
import ctypes
import os

import pytest

import tte_inputs as ti
from conftest import gpu_available
from transformer_text_embedding_amd import B, make_config


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from transformer_text_embedding_amd.build import build
        build()
    return B.lib()


def _cfg(name="full_bf16_packs2048", **kw):
    c = make_config(ti.workload(name)["cfg"], max_tokens=2048, max_text_len=512, max_texts=256)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_library_exports_every_declared_function(lib):
    names = B.header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
        assert n in B._SIGS, f"{n} has no binding"


def test_workspace_size_grows_with_limits(lib):
    a = B.tte_workspace_size(_cfg())
    b = B.tte_workspace_size(_cfg(max_tokens=4096))
    assert 0 < a < b
    assert a % 256 == 0


def test_split_k_flag_adds_partials_workspace(lib):
    a = B.tte_workspace_size(_cfg())
    b = B.tte_workspace_size(_cfg(flags=B.TTE_FLAG_SPLIT_K))
    assert b - a == 4 * 2048 * 768 * 4  # up to four fp32 partial products [max_tokens, H]


def test_graph_stats_rejects_null(lib):
    import ctypes as ct
    a, b, c = ct.c_int32(0), ct.c_int32(0), ct.c_int64(0)
    assert lib.tte_graph_stats(None, ct.byref(a), ct.byref(b), ct.byref(c)) == B.TTE_E_INVALID
    assert B.last_error()


def test_graph_flag_accepted_without_extra_workspace(lib):
    """TTE_FLAG_GRAPH keeps its graphs host-side: the workspace is the same."""
    assert B.tte_workspace_size(_cfg(flags=B.TTE_FLAG_GRAPH)) == B.tte_workspace_size(_cfg())
    assert B.tte_workspace_size(_cfg(flags=B.TTE_FLAG_GRAPH | B.TTE_FLAG_SPLIT_K)) == \
        B.tte_workspace_size(_cfg(flags=B.TTE_FLAG_SPLIT_K))


@pytest.mark.parametrize("field,value", [
    ("head_dim", 32), ("hidden", 700), ("intermediate", 3000), ("precision", 7), ("max_tokens", 0),
    ("global_every", 0), ("window", -1), ("ln_eps", 0.0), ("n_layers", 0), ("max_texts", 0), ("flags", 4)])
def test_bad_configs_rejected(lib, field, value):
    c = _cfg(**{field: value})
    n = ctypes.c_size_t(0)
    st = lib.tte_workspace_size(ctypes.byref(c), ctypes.byref(n))
    assert st == B.TTE_E_INVALID
    assert B.last_error()


@pytest.mark.parametrize("T,offsets,ok", [
    (10, [0, 3, 10], True),
    (0, [0], True),                 # empty pack: a no-op
    (10, [1, 3, 10], False),        # offsets[0] != 0
    (10, [0, 3, 3, 10], False),     # empty text
    (10, [0, 6, 4, 10], False),     # decreasing
    (10, [0, 3, 9], False),         # last != n_tokens
    (3000, [0, 500, 1000, 1500, 2000, 2500, 3000], False),  # n_tokens > max_tokens
    (600, [0, 600], False),         # text longer than max_text_len
])
def test_pack_validation(lib, T, offsets, ok):
    st = B.tte_check_pack(_cfg(), T, offsets)
    assert (st == B.TTE_OK) == ok, B.last_error()
    if not ok:
        assert st == B.TTE_E_INVALID and B.last_error()


def test_too_many_texts(lib):
    c = _cfg(max_texts=2)
    assert B.tte_check_pack(c, 6, [0, 2, 4, 6]) == B.TTE_E_INVALID
    assert "max_texts" in B.last_error()


def test_null_model_is_invalid(lib):
    st = lib.tte_embed(None, None, 0, None, 0, None, None)
    assert st == B.TTE_E_INVALID
    assert lib.tte_destroy(None) == B.TTE_E_INVALID


def test_op_gemm_shape_checks_need_no_gpu(lib):
    # N not a multiple of 128 is refused before any launch
    st = lib.tte_op_gemm(B.TTE_BF16, B.TTE_EPI_STORE, None, None, None, None, 16, 100, 128, None, 0, None)
    assert st == B.TTE_E_UNSUPPORTED
    st = lib.tte_op_gemm(B.TTE_BF16, B.TTE_EPI_STORE, None, None, None, None, 16, 128, 96, None, 0, None)
    assert st == B.TTE_E_UNSUPPORTED
    st = lib.tte_op_gemm(B.TTE_INT8, B.TTE_EPI_RESIDUAL, None, None, None, None, 16, 128, 128, None, 1, None)
    assert st == B.TTE_E_INVALID
    st = lib.tte_op_gemm(B.TTE_FP32, B.TTE_EPI_RESIDUAL, None, None, None, None, 16, 128, 128, None, 1, None)
    assert st == B.TTE_E_INVALID
    # a bf16 residual stream is accepted with bf16 operands (M = 0: no launch)
    st = lib.tte_op_gemm(B.TTE_BF16, B.TTE_EPI_RESIDUAL, None, None, None, None, 0, 128, 128, None, 1, None)
    assert st == B.TTE_OK
    # split-K: K must divide into parts of whole 128-byte chunks
    st = lib.tte_op_gemm_splitk(B.TTE_BF16, None, None, None, None, 16, 128, 320, 2, None, None)
    assert st == B.TTE_E_UNSUPPORTED
    st = lib.tte_op_gemm_splitk(B.TTE_BF16, None, None, None, None, 16, 128, 512, 0, None, None)
    assert st == B.TTE_E_INVALID
    st = lib.tte_op_resid_ln(None, None, 1, None, 4, 768, 1e-5, 3, None, None, None)
    assert st == B.TTE_E_INVALID


@pytest.mark.parametrize("prec,epi,N,K,ok", [
    # the kernels address W rows with 32-bit byte offsets: W must stay below 4 GiB
    (B.TTE_FP32, B.TTE_EPI_STORE, 32768, 32768, False),     # 2^32 bytes
    (B.TTE_FP32, B.TTE_EPI_STORE, 32768 - 128, 32768, True),
    (B.TTE_BF16, B.TTE_EPI_STORE, 65536, 32768, False),     # 2^32 bytes
    (B.TTE_BF16, B.TTE_EPI_STORE, 65536 - 128, 32768, True),
    (B.TTE_BF16, B.TTE_EPI_GEGLU, 32768, 32768, False),     # 2N rows: 2^32 bytes
    (B.TTE_BF16, B.TTE_EPI_GEGLU, 32768 - 64, 32768, True),
    (B.TTE_INT8, B.TTE_EPI_STORE, 1 << 20, 4096, False),    # 2^32 bytes
    (B.TTE_INT4, B.TTE_EPI_STORE, 1 << 20, 8192, False),    # 4-bit codes: K/2 bytes a row, 2^32
    (B.TTE_INT4, B.TTE_EPI_STORE, 1 << 20, 4096, True),
])
def test_op_gemm_refuses_weights_beyond_32bit_offsets(lib, prec, epi, N, K, ok):
    """Refused before anything is launched: fake non-null pointers are never
    dereferenced on either path here (the accepted shapes stop at M = 0)."""
    fake = ctypes.c_void_p(256)
    st = lib.tte_op_gemm(prec, epi, fake, fake, fake, fake, 0 if ok else 16, N, K, fake, 0, None)
    assert st == (B.TTE_OK if ok else B.TTE_E_UNSUPPORTED), (st, B.last_error())
    if not ok:
        assert "32-bit" in B.last_error()
    if epi == B.TTE_EPI_STORE and not ok:
        st = lib.tte_op_gemm_splitk(prec, fake, fake, fake, fake, 16, N, K, 1, fake, None)
        assert st == B.TTE_E_UNSUPPORTED and "32-bit" in B.last_error()


@pytest.mark.skipif(gpu_available(), reason="checks the no-device path")
def test_create_without_device_reports_device_error(lib):
    cfg = _cfg()
    layers = (B.tte_layer_weights * cfg.n_layers)()
    fake = 256
    for l in range(cfg.n_layers):
        for f in ("wqkv", "wo", "wi", "wo2", "mlp_norm", "attn_norm"):
            setattr(layers[l], f, fake)
    w = B.tte_weights(tok_emb=fake, emb_norm=fake, final_norm=fake, layers=layers)
    out = ctypes.c_void_p(0)
    st = lib.tte_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.c_void_p(fake), 1 << 40, ctypes.byref(out))
    assert st == B.TTE_E_DEVICE
    assert "device" in B.last_error()


def test_similarity_and_token_entry_checks_need_no_gpu(lib):
    assert lib.tte_similarity(None, 4, 100, None, None) == B.TTE_E_UNSUPPORTED  # dim not a multiple of 16
    assert lib.tte_similarity(None, -1, 128, None, None) == B.TTE_E_INVALID
    assert lib.tte_similarity(None, 0, 128, None, None) == B.TTE_OK  # empty: no-op
    assert lib.tte_similarity(None, 3, 128, None, None) == B.TTE_E_INVALID  # NULL buffers
    assert lib.tte_embed_tokens(None, None, 0, None, 0, None, None) == B.TTE_E_INVALID  # NULL model
