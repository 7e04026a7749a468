"""ctypes binding of libtte.so: the C ABI of include/tte.h, same names,
argument marshalling only.  Every step of the pass runs in the library's HIP
kernels; PyTorch supplies device memory and streams.  There is no fallback:
if the library is missing, loading raises."""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_char_p, c_double, c_float, c_int8, c_int32, c_int64, c_size_t, c_uint32, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
# TTE_LIBRARY: path of another build of the library (e.g. a variant to
# compare against); the package's own libtte.so otherwise
LIB_PATH = os.environ.get("TTE_LIBRARY") or os.path.join(PKG, "libtte.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "tte.h")

TTE_OK, TTE_E_INVALID, TTE_E_UNSUPPORTED, TTE_E_NOMEM, TTE_E_DEVICE = range(5)
STATUS_NAMES = {0: "TTE_OK", 1: "TTE_E_INVALID", 2: "TTE_E_UNSUPPORTED", 3: "TTE_E_NOMEM", 4: "TTE_E_DEVICE"}
TTE_FP32, TTE_BF16, TTE_INT8, TTE_INT4 = 0, 1, 2, 3
TTE_FLAG_SPLIT_K, TTE_FLAG_GRAPH = 1, 2
PRECISIONS = {"fp32": TTE_FP32, "bf16": TTE_BF16, "int8": TTE_INT8, "int4": TTE_INT4}
TTE_OUT_F32, TTE_OUT_BF16, TTE_OUT_I8 = 0, 1, 2
TTE_EPI_STORE, TTE_EPI_RESIDUAL, TTE_EPI_GEGLU = 0, 1, 2
KERNEL_CLASSES = ["embed", "norm", "quant", "gemm_qkv", "attn_global", "attn_local", "gemm_o", "gemm_geglu",
                  "gemm_o2", "pool"]
TTE_K_COUNT = len(KERNEL_CLASSES)


class tte_config(ctypes.Structure):
    _fields_ = [("vocab", c_int32), ("hidden", c_int32), ("n_heads", c_int32), ("head_dim", c_int32),
                ("intermediate", c_int32), ("n_layers", c_int32), ("global_every", c_int32), ("window", c_int32),
                ("rope_base_global", c_float), ("rope_base_local", c_float), ("ln_eps", c_float),
                ("max_tokens", c_int32), ("max_text_len", c_int32), ("max_texts", c_int32), ("precision", c_int32),
                ("flags", c_int32)]


class tte_layer_weights(ctypes.Structure):
    _fields_ = [("wqkv", c_void_p), ("wqkv_scale", c_void_p), ("wo", c_void_p), ("wo_scale", c_void_p),
                ("wi", c_void_p), ("wi_scale", c_void_p), ("wo2", c_void_p), ("wo2_scale", c_void_p),
                ("attn_norm", c_void_p), ("mlp_norm", c_void_p)]


class tte_weights(ctypes.Structure):
    _fields_ = [("tok_emb", c_void_p), ("tok_emb_scale", c_void_p), ("emb_norm", c_void_p),
                ("final_norm", c_void_p), ("layers", POINTER(tte_layer_weights))]


_SIGS = {
    "tte_workspace_size": (c_int32, [POINTER(tte_config), POINTER(c_size_t)]),
    "tte_check_pack": (c_int32, [POINTER(tte_config), c_int32, POINTER(c_int32), c_int32]),
    "tte_create": (c_int32, [POINTER(tte_config), POINTER(tte_weights), c_void_p, c_size_t, POINTER(c_void_p)]),
    "tte_embed": (c_int32, [c_void_p, c_void_p, c_int32, POINTER(c_int32), c_int32, c_void_p, c_void_p]),
    "tte_embed_trace": (c_int32, [c_void_p, c_void_p, c_int32, POINTER(c_int32), c_int32, c_void_p, c_void_p,
                                  c_int32, c_void_p]),
    "tte_destroy": (c_int32, [c_void_p]),
    "tte_last_error": (c_char_p, []),
    "tte_op_layernorm": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_float, c_int32, c_void_p, c_void_p,
                                   c_void_p]),
    "tte_op_quant7": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    "tte_op_gemm": (c_int32, [c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                              c_void_p, c_int32, c_void_p]),
    "tte_embed_tokens": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p]),
    "tte_similarity": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
    "tte_op_gemm_splitk": (c_int32, [c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                     c_int32, c_void_p, c_void_p]),
    "tte_op_resid_ln": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_int32, c_float, c_int32, c_void_p,
                                  c_void_p, c_void_p]),
    "tte_op_attention": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, POINTER(c_int32), c_int32, c_void_p,
                                   c_void_p]),
    "tte_op_qkv": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int32, POINTER(c_int32), c_int32, c_void_p,
                             c_void_p, c_void_p]),
    "tte_op_pool": (c_int32, [c_void_p, c_void_p, c_int32, POINTER(c_int32), c_int32, c_void_p, c_void_p]),
    "tte_op_pool_static": (c_int32, [c_void_p, c_void_p, c_int32, POINTER(c_int32), c_int32, c_void_p, c_void_p]),
    "tte_profile_start": (c_int32, [c_void_p, c_uint32, c_int32]),
    "tte_profile_stop": (c_int32, [c_void_p, POINTER(c_double), POINTER(c_int64)]),
    "tte_graph_stats": (c_int32, [c_void_p, POINTER(c_int32), POINTER(c_int32), POINTER(c_int64)]),
}

_lib = None


class TteError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m transformer_text_embedding_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().tte_last_error().decode()


def check(status: int) -> None:
    if status != TTE_OK:
        raise TteError(status, last_error())


def header_functions(path: str = HEADER):
    """Names of the functions include/tte.h declares."""
    text = open(path).read()
    return re.findall(r"^\s*(?:tte_status|const char\s*\*)\s*(tte_\w+)\s*\(", text, flags=re.M)


def int32_array(values):
    arr = (c_int32 * len(values))(*[int(v) for v in values])
    return arr


# thin same-name wrappers ---------------------------------------------------

def tte_workspace_size(cfg: tte_config) -> int:
    n = c_size_t(0)
    check(lib().tte_workspace_size(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def tte_check_pack(cfg: tte_config, n_tokens: int, offsets) -> int:
    arr = int32_array(offsets) if offsets is not None else None
    n_texts = max(len(offsets) - 1, 0) if offsets is not None else 0
    return lib().tte_check_pack(ctypes.byref(cfg), n_tokens, arr, n_texts)


def tte_create(cfg: tte_config, w: tte_weights, d_ws: int, ws_bytes: int) -> int:
    out = c_void_p(0)
    check(lib().tte_create(ctypes.byref(cfg), ctypes.byref(w), c_void_p(d_ws), ws_bytes, ctypes.byref(out)))
    return out.value


def tte_embed(model: int, d_ids: int, n_tokens: int, offsets, d_out: int, stream: int) -> None:
    arr = int32_array(offsets)
    check(lib().tte_embed(c_void_p(model), c_void_p(d_ids), n_tokens, arr, len(offsets) - 1, c_void_p(d_out),
                          c_void_p(stream)))


def tte_embed_trace(model: int, d_ids: int, n_tokens: int, offsets, d_out: int, d_states: int, n_dump: int,
                    stream: int) -> None:
    arr = int32_array(offsets)
    check(lib().tte_embed_trace(c_void_p(model), c_void_p(d_ids), n_tokens, arr, len(offsets) - 1,
                                c_void_p(d_out) if d_out else None, c_void_p(d_states), n_dump, c_void_p(stream)))


def tte_destroy(model: int) -> None:
    check(lib().tte_destroy(c_void_p(model)))


def tte_op_layernorm(d_x: int, d_gamma: int, rows: int, width: int, eps: float, out_kind: int, d_out: int,
                     d_scale: int, stream: int) -> None:
    check(lib().tte_op_layernorm(c_void_p(d_x), c_void_p(d_gamma) if d_gamma else None, rows, width, eps, out_kind,
                                 c_void_p(d_out), c_void_p(d_scale) if d_scale else None, c_void_p(stream)))


def tte_op_quant7(d_x: int, rows: int, width: int, d_q: int, d_scale: int, stream: int) -> None:
    check(lib().tte_op_quant7(c_void_p(d_x), rows, width, c_void_p(d_q), c_void_p(d_scale), c_void_p(stream)))


def tte_op_gemm(precision: int, epilogue: int, d_a: int, d_a_scale: int, d_w: int, d_w_scale: int, M: int, N: int,
                K: int, d_c: int, out_kind: int, stream: int) -> None:
    check(lib().tte_op_gemm(precision, epilogue, c_void_p(d_a), c_void_p(d_a_scale) if d_a_scale else None,
                            c_void_p(d_w), c_void_p(d_w_scale) if d_w_scale else None, M, N, K, c_void_p(d_c),
                            out_kind, c_void_p(stream)))


def tte_embed_tokens(model: int, d_ids: int, n_tokens: int, offsets, d_out_tokens: int, stream: int) -> None:
    arr = int32_array(offsets)
    check(lib().tte_embed_tokens(c_void_p(model), c_void_p(d_ids), n_tokens, arr, len(offsets) - 1,
                                 c_void_p(d_out_tokens), c_void_p(stream)))


def tte_similarity(d_emb: int, n: int, dim: int, d_sim: int, stream: int) -> None:
    check(lib().tte_similarity(c_void_p(d_emb), n, dim, c_void_p(d_sim), c_void_p(stream)))


def tte_op_gemm_splitk(precision: int, d_a: int, d_a_scale: int, d_w: int, d_w_scale: int, M: int, N: int, K: int,
                       splits: int, d_partials: int, stream: int) -> None:
    check(lib().tte_op_gemm_splitk(precision, c_void_p(d_a), c_void_p(d_a_scale) if d_a_scale else None, c_void_p(d_w),
                                   c_void_p(d_w_scale) if d_w_scale else None, M, N, K, splits, c_void_p(d_partials),
                                   c_void_p(stream)))


def tte_op_resid_ln(d_x: int, d_partials: int, splits: int, d_gamma: int, rows: int, width: int, eps: float,
                    out_kind: int, d_out: int, d_scale: int, stream: int) -> None:
    check(lib().tte_op_resid_ln(c_void_p(d_x), c_void_p(d_partials) if d_partials else None, splits,
                                c_void_p(d_gamma) if d_gamma else None, rows, width, eps, out_kind,
                                c_void_p(d_out) if d_out else None, c_void_p(d_scale) if d_scale else None,
                                c_void_p(stream)))


def tte_op_attention(model: int, layer: int, d_qkv: int, n_tokens: int, offsets, d_o: int, stream: int) -> None:
    arr = int32_array(offsets)
    check(lib().tte_op_attention(c_void_p(model), layer, c_void_p(d_qkv), n_tokens, arr, len(offsets) - 1,
                                 c_void_p(d_o), c_void_p(stream)))


def tte_op_qkv(model: int, layer: int, d_a: int, d_a_scale: int, n_tokens: int, offsets, d_qk: int, d_vt: int,
               stream: int) -> None:
    arr = int32_array(offsets)
    check(lib().tte_op_qkv(c_void_p(model), layer, c_void_p(d_a), c_void_p(d_a_scale) if d_a_scale else None,
                           n_tokens, arr, len(offsets) - 1, c_void_p(d_qk), c_void_p(d_vt), c_void_p(stream)))


def tte_op_pool(model: int, d_x: int, n_tokens: int, offsets, d_out: int, stream: int) -> None:
    arr = int32_array(offsets)
    check(lib().tte_op_pool(c_void_p(model), c_void_p(d_x), n_tokens, arr, len(offsets) - 1, c_void_p(d_out),
                            c_void_p(stream)))


def tte_op_pool_static(model: int, d_x: int, n_tokens: int, offsets, d_out: int, stream: int) -> None:
    arr = int32_array(offsets)
    check(lib().tte_op_pool_static(c_void_p(model), c_void_p(d_x), n_tokens, arr, len(offsets) - 1, c_void_p(d_out),
                                   c_void_p(stream)))


def tte_profile_start(model: int, class_mask: int, max_launches: int) -> None:
    check(lib().tte_profile_start(c_void_p(model), class_mask, max_launches))


def tte_graph_stats(model: int):
    """(shapes recorded, graphs instantiated, graph launches) of a model."""
    a, b, c = c_int32(0), c_int32(0), c_int64(0)
    check(lib().tte_graph_stats(c_void_p(model), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def tte_profile_stop(model: int):
    ms = (c_double * TTE_K_COUNT)()
    n = (c_int64 * TTE_K_COUNT)()
    check(lib().tte_profile_stop(c_void_p(model), ms, n))
    return {KERNEL_CLASSES[k]: (ms[k], n[k]) for k in range(TTE_K_COUNT)}
