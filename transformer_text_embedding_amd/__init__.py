"""MI355X-native packed text-embedding encoder (ModernBERT layout).

`Model` holds device copies of the weights (torch tensors), a workspace and a
handle of the C library; `Model.embed_pack` runs one pack through the HIP
kernels on a torch stream; `Model.embed` packs whole texts and returns numpy
vectors.  All arithmetic happens in libtte.so (see include/tte.h).
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from . import binding as B

__all__ = ["Model", "make_config", "similarity", "B"]


def similarity(emb_dev, stream=None):
    """Cosine-similarity matrix fp32 [n, n] of unit vectors emb_dev fp32
    [n, dim] (device tensor; dim a multiple of 16)."""
    import torch
    n, dim = emb_dev.shape
    out = torch.empty((n, n), dtype=torch.float32, device=emb_dev.device)
    st = stream.cuda_stream if stream is not None else torch.cuda.current_stream(emb_dev.device).cuda_stream
    B.tte_similarity(emb_dev.data_ptr() if n else 0, n, dim, out.data_ptr() if n else 0, st)
    return out


def make_config(spec, max_tokens: int, max_text_len: int, max_texts: Optional[int] = None,
                split_k: bool = False, graph: bool = False) -> B.tte_config:
    """tte_config from a dict / dataclass with the encoder's shape fields.
    split_k sets TTE_FLAG_SPLIT_K (lower latency of one call on an idle GPU,
    lower throughput under concurrent calls); graph sets TTE_FLAG_GRAPH
    (per-shape HIP-graph replay on non-null streams)."""
    d = spec if isinstance(spec, dict) else spec.as_dict()
    return B.tte_config(
        vocab=d["vocab"], hidden=d["hidden"], n_heads=d["heads"], head_dim=d["head_dim"],
        intermediate=d["intermediate"], n_layers=d["layers"], global_every=d.get("global_every", 3),
        window=d.get("window", 64), rope_base_global=d.get("rope_base_global", 160000.0),
        rope_base_local=d.get("rope_base_local", 10000.0), ln_eps=d.get("ln_eps", 1e-5),
        max_tokens=max_tokens, max_text_len=max_text_len,
        max_texts=max_texts if max_texts is not None else max_tokens,
        precision=B.PRECISIONS[d["precision"]],
        flags=(B.TTE_FLAG_SPLIT_K if split_k else 0) | (B.TTE_FLAG_GRAPH if graph else 0))


class Model:
    """One encoder instance on one device and stream.

    weights: storage-format arrays (numpy) as produced by tte_inputs
    (fp32 arrays; uint16 bf16 bits under *_bf16 keys; int8 codes and fp32
    scales under *_q / *_s keys).  They are copied to the device once.
    """

    def __init__(self, spec, weights: dict, max_tokens: int = 2048, max_text_len: Optional[int] = None,
                 max_texts: Optional[int] = None, device: str = "cuda:0", shared_from: "Model" = None,
                 split_k: bool = False, graph: bool = False):
        import torch
        self.torch = torch
        B.lib()
        self.device = torch.device(device)
        self.spec = spec if isinstance(spec, dict) else spec.as_dict()
        self.cfg = make_config(self.spec, max_tokens, max_text_len or max_tokens, max_texts, split_k, graph)
        self.precision = self.spec["precision"]
        if shared_from is not None:
            self._keep = shared_from._keep
            self._w = shared_from._w
            self._layers = shared_from._layers
        else:
            self._upload(weights)
        self.ws_bytes = B.tte_workspace_size(self.cfg)
        self.workspace = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=self.device)
        base = self.workspace.data_ptr()
        self._ws_ptr = (base + 255) // 256 * 256
        with torch.cuda.device(self.device):
            self.handle = B.tte_create(self.cfg, self._w, self._ws_ptr, self.ws_bytes)

    # -- weights -------------------------------------------------------------
    def _dev(self, arr):
        t = self.torch
        a = np.ascontiguousarray(arr)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        x = t.from_numpy(a).to(self.device)
        self._keep.append(x)
        return x.data_ptr()

    def _mat(self, d: dict, name: str):
        if self.precision == "fp32":
            return self._dev(d[name]), None
        if self.precision == "bf16":
            return self._dev(d[name + "_bf16"]), None
        if self.precision == "int4" and name != "tok_emb":
            return self._dev(d[name + "_q4"]), self._dev(d[name + "_q4m"])
        return self._dev(d[name + "_q"]), self._dev(d[name + "_s"])

    def _upload(self, w: dict):
        self._keep = []
        emb, emb_s = self._mat(w, "tok_emb")
        layers = (B.tte_layer_weights * self.cfg.n_layers)()
        for l in range(self.cfg.n_layers):
            L = w["layers"][l]
            lw = layers[l]
            lw.wqkv, lw.wqkv_scale = self._mat(L, "wqkv")
            lw.wo, lw.wo_scale = self._mat(L, "wo")
            lw.wi, lw.wi_scale = self._mat(L, "wi")
            lw.wo2, lw.wo2_scale = self._mat(L, "wo2")
            lw.attn_norm = self._dev(L["attn_norm"]) if L.get("attn_norm") is not None else None
            lw.mlp_norm = self._dev(L["mlp_norm"])
        self._layers = layers
        self._w = B.tte_weights(tok_emb=emb, tok_emb_scale=emb_s, emb_norm=self._dev(w["emb_norm"]),
                                final_norm=self._dev(w["final_norm"]), layers=layers)

    # -- calls ---------------------------------------------------------------
    def _stream(self, stream):
        if stream is None:
            stream = self.torch.cuda.current_stream(self.device)
        return stream.cuda_stream

    def embed_pack(self, ids_dev, offsets: Sequence[int], out=None, stream=None):
        """Enqueue one pack; returns the fp32 [B, H] device tensor (valid once
        the stream reaches it)."""
        t = self.torch
        n_texts = len(offsets) - 1
        if out is None:
            out = t.empty((max(n_texts, 0), self.cfg.hidden), dtype=t.float32, device=self.device)
        B.tte_embed(self.handle, ids_dev.data_ptr() if ids_dev.numel() else 0, int(ids_dev.numel()), offsets,
                    out.data_ptr() if out.numel() else 0, self._stream(stream))
        return out

    def embed_tokens(self, ids_dev, offsets: Sequence[int], out=None, stream=None):
        """Enqueue one pack; returns the per-token output states, fp32 [T, H]
        (device; the final LayerNorm of every token, no pooling)."""
        t = self.torch
        T = int(ids_dev.numel())
        if out is None:
            out = t.empty((T, self.cfg.hidden), dtype=t.float32, device=self.device)
        B.tte_embed_tokens(self.handle, ids_dev.data_ptr() if T else 0, T, offsets, out.data_ptr() if T else 0,
                           self._stream(stream))
        return out

    def trace(self, ids_dev, offsets, n_dump: int, stream=None):
        """Residual-stream states after the embedding norm and each of the
        first n_dump layers: fp32 [n_dump + 1, T, H] (device)."""
        t = self.torch
        T = int(ids_dev.numel())
        states = t.empty((n_dump + 1, T, self.cfg.hidden), dtype=t.float32, device=self.device)
        out = None
        if n_dump == self.cfg.n_layers:
            out = t.empty((len(offsets) - 1, self.cfg.hidden), dtype=t.float32, device=self.device)
        B.tte_embed_trace(self.handle, ids_dev.data_ptr(), T, offsets, out.data_ptr() if out is not None else 0,
                          states.data_ptr(), n_dump, self._stream(stream))
        return states, out

    def embed(self, texts: List[Sequence[int]], budget: Optional[int] = None) -> np.ndarray:
        """Unit vectors [len(texts), H] (numpy fp32).  Whole texts are packed
        greedily up to `budget` tokens (default max_tokens); a text is never
        split across passes."""
        t = self.torch
        budget = budget or self.cfg.max_tokens
        for x in texts:
            if len(x) == 0 or len(x) > min(budget, self.cfg.max_text_len):
                raise ValueError("every text needs 1 .. min(budget, max_text_len) tokens")
            if min(x) < 0 or max(x) >= self.cfg.vocab:
                raise ValueError("token id out of range")
        outs, cur, cur_len = [], [], 0
        packs = []
        for x in texts:
            if cur and (cur_len + len(x) > budget or len(cur) == self.cfg.max_texts):
                packs.append(cur)
                cur, cur_len = [], 0
            cur.append(x)
            cur_len += len(x)
        if cur:
            packs.append(cur)
        for p in packs:
            offsets = np.concatenate([[0], np.cumsum([len(x) for x in p])]).astype(np.int32)
            ids = t.from_numpy(np.concatenate([np.asarray(x, np.int32) for x in p])).to(self.device)
            outs.append(self.embed_pack(ids, offsets))
        t.cuda.synchronize(self.device)
        if not outs:
            return np.zeros((0, self.cfg.hidden), np.float32)
        return t.cat(outs).cpu().numpy()

    def close(self):
        if getattr(self, "handle", None):
            B.tte_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
