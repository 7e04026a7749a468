"""HIP-graph replay of the pass (TTE_FLAG_GRAPH; the tensai batching page
keeps a pool of graphs keyed by batch size, here keyed by pack shape): the
first call of a shape runs eagerly, the second captures and replays, later
ones replay.  Every call is compared bit for bit with the same pack run by
a model without the flag, each call with its own freshly allocated id and
output buffers (the graph reads them from device memory at run time), with
eager work and synchronisations between replays."""
import numpy as np
import pytest

import tte_inputs as ti
from gpu_util import dev, host, say, sync, torch
from transformer_text_embedding_amd import B, Model

pytestmark = pytest.mark.gpu


def _check_replays(cfg, w, shapes, max_tokens, rounds=3):
    t = torch()
    eager = Model(cfg, w, max_tokens=max_tokens, max_text_len=max_tokens, max_texts=256)
    graph = Model(cfg, None, max_tokens=max_tokens, max_text_len=max_tokens, max_texts=256, shared_from=eager,
                  graph=True)
    try:
        rng = np.random.default_rng(5)
        # two packs per shape: same lengths, different ids
        packs = [ti.random_pack(rng, L, cfg.vocab) for L in shapes for _ in range(2)]
        ref_pool = [host(eager.embed_pack(dev(p.ids), p.offsets)) for p in packs]
        ref_tok = [host(eager.embed_tokens(dev(p.ids), p.offsets)) for p in packs[:2]]
        s = t.cuda.Stream()
        keep = []
        results = []
        order = [i for r in range(rounds) for i in range(len(packs))]
        with t.cuda.stream(s):
            for n, i in enumerate(order):
                ids = dev(packs[i].ids)
                out = graph.embed_pack(ids, packs[i].offsets, stream=s)
                keep.append(ids)
                results.append((i, out))
                # unrelated eager work on the same stream between calls
                junk = t.randn(64, 64, device=ids.device) @ t.randn(64, 64, device=ids.device)
                keep.append(junk)
                if n % 3 == 2:
                    sync()
            tok = []
            for r in range(3):
                for i in range(2):
                    ids = dev(packs[i].ids)
                    keep.append(ids)
                    tok.append((i, graph.embed_tokens(ids, packs[i].offsets, stream=s)))
        sync()
        # every shape was captured at its second call and replayed after
        n_shapes = len(shapes)
        shapes_seen, graphs, replays = B.tte_graph_stats(graph.handle)
        assert (shapes_seen, graphs) == (n_shapes + 1, n_shapes + 1), (shapes_seen, graphs)
        assert replays == n_shapes * (2 * rounds - 1) + 5, replays  # per-token: 6 calls, 5 replays
        assert B.tte_graph_stats(eager.handle) == (0, 0, 0)
        for n, (i, out) in enumerate(results):
            assert np.array_equal(host(out), ref_pool[i]), f"pooled call {n} (pack {i}) differs from the eager pass"
        for n, (i, out) in enumerate(tok):
            assert np.array_equal(host(out), ref_tok[i]), f"per-token call {n} (pack {i}) differs"
        # a call on the null stream runs eagerly and agrees too
        assert np.array_equal(host(graph.embed_pack(dev(packs[0].ids), packs[0].offsets)), ref_pool[0])
        say(f"  {len(results)} pooled and {len(tok)} per-token calls bit-identical to the eager pass")
    finally:
        graph.close()
        eager.close()


@pytest.mark.parametrize("precision", ["fp32", "bf16", "int8"])
def test_graph_replay_tiny(precision):
    cfg = ti.workload("tiny_fp32")["cfg"]
    cfg = ti.EncoderConfig(**{**cfg.as_dict(), "precision": precision})
    w = ti.storage_weights(cfg, ti.make_fp32_weights(cfg))
    _check_replays(cfg, w, [[8, 40, 130], [1, 64, 65, 300, 3], [7]], max_tokens=1024)


@pytest.mark.parametrize("name", ["full_bf16_packs2048", "full_int4_packs2048"])
def test_graph_replay_full(name):
    cfg = ti.workload(name)["cfg"]
    w = ti.cached_storage_weights(cfg)
    shapes = [list(np.diff(p.offsets)) for p in ti.make_packs(name)[:2]]
    _check_replays(cfg, w, shapes, max_tokens=2048, rounds=2)


def test_graph_table_drops_least_recently_used():
    """More pack shapes than the table keeps (64): the least recently used
    are dropped, captured graphs among them released after a device
    synchronisation, and a dropped shape starts over (eager, then captured);
    every call still matches the eager pass."""
    t = torch()
    cfg = ti.workload("tiny_fp32")["cfg"]
    w = ti.storage_weights(cfg, ti.make_fp32_weights(cfg))
    eager = Model(cfg, w, max_tokens=512, max_text_len=512, max_texts=64)
    graph = Model(cfg, None, max_tokens=512, max_text_len=512, max_texts=64, shared_from=eager, graph=True)
    try:
        rng = np.random.default_rng(11)
        packs = [ti.random_pack(rng, [3 + i, 5], cfg.vocab) for i in range(70)]  # 70 distinct shapes
        ref = [host(eager.embed_pack(dev(p.ids), p.offsets)) for p in packs]
        s = t.cuda.Stream()
        order = list(range(10)) * 2 + list(range(10, 70)) + [0, 0]
        outs = []
        with t.cuda.stream(s):
            for i in order:
                outs.append((i, graph.embed_pack(dev(packs[i].ids), packs[i].offsets, stream=s)))
        sync()
        # shapes 0-9 captured at their second call (10 graphs); 60 new shapes
        # drop shapes 0-5 with their graphs; shape 0 returns, drops shape 6,
        # runs eagerly, and is captured again at its next call
        assert B.tte_graph_stats(graph.handle) == (64, 4, 11), B.tte_graph_stats(graph.handle)
        for n, (i, out) in enumerate(outs):
            assert np.array_equal(host(out), ref[i]), f"call {n} (pack {i}) differs"
    finally:
        graph.close()
        eager.close()
