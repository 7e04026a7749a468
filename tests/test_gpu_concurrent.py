"""Concurrent use of the library the way bench.py drives it: four models
over one shared copy of the weights, each on its own stream and driven by
its own host thread (the library calls release the interpreter lock, so the
four threads enqueue at once).  Every pack's vectors must equal, bit for
bit, those of the same pack run alone on one model: packs never interact,
and every kernel is deterministic."""
import threading

import numpy as np
import pytest

import tte_inputs as ti
from gpu_util import dev, host, say, sync, torch
from transformer_text_embedding_amd import Model

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("graph", [False, True])
def test_four_threads_four_streams(graph):
    t = torch()
    name = "full_bf16_packs2048"
    cfg = ti.workload(name)["cfg"]
    w = ti.cached_storage_weights(cfg)
    packs = ti.make_packs(name)[:12]
    kw = dict(max_tokens=2048, max_text_len=2048, max_texts=256)
    alone = Model(cfg, w, **kw)
    models = [Model(cfg, None, shared_from=alone, graph=graph, **kw) for _ in range(4)]
    try:
        ids = [dev(p.ids) for p in packs]
        ref = [host(alone.embed_pack(ids[i], p.offsets)) for i, p in enumerate(packs)]
        streams = [t.cuda.Stream() for _ in range(4)]
        rounds = 3  # with graph replay: eager, captured, replayed
        outs = [[t.empty((p.n_texts, cfg.hidden), dtype=t.float32, device=ids[0].device) for p in packs]
                for _ in range(rounds)]
        sync()
        errors = []

        def worker(k):
            try:
                for r in range(rounds):
                    for i in range(k, len(packs), 4):
                        models[k].embed_pack(ids[i], packs[i].offsets, out=outs[r][i], stream=streams[k])
            except Exception as e:  # reported on the main thread
                errors.append(e)

        threads = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        sync()
        assert not errors, errors
        for r in range(rounds):
            for i in range(len(packs)):
                assert np.array_equal(host(outs[r][i]), ref[i]), f"round {r}, pack {i} differs from the pack alone"
        say(f"  {rounds * len(packs)} concurrent calls on 4 threads / 4 streams bit-identical (graph={graph})")
    finally:
        for m in models:
            m.close()
        alone.close()
