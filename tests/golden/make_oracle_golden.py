"""Write the oracle's expected embeddings for the full-size workloads.

Usage: python tests/golden/make_oracle_golden.py [workload ... | spread]

Calls only the CPU oracle (oracle/) on the seeded inputs of tte_inputs, and
stores the fp64 unit vectors with fingerprints of the inputs they came from
in tests/golden/<workload>.npz (numpy, no pickle).  GPU tests compare the HIP
library against these files and recompute with the oracle if a fingerprint
does not match.  Each full-size workload is reduced to packs/texts the oracle
finishes in minutes: the packing paragraph of the tensai page's section
何が動くか makes every text's vector independent of what it is packed with.
"""
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import tte_inputs as ti  # noqa: E402

# workload -> list of (pack index, text indices or None for the whole pack)
SELECTION = {
    "full_fp32_957": [(0, None)],
    "full_bf16_packs2048": [(0, None), (1, None)],
    "full_bf16_4x4096": [(0, [0, 1, 2, 3])],
    "full_int8_packs2048": [(0, None), (1, None)],
    "full_int4_packs2048": [(0, None)],
}


def fingerprint(cfg, w, pack, texts):
    h = hashlib.sha256()
    h.update(repr(sorted(cfg.as_dict().items())).encode())
    for key in sorted(k for k in w if isinstance(w[k], np.ndarray)):
        h.update(np.ascontiguousarray(w[key]).tobytes()[:1 << 20])
    for L in (w["layers"][0], w["layers"][-1]):
        for key in sorted(k for k, v in L.items() if isinstance(v, np.ndarray)):
            h.update(np.ascontiguousarray(L[key]).tobytes()[:1 << 20])
    h.update(pack.ids.tobytes())
    h.update(pack.offsets.tobytes())
    h.update(repr(texts).encode())
    return h.hexdigest()


def expected(name, pack_index, texts):
    spec = ti.workload(name)
    cfg = spec["cfg"]
    w = ti.cached_storage_weights(cfg)
    pack = ti.make_packs(name)[pack_index]
    if texts is None:
        emb = oracle.encode(cfg.as_dict(), w, pack.ids, pack.offsets)
    else:
        emb = np.stack([oracle.encode(cfg.as_dict(), w, pack.text(b), [0, len(pack.text(b))])[0] for b in texts])
    return emb, fingerprint(cfg, w, pack, texts)


# integer workloads -> pack whose fp32-rounding spread is stored: how far the
# oracle's own pass moves when every intermediate is rounded to fp32, per
# layer (the integer paths' 7-bit codes amplify such roundings)
SPREAD = {"full_int8_packs2048": 0, "full_int4_packs2048": 0}
SPREAD_FILE = os.path.join(HERE, "rounding_spread.npz")


def write_spreads():
    sys.path.insert(0, os.path.dirname(HERE))
    from parity_bounds import rounding_spread  # composed from oracle functions only
    arrays = {}
    for name, pi in SPREAD.items():
        t0 = time.time()
        cfg = ti.workload(name)["cfg"]
        w = ti.cached_storage_weights(cfg)
        pack = ti.make_packs(name)[pi]
        per_min, per_mean, fin_min, fin_mean = rounding_spread(cfg.as_dict(), w, pack.ids, pack.offsets)
        key = f"{name}_pack{pi}"
        arrays[key + "_min"] = per_min
        arrays[key + "_mean"] = per_mean
        arrays[key + "_final"] = np.array([fin_min, fin_mean])
        arrays[key + "_fp"] = np.frombuffer(fingerprint(cfg, w, pack, None).encode(), np.uint8)
        print(f"{name} pack {pi}: final 1-cos min {fin_min:.3e} mean {fin_mean:.3e} in {time.time() - t0:.1f}s",
              flush=True)
    np.savez(SPREAD_FILE, **arrays)


def main(names):
    if names == ["spread"]:
        write_spreads()
        return
    for name in names:
        arrays = {}
        for pi, texts in SELECTION[name]:
            t0 = time.time()
            emb, fp = expected(name, pi, texts)
            arrays[f"pack{pi}_emb"] = emb
            arrays[f"pack{pi}_texts"] = np.array([-1] if texts is None else texts, np.int64)
            arrays[f"pack{pi}_fp"] = np.frombuffer(fp.encode(), np.uint8)
            print(f"{name} pack {pi}: {emb.shape} in {time.time() - t0:.1f}s", flush=True)
        np.savez(os.path.join(HERE, f"{name}.npz"), **arrays)


if __name__ == "__main__":
    main(sys.argv[1:] or list(SELECTION))
