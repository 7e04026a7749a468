"""The TTE_LOG and TTE_DEBUG switches of the library (read from the
environment once per process, so every case runs in a fresh interpreter).
CPU cases: the log line of a refused configuration, and the workspace
guards TTE_DEBUG adds.  GPU cases: a debug pass agrees with the oracle, and
an out-of-range token id is refused before anything is enqueued (without
the switch it is clamped on the device)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

HOST = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
import tte_inputs as ti
from transformer_text_embedding_amd import B, make_config
c = make_config(ti.workload("full_bf16_packs2048")["cfg"], max_tokens=2048, max_text_len=512, max_texts=256)
ws = B.tte_workspace_size(c)
c.head_dim = 32
st = B.lib().tte_workspace_size(c, None)
print(json.dumps({"ws": ws, "bad_status": st}))
"""

GPU = r"""
import json, sys
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + "/tests")
import numpy as np
import oracle
import tte_inputs as ti
from gpu_util import dev, host
from transformer_text_embedding_amd import B, Model
cfg = ti.workload("tiny_fp32")["cfg"]
w = ti.storage_weights(cfg, ti.make_fp32_weights(cfg))
m = Model(cfg, w, max_tokens=512, max_text_len=256, max_texts=16)
pack = ti.random_pack(np.random.default_rng(5), [8, 40, 130], cfg.vocab)
got = host(m.embed_pack(dev(pack.ids), pack.offsets))
ref = oracle.encode(cfg.as_dict(), w, pack.ids, pack.offsets)
bad = pack.ids.copy(); bad[17] = cfg.vocab + 3
try:
    m.embed_pack(dev(bad), pack.offsets)
    refused = ""
except B.TteError as e:
    refused = str(e)
m.close()
print(json.dumps({"maxdiff": float(np.abs(got - ref).max()), "refused": refused}))
"""


def _run(code, env_extra, timeout=300):
    env = {k: v for k, v in os.environ.items() if k not in ("TTE_LOG", "TTE_DEBUG")}
    env.update(env_extra)
    r = subprocess.run([sys.executable, "-c", code, ROOT], capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, r.stderr[-2000:]
    return json.loads(r.stdout.strip().splitlines()[-1]), r.stderr


def test_log_reports_refused_config():
    out, err = _run(HOST, {"TTE_LOG": "1"})
    assert out["bad_status"] != 0
    assert "[tte] error" in err and "head_dim" in err
    _, quiet = _run(HOST, {})
    assert "[tte]" not in quiet


def test_debug_adds_a_guard_after_every_workspace_region():
    plain, _ = _run(HOST, {})
    guarded, _ = _run(HOST, {"TTE_DEBUG": "1"})
    assert guarded["ws"] - plain["ws"] == 15 * 256  # 15 regions, 256 guard bytes each


@pytest.mark.gpu
def test_debug_pass_matches_oracle_and_refuses_bad_ids():
    out, err = _run(GPU, {"TTE_DEBUG": "1", "TTE_LOG": "1"})
    assert out["maxdiff"] <= 1e-4
    assert "outside [0, vocab)" in out["refused"] and "index 17" in out["refused"]
    assert "[tte] create:" in err and "(with guards)" in err and "[tte] pass:" in err
