"""Write the LM-head top-k goldens ``topk_full.npz`` and ``topk_large.npz``.

For every checked row the file holds the oracle's ranking near the k-th place
(``tests.parity.topk_row_summary``): each id whose bf16 key is at least the k-th
key minus the value tolerance, sorted by (key desc, id asc), with its key.  The
first k entries are the oracle's top-k (``oracle.dflash_oracle.topk_from_keys``,
checked here row by row).  Every value comes from ``oracle/`` on the seeded
inputs of ``workloads/``; a SHA-256 of those inputs is stored with it, so a test
can tell when the generator no longer makes the same bits.

* full:  all 4096 rows of the 256 requests x 16 steps workload (k = 16).
* large: 32 whole requests (every 16th: one per 256-row tile, 512 rows) of the
         tie-heavy large-vocabulary workload (k = 32).

    python -m tests.golden.make_topk_goldens [full] [large]
"""
from __future__ import annotations

import hashlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import dflash_oracle as O  # noqa: E402
import workloads as WL  # noqa: E402
from tests.parity import topk_row_summary  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def input_digest(d) -> str:
    h = hashlib.sha256()
    for name in ("H", "W"):
        h.update(np.ascontiguousarray(d[name]).view(np.uint8))
    return h.hexdigest()


def golden_rows(name: str) -> np.ndarray:
    d = WL.CONFIGS[name]
    S = d["steps"]
    if name == "full":
        return np.arange(d["requests"] * S)
    reqs = np.arange(0, d["requests"], 16)
    return (reqs[:, None] * S + np.arange(S)[None, :]).reshape(-1)


def write(name: str, chunk: int = 512) -> str:
    t0 = time.time()
    d = WL.candidate_inputs(name)
    k, V = d["top_k"], d["vocab"]
    rows = golden_rows(name)
    ids, keys, offsets = [], [], [0]
    for c0 in range(0, len(rows), chunk):
        rr = rows[c0:c0 + chunk]
        kk = O.lm_logit_keys(d["H"], d["W"], d["multiplier"], d["softcap"], rows=rr)
        top_ids, top_vals = O.topk_from_keys(kk, k)
        for t in range(len(rr)):
            sid, sval = topk_row_summary(kk[t], k)
            assert np.array_equal(sid[:k], top_ids[t]) and np.array_equal(sval[:k], top_vals[t].astype(np.float64))
            ids.append(sid.astype(np.int32))
            keys.append(O.f64_to_bf16(sval))
            offsets.append(offsets[-1] + len(sid))
        print(f"{name}: rows {c0 + len(rr)} / {len(rows)}  ({time.time() - t0:.0f} s)", flush=True)
    path = os.path.join(HERE, f"topk_{name}.npz")
    np.savez_compressed(path, rows=rows.astype(np.int64), offsets=np.asarray(offsets, np.int64),
                        ids=np.concatenate(ids), keys=np.concatenate(keys), k=np.int64(k), vocab=np.int64(V),
                        input_sha256=np.array(input_digest(d)))
    print(f"wrote {path}: {len(rows)} rows, {offsets[-1]} entries ({time.time() - t0:.0f} s)", flush=True)
    return path


def load(name: str):
    """(rows, summaries [(ids int64, keys float64)], k, V, input_sha256) of a golden file."""
    z = np.load(os.path.join(HERE, f"topk_{name}.npz"), allow_pickle=False)
    off = z["offsets"]
    ids, keys = z["ids"].astype(np.int64), O.bf16_to_f64(z["keys"])
    summ = [(ids[off[i]:off[i + 1]], keys[off[i]:off[i + 1]]) for i in range(len(off) - 1)]
    return z["rows"], summ, int(z["k"]), int(z["vocab"]), str(z["input_sha256"])


if __name__ == "__main__":
    for n in (sys.argv[1:] or ["full", "large"]):
        write(n)
