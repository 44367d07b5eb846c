"""Write the expected page tables of the 24-layer token-budget stream.

Runs only the CPU oracle (oracle.budget) on the seeded raw-score table of the
workload (bounded_kv_cache_stream_amd.synth, input generation only) and stores,
for every layer and every frame, a digest of the page table after that frame's
score-and-compact step and of the kept token ids of the step (if one ran).

    python tests/golden/make_budget_golden.py      # writes budget_l24_f500.json
"""

from __future__ import annotations

import hashlib
import json
import os
import sys
from multiprocessing import Pool

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

OUT = os.path.join(HERE, "budget_l24_f500.json")
WORKLOAD = 4


def table_digest(entries) -> str:
    """Digest of a page table given as (page_id, frame, length) triples."""
    s = ";".join(f"{int(p)}:{int(f)}:{int(n)}" for p, f, n in entries)
    return hashlib.sha256(s.encode()).hexdigest()[:16]


def ids_digest(ids) -> str:
    s = ",".join(str(int(i)) for i in ids)
    return hashlib.sha256(s.encode()).hexdigest()[:16]


def simulate_layer(layer: int, frames: int | None = None, record_ids_at=()):
    from bounded_kv_cache_stream_amd import synth
    from oracle import budget
    w = synth.WORKLOADS[WORKLOAD]
    T, B, F, L = w["tokens"], w["budget"], w["frames"], w["layers"]
    F = frames or F
    scores = synth.raw_scores(WORKLOAD, w["frames"] * T, L)
    c = budget.BudgetCache(layer, T, B, w["frames"], window=w["clces_window"], lam=w["lam"])
    tables, keeps, attended = [], [], {}
    for t in range(F):
        c.append(t)
        if t in record_ids_at:
            attended[t] = c.all_ids().copy()
        ran = c.score_and_compact(scores)
        tables.append(table_digest(c.page_table()))
        keeps.append(ids_digest(c.last["keep_ids"]) if ran else None)
    return layer, tables, keeps, attended


def _one(layer):
    l, tables, keeps, _ = simulate_layer(layer)
    print(f"layer {l} done", flush=True)
    return l, tables, keeps


def main():
    from bounded_kv_cache_stream_amd import synth
    L = synth.WORKLOADS[WORKLOAD]["layers"]
    with Pool(min(8, os.cpu_count() or 1)) as pool:
        res = pool.map(_one, range(L))
    out = {"workload": synth.WORKLOADS[WORKLOAD]["name"],
           "note": "written by tests/golden/make_budget_golden.py from oracle.budget only",
           "tables": {str(l): t for l, t, _ in res}, "keeps": {str(l): k for l, _, k in res}}
    with open(OUT, "w") as f:
        json.dump(out, f, separators=(",", ":"))
    print(OUT)


if __name__ == "__main__":
    main()
