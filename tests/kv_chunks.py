"""The dK / dV pass's work split, written out from the planner's stated rule,
so tests can tell which KV tiles go through the workspace slots and the
ordered reduce (``test_planner_parity`` checks it against the library's slot
count)."""
import numpy as np

import long_context_sequence_doc_amd as sap

TARGET_CHUNKS, MIN_CHUNK = 128, 8


def kv_chunks(plan) -> dict:
    """Partner counts of the work items of each touched KV tile: the tile's
    partner Q tiles (ascending index) are cut where the index crosses a
    multiple of per = max(8, ceil(n_tiles / 128)); a piece shorter than
    per // 2 joins the next one, and a short last piece the one before. A tile
    with more than one piece is split (one workspace slot per piece)."""
    q, k, _ = sap.sap_plan_tiles(plan)
    per = max(MIN_CHUNK, -(-len(q) // TARGET_CHUNKS))
    out = {}
    for t in np.unique(k):
        qs = np.sort(q[k == t])
        bins = qs // per
        runs, start = [], 0
        for i in range(1, len(qs) + 1):
            if i < len(qs) and bins[i] == bins[i - 1]:
                continue
            if runs and runs[-1] < per // 2:
                runs[-1] += i - start
            else:
                runs.append(i - start)
            start = i
        if len(runs) > 1 and runs[-1] < per // 2:
            last = runs.pop()
            runs[-1] += last
        out[int(t)] = runs
    return out


def n_slots(plan) -> int:
    return sum(len(r) for r in kv_chunks(plan).values() if len(r) > 1)
