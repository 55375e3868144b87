"""Route histogram, exclusive scan and stable pack (oracle side).

exllamav3 #284 (Summary; Relationship to #246) describes a fused route
histogram, scan and stable packing of (row, expert) pairs; (API contract)
num_active counts every non-empty expert and is only a hint; (Validation)
route IDs are int32 or int64 and weights fp16, bf16 or fp32.

Reading used (the pages give no formula): pair q = r * topk + j in row-major
order; IDs outside [0, E) are dropped and counted; the packed position of a
kept pair is offset[e] + #{q' < q kept with the same expert}. The result is
unique, so the kernels must match it bit for bit.

This is a plain sequential counting pass; ``tests`` pin it against numpy's
stable argsort, bincount and cumsum.
"""

import numpy as np


def route_pack(ids, weights, num_experts):
    """Return a dict with count, offset, pair_of_pos, weight_of_pos,
    pos_of_pair, num_active and dropped, following the reading above.

    ``weights`` must already be the exact float values of the routing
    weights (fp16/bf16/fp32 inputs widen exactly).
    """
    ids = np.asarray(ids).reshape(-1)
    w = np.asarray(weights, dtype=np.float64).reshape(-1)
    pairs = ids.shape[0]
    E = int(num_experts)

    count = [0] * E
    dropped = 0
    for q in range(pairs):
        e = int(ids[q])
        if 0 <= e < E:
            count[e] += 1
        else:
            dropped += 1

    offset = [0] * (E + 1)
    for e in range(E):
        offset[e + 1] = offset[e] + count[e]

    pair_of_pos = np.full(pairs, -1, dtype=np.int64)
    weight_of_pos = np.zeros(pairs, dtype=np.float64)
    pos_of_pair = np.full(pairs, -1, dtype=np.int64)
    cursor = list(offset[:E])
    for q in range(pairs):
        e = int(ids[q])
        if not (0 <= e < E):
            continue
        p = cursor[e]
        cursor[e] += 1
        pair_of_pos[p] = q
        weight_of_pos[p] = w[q]
        pos_of_pair[q] = p

    return {
        "count": np.array(count, dtype=np.int64),
        "offset": np.array(offset, dtype=np.int64),
        "pair_of_pos": pair_of_pos,
        "weight_of_pos": weight_of_pos,
        "pos_of_pair": pos_of_pair,
        "num_active": int(sum(1 for c in count if c > 0)),
        "dropped": int(dropped),
    }
