"""Dense brute-force attention in pure Python (oracle self-check, test only).

For tiny inputs only.  It works on a dense, already logical K/V (no pages),
builds the full mask matrix explicitly, and sums with ``math.fsum`` (exactly
rounded sums), so it shares neither code nor summation order with the
oracle's matrix-product path.  Agreement between the two pins the oracle's
de-paging, masking, head mapping and softmax.
"""
from __future__ import annotations

import math
from typing import List, Sequence


def dense_attention_bruteforce(q: Sequence, k: Sequence, v: Sequence,
                               seq_len: int, q_len: int, window: int,
                               scale: float, group: int):
    """Attention of one sequence.

    q: [q_len][Hq][D] floats; k, v: [Hkv][seq_len][D] floats (logical order).
    Returns (out [q_len][Hq][D], lse [q_len][Hq]).
    """
    Hq = len(q[0]) if q_len else 0
    D = len(k[0][0]) if seq_len else 0
    # mask[i][j]: True if new row i (at position seq_len - q_len + i) sees key j
    mask: List[List[bool]] = []
    for i in range(q_len):
        p = seq_len - q_len + i
        row = []
        for j in range(seq_len):
            ok = j <= p
            if window > 0 and j < p - window + 1:
                ok = False
            row.append(ok)
        mask.append(row)
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(q_len)]
    lse = [[0.0] * Hq for _ in range(q_len)]
    for i in range(q_len):
        for h in range(Hq):
            g = h // group
            scores = []
            for j in range(seq_len):
                if mask[i][j]:
                    scores.append((j, scale * math.fsum(q[i][h][d] * k[g][j][d] for d in range(D))))
            mx = max(s for _, s in scores)
            w = [(j, math.exp(s - mx)) for j, s in scores]
            z = math.fsum(x for _, x in w)
            for d in range(D):
                out[i][h][d] = math.fsum(x * v[g][j][d] for j, x in w) / z
            lse[i][h] = mx + math.log(z)
    return out, lse
