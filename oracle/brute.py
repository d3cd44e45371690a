"""Pure-Python brute force for tiny inputs (oracle; test infrastructure only).

Triple loops with math.fsum, written straight from the attention definition
(softmax_attention.py), used to pin the NumPy oracle on tiny shapes.  Masks are
passed in as a Python predicate so this file shares no mask code either.
"""
import math


def brute_attention(q, k, v, seqs, pred, scale):
    """q: [Nq][Hq][d] nested lists; k, v: [Nk][Hkv][d]; seqs: list of
    (q_rows, q_positions, k_rows, k_positions) per sequence; pred(pq, pk) -> bool.
    Returns (out [Nq][Hq][d], lse [Hq][Nq])."""
    nq, hq, d = len(q), len(q[0]), len(q[0][0])
    hkv = len(k[0])
    grp = hq // hkv
    out = [[[0.0] * d for _ in range(hq)] for _ in range(nq)]
    lse = [[-math.inf] * nq for _ in range(hq)]
    for q_rows, q_pos, k_rows, k_pos in seqs:
        for qi, pq in zip(q_rows, q_pos):
            for h in range(hq):
                g = h // grp
                scores = []
                for kj, pk in zip(k_rows, k_pos):
                    if pred(pq, pk):
                        s = scale * math.fsum(q[qi][h][c] * k[kj][g][c] for c in range(d))
                        scores.append((s, kj))
                if not scores:
                    continue
                mx = max(s for s, _ in scores)
                w = [(math.exp(s - mx), kj) for s, kj in scores]
                z = math.fsum(x for x, _ in w)
                for c in range(d):
                    out[qi][h][c] = math.fsum(x * v[kj][g][c] for x, kj in w) / z
                lse[h][qi] = mx + math.log(z)
    return out, lse
