"""Zigzag split of packed sequences over cp ranks (oracle; test infrastructure only).

The LongVILA article names ZIGZAG-RINGATTN and says its chunk assignment
balances compute under a causal mask, but never prints the rule.  Reading
taken here (the plainest one that balances causal work exactly): every
sequence b of length L_b is cut into 2*cp equal chunks of C_b = L_b/(2*cp)
tokens; rank r keeps chunks r and 2*cp-1-r, in that order.  The local THD
tensor of a rank is, sequence after sequence, [chunk r ; chunk 2cp-1-r].
cp = 1 is the identity (no split, no divisibility requirement).

Ring step order ("Scaling Video Training with Parallelism", section 2, Ring
Attention paragraph: K/V blocks circulate while each device computes its
local attention): at step s rank r holds the K/V share of rank (r - s) mod cp;
step 0 is its own share.
"""
import numpy as np

from .masks import allowed


def rank_chunks(cp, r):
    """Chunk ids (out of 2*cp) that rank r keeps, in local order."""
    if cp == 1:
        return [0]
    return [r, 2 * cp - 1 - r]


def step_source(cp, r, s):
    """Rank whose K/V share rank r uses at ring step s."""
    return (r - s) % cp


def local_rows(cu_seqlens, cp, r):
    """Index plan of rank r.

    Returns (cu_local int32 [nseq+1], l2g int64 [T/cp] global row of each local
    row, pos int64 in-sequence position of each local row, seq int64 sequence
    id of each local row).
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    nseq = len(cu) - 1
    l2g, pos, seq = [], [], []
    cu_local = [0]
    for b in range(nseq):
        start, length = int(cu[b]), int(cu[b + 1] - cu[b])
        if cp > 1 and length % (2 * cp):
            raise ValueError(f"sequence {b} length {length} not divisible by 2*cp={2 * cp}")
        chunk = length if cp == 1 else length // (2 * cp)
        for c in rank_chunks(cp, r):
            p = np.arange(c * chunk, (c + 1) * chunk, dtype=np.int64)
            pos.append(p)
            l2g.append(start + p)
            seq.append(np.full(len(p), b, dtype=np.int64))
        cu_local.append(cu_local[-1] + (length if cp == 1 else 2 * chunk))
    cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int64)  # noqa: E731
    return np.asarray(cu_local, np.int32), cat(l2g), cat(pos), cat(seq)


def partition(x_global, cu_seqlens, cp, r):
    """Rank r's share of a global THD tensor (pure row gather)."""
    _, l2g, _, _ = local_rows(cu_seqlens, cp, r)
    return np.asarray(x_global)[l2g]


def count_pairs(cu_seqlens, cp, r, s, mode, tf_chunk=0, tf_num=0):
    """Allowed (query row, key row) pairs per head between rank r's queries
    and the keys rank r holds at step s, counted by brute force over the mask
    (a sequence at a time)."""
    _, _, qpos, qseq = local_rows(cu_seqlens, cp, r)
    _, _, kpos, kseq = local_rows(cu_seqlens, cp, step_source(cp, r, s))
    total = 0
    for b in np.unique(qseq):
        pq = qpos[qseq == b]
        pk = kpos[kseq == b]
        for i0 in range(0, len(pq), 4096):
            total += int(allowed(mode, pq[i0:i0 + 4096, None], pk[None, :],
                                 tf_chunk, tf_num).sum())
    return total
