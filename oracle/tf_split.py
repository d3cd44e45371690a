"""Balanced teacher-forcing split over cp ranks (oracle; test infrastructure only).

"Scaling Video Training with Parallelism", section 4 (balanced SP for
LongLive-2.0): a plain cut of the [clean history ; noisy target] sequence can
leave some ranks with only clean context and others with all of the
loss-carrying noisy targets.  Balanced SP instead gives every rank the clean
and the noisy chunk of the same time segments, so the targets spread evenly.
The page is cut off before it states the assignment.  Reading taken here:

  * time chunks c = 0..N-1 are dealt to ranks in snake order over rounds of
    2*cp chunks: 0, 1, .., cp-1, cp-1, .., 1, 0, 0, 1, ...  Teacher-forcing
    work of chunk c grows with c + 1 (both streams), so each full round gives
    every rank the same work; N must be a multiple of cp (equal shares), and
    the work is exactly equal when N is a multiple of 2*cp;
  * a rank's local rows of a sequence are its clean chunks in ascending time
    order followed by its noisy chunks in the same order;
  * ring steps are unchanged: at step s rank r uses the K/V share of rank
    (r - s) mod cp (zigzag.step_source), and the mask is the TF_BLOCK
    predicate on positions in the unsplit sequence.
"""
import numpy as np

from .masks import TF_BLOCK, allowed
from .zigzag import step_source


def chunk_owners(num_chunks, cp):
    """Owner rank of every time chunk, dealt in snake order."""
    order = []
    while len(order) < num_chunks:
        order.extend(range(cp))
        order.extend(reversed(range(cp)))
    return order[:num_chunks]


def rank_time_chunks(num_chunks, cp, r):
    """Time chunks rank r holds, ascending."""
    return [c for c, o in enumerate(chunk_owners(num_chunks, cp)) if o == r]


def local_rows(cu_seqlens, cp, r, tf_chunk, tf_num):
    """Index plan of rank r for packed teacher-forcing sequences (every
    sequence is [clean_0..clean_{N-1} ; noisy_0..noisy_{N-1}], B = tf_chunk
    tokens per chunk, N = tf_num).

    Returns (cu_local int32 [nseq+1], l2g int64, pos int64, seq int64) like
    zigzag.local_rows.
    """
    B, N = int(tf_chunk), int(tf_num)
    if N % cp:
        raise ValueError(f"{N} time chunks do not split evenly over cp={cp}")
    mine = rank_time_chunks(N, cp, r)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    l2g, pos, seq = [], [], []
    cu_local = [0]
    for b in range(len(cu) - 1):
        start, length = int(cu[b]), int(cu[b + 1] - cu[b])
        if length != 2 * B * N:
            raise ValueError(f"sequence {b} has {length} tokens, teacher forcing needs 2*B*N = {2 * B * N}")
        for stream in (0, 1):                      # clean chunks, then noisy chunks
            for c in mine:
                p = stream * N * B + c * B + np.arange(B, dtype=np.int64)
                pos.append(p)
                l2g.append(start + p)
                seq.append(np.full(B, b, dtype=np.int64))
        cu_local.append(cu_local[-1] + 2 * B * len(mine))
    cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int64)  # noqa: E731
    return np.asarray(cu_local, np.int32), cat(l2g), cat(pos), cat(seq)


def partition(x_global, cu_seqlens, cp, r, tf_chunk, tf_num):
    """Rank r's balanced share of a global THD tensor (pure row gather)."""
    _, l2g, _, _ = local_rows(cu_seqlens, cp, r, tf_chunk, tf_num)
    return np.asarray(x_global)[l2g]


def count_pairs(cu_seqlens, cp, r, s, tf_chunk, tf_num):
    """Allowed (query, key) pairs per head between rank r's queries and the
    keys it holds at ring step s, by brute force over the mask."""
    _, _, qpos, qseq = local_rows(cu_seqlens, cp, r, tf_chunk, tf_num)
    _, _, kpos, kseq = local_rows(cu_seqlens, cp, step_source(cp, r, s), tf_chunk, tf_num)
    total = 0
    for b in np.unique(qseq):
        pq = qpos[qseq == b]
        pk = kpos[kseq == b]
        for i0 in range(0, len(pq), 4096):
            total += int(allowed(TF_BLOCK, pq[i0:i0 + 4096, None], pk[None, :], tf_chunk, tf_num).sum())
    return total
