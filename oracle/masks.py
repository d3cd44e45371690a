"""Mask predicates over in-sequence positions (oracle; test infrastructure only).

The mask M(p_q, p_k) says whether a query at in-sequence position p_q may
attend a key at position p_k of the same sequence.

CAUSAL   p_k <= p_q (diagonal included).  The pages never print the mask; this
         is the plain autoregressive reading, applied on positions in the
         unsplit sequence so that splitting changes nothing ("Scaling Video
         Training with Parallelism", section 1).
BIDIR    every key of the same sequence.
TF_BLOCK teacher forcing ("Scaling Video Training with Parallelism",
         section 4): the sequence is [clean history ; noisy target], N time
         chunks of B tokens in each stream.  A clean query of chunk c sees
         clean keys of chunks <= c; a noisy query of chunk c sees clean keys
         of chunks < c and the noisy keys of its own chunk (bidirectional
         inside the chunk).  Clean never sees noisy.
"""
import numpy as np

CAUSAL, BIDIR, TF_BLOCK = 0, 1, 2


def allowed(mode, pq, pk, tf_chunk=0, tf_num=0):
    """Boolean array M(pq, pk) (numpy broadcasting over pq, pk)."""
    pq = np.asarray(pq, dtype=np.int64)
    pk = np.asarray(pk, dtype=np.int64)
    if mode == CAUSAL:
        return pk <= pq
    if mode == BIDIR:
        return np.ones(np.broadcast_shapes(pq.shape, pk.shape), dtype=bool)
    if mode == TF_BLOCK:
        if tf_chunk <= 0 or tf_num <= 0:
            raise ValueError("TF_BLOCK needs tf_chunk > 0 and tf_num > 0")
        span = tf_chunk * tf_num          # length of one stream
        q_noisy = pq >= span
        k_noisy = pk >= span
        cq = np.where(q_noisy, pq - span, pq) // tf_chunk
        ck = np.where(k_noisy, pk - span, pk) // tf_chunk
        clean_q = ~q_noisy & ~k_noisy & (ck <= cq)
        noisy_q = q_noisy & ((~k_noisy & (ck < cq)) | (k_noisy & (ck == cq)))
        return clean_q | noisy_q
    raise ValueError(f"unknown mask mode {mode}")


def seq_mask(mode, q_seq, q_pos, k_seq, k_pos, tf_chunk=0, tf_num=0):
    """Full [Nq, Nk] mask: same sequence and M(p_q, p_k)."""
    same = np.asarray(q_seq)[:, None] == np.asarray(k_seq)[None, :]
    return same & allowed(mode, np.asarray(q_pos)[:, None], np.asarray(k_pos)[None, :],
                          tf_chunk, tf_num)
