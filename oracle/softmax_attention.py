"""Masked softmax attention and its gradient in fp64 (oracle; test
infrastructure only).

Definition (the pages never print it; this is the textbook scaled dot-product
attention that the blockwise Ring Attention of "Scaling Video Training with
Parallelism", section 2, computes piece by piece).  For query row i, q-head h,
kv-head g = h // (Hq/Hkv) (contiguous GQA groups), and A(i) the keys of the
same sequence allowed by the mask:

    s_ij  = scale * <q_i, k_j>,              scale = 1/sqrt(d) by default
    LSE_i = log sum_{j in A(i)} exp(s_ij)    (natural log)
    P_ij  = exp(s_ij - LSE_i)
    O_i   = sum_{j in A(i)} P_ij v_j
    A(i) empty:  O_i = 0, LSE_i = -inf.

Backward, for the loss l = sum_i <dO_i, O_i> over the evaluated query rows,
with LSE and O the final ones (over every key of every ring step):

    delta_i = <dO_i, O_i>
    dS_ij   = P_ij (<dO_i, v_j> - delta_i)
    dQ_i    = scale * sum_j dS_ij k_j
    dK_j    = scale * sum_i dS_ij q_i     (summed over the q-heads of a group)
    dV_j    = sum_i P_ij dO_i             (summed over the q-heads of a group)

Restricting j to the keys one ring step holds gives that step's share of dQ
and that source rank's dK/dV.
"""
import numpy as np

from .masks import allowed


def default_scale(d):
    return 1.0 / np.sqrt(d)


def kv_head(h, hq, hkv):
    """GQA head map: contiguous groups of Hq/Hkv q-heads share kv-head h // (Hq/Hkv)."""
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (hq // hkv)


def attention(q, k, v, q_seq, q_pos, k_seq, k_pos, mode, scale=None,
              tf_chunk=0, tf_num=0, row_block=2048):
    """O [Nq, Hq, d] and LSE [Hq, Nq] in fp64.

    q: [Nq, Hq, d]; k, v: [Nk, Hkv, d]; *_seq / *_pos: sequence id and
    in-sequence position of every row.  Keys of other sequences are never
    attended.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    nq, hq, d = q.shape
    hkv = k.shape[1]
    scale = default_scale(d) if scale is None else scale
    q_seq, q_pos = np.asarray(q_seq), np.asarray(q_pos)
    k_seq, k_pos = np.asarray(k_seq), np.asarray(k_pos)
    out = np.zeros((nq, hq, d), np.float64)
    lse = np.full((hq, nq), -np.inf, np.float64)
    for b in np.unique(q_seq):
        qi = np.nonzero(q_seq == b)[0]
        ki = np.nonzero(k_seq == b)[0]
        if len(ki) == 0:
            continue
        for r0 in range(0, len(qi), row_block):
            rows = qi[r0:r0 + row_block]
            m = allowed(mode, q_pos[rows][:, None], k_pos[ki][None, :], tf_chunk, tf_num)
            empty = ~m.any(axis=1)
            for h in range(hq):
                g = kv_head(h, hq, hkv)
                s = (q[rows, h, :] @ k[ki, g, :].T) * scale
                s = np.where(m, s, -np.inf)
                mx = np.where(empty, 0.0, s.max(axis=1))
                p = np.exp(s - mx[:, None])
                z = p.sum(axis=1)
                zs = np.where(empty, 1.0, z)
                o = (p @ v[ki, g, :]) / zs[:, None]
                out[rows, h, :] = np.where(empty[:, None], 0.0, o)
                lse[h, rows] = np.where(empty, -np.inf, mx + np.log(zs))
    return out, lse


def bwd_delta(out, dout):
    """delta [Hq, Nq] = rowwise <dO_i, O_i> (fp64)."""
    return np.einsum("nhd,nhd->hn", np.asarray(out, np.float64), np.asarray(dout, np.float64))


def attention_backward(q, k, v, dout, lse, delta, q_seq, q_pos, k_seq, k_pos, mode,
                       scale=None, tf_chunk=0, tf_num=0, row_block=2048):
    """(dQ [Nq,Hq,d], dK [Nk,Hkv,d], dV [Nk,Hkv,d]) in fp64 from the final LSE
    and delta of the evaluated query rows, restricted to the given keys."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dout = np.asarray(dout, np.float64)
    lse = np.asarray(lse, np.float64)
    delta = np.asarray(delta, np.float64)
    nq, hq, d = q.shape
    hkv = k.shape[1]
    scale = default_scale(d) if scale is None else scale
    q_seq, q_pos = np.asarray(q_seq), np.asarray(q_pos)
    k_seq, k_pos = np.asarray(k_seq), np.asarray(k_pos)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in np.unique(q_seq):
        qi = np.nonzero(q_seq == b)[0]
        ki = np.nonzero(k_seq == b)[0]
        if len(ki) == 0:
            continue
        for r0 in range(0, len(qi), row_block):
            rows = qi[r0:r0 + row_block]
            m = allowed(mode, q_pos[rows][:, None], k_pos[ki][None, :], tf_chunk, tf_num)
            for h in range(hq):
                g = kv_head(h, hq, hkv)
                lrow = lse[h, rows]
                finite = np.isfinite(lrow)
                s = (q[rows, h, :] @ k[ki, g, :].T) * scale
                p = np.where(m & finite[:, None],
                             np.exp(s - np.where(finite, lrow, 0.0)[:, None]), 0.0)
                dp = dout[rows, h, :] @ v[ki, g, :].T
                ds = p * (dp - delta[h, rows][:, None])
                dq[rows, h, :] += scale * (ds @ k[ki, g, :])
                dk[ki, g, :] += scale * (ds.T @ q[rows, h, :])
                dv[ki, g, :] += p.T @ dout[rows, h, :]
    return dq, dk, dv
