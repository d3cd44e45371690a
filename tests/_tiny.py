"""Small helpers shared by the CPU tests: independent mask predicates written
as plain Python (not the oracle's), and tiny seeded inputs."""
import numpy as np


def pred_causal(pq, pk):
    return pk <= pq


def pred_bidir(pq, pk):
    return True


def make_pred_tf(B, N):
    """Teacher forcing: clean chunk c sees clean <= c; noisy chunk c sees
    clean < c and noisy == c."""
    def pred(pq, pk):
        q_noisy, k_noisy = pq >= N * B, pk >= N * B
        cq = (pq - N * B if q_noisy else pq) // B
        ck = (pk - N * B if k_noisy else pk) // B
        if not q_noisy:
            return (not k_noisy) and ck <= cq
        return (k_noisy and ck == cq) or ((not k_noisy) and ck < cq)
    return pred


def tiny_inputs(seed, lens, hq, hkv, d, dout=False):
    rng = np.random.default_rng(seed)
    t = sum(lens)
    q = rng.standard_normal((t, hq, d))
    k = rng.standard_normal((t, hkv, d))
    v = rng.standard_normal((t, hkv, d))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    seq = np.repeat(np.arange(len(lens)), lens)
    pos = np.concatenate([np.arange(l) for l in lens])
    out = dict(q=q, k=k, v=v, cu=cu, seq=seq, pos=pos)
    if dout:
        out["dout"] = rng.standard_normal((t, hq, d))
    return out
