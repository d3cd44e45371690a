"""Log-sum-exp merge of two partial attention results (oracle; test
infrastructure only).

Ring Attention ("Scaling Video Training with Parallelism", section 2)
computes attention against one K/V block at a time; the pages do not print
how the pieces are combined.  Reading taken: the partial results over two
disjoint key sets are combined as the softmax over their union, i.e.

    LSE' = log(exp(LSE) + exp(LSE_p))
    O'   = exp(LSE - LSE') O + exp(LSE_p - LSE') O_p

A row whose partial LSE is -inf (no allowed key in that block) passes through
unchanged; a running row at -inf takes the partial as it is.
"""
import numpy as np


def merge(out, lse, out_p, lse_p):
    """Return (out', lse') for out/out_p [N, H, d] and lse/lse_p [H, N] (fp64)."""
    out = np.asarray(out, np.float64)
    out_p = np.asarray(out_p, np.float64)
    lse = np.asarray(lse, np.float64)
    lse_p = np.asarray(lse_p, np.float64)
    new_out = out.copy()
    new_lse = lse.copy()
    n_heads, n_rows = lse.shape
    for h in range(n_heads):
        for i in range(n_rows):
            a, b = lse[h, i], lse_p[h, i]
            if b == -np.inf:
                continue
            if a == -np.inf:
                new_out[i, h] = out_p[i, h]
                new_lse[h, i] = b
                continue
            hi = max(a, b)
            tot = hi + np.log(np.exp(a - hi) + np.exp(b - hi))
            new_out[i, h] = np.exp(a - tot) * out[i, h] + np.exp(b - tot) * out_p[i, h]
            new_lse[h, i] = tot
    return new_out, new_lse
