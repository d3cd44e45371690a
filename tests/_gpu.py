"""Helpers for the GPU parity tests: upload seeded inputs, run the ring loop
through the C ABI, and the tolerance checks."""
import numpy as np
import torch

import oracle

TOL_F32_MAXABS = 1e-5
TOL_BF16_RELRMS = 5e-3
TOL_BF16_MAXABS = 2e-2
TOL_LSE_ABS = 1e-3
TOL_GRAD_RELRMS = 1e-2


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).cuda()


def tdtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def rel_rms(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.sqrt(np.mean(ref ** 2))
    return float(np.sqrt(np.mean((x - ref) ** 2)) / (den if den > 0 else 1.0))


def check_lse(lse, ref, tol=TOL_LSE_ABS):
    lse = np.asarray(lse, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(lse), fin), "finite pattern of LSE differs"
    assert np.all(lse[~fin] == -np.inf)
    if fin.any():
        err = np.max(np.abs(lse[fin] - ref[fin]))
        assert err <= tol, f"LSE abs err {err}"


def check_out(out, ref, dtype):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(out)), "non-finite output"
    err = np.max(np.abs(out - ref)) if out.size else 0.0
    if dtype == "f32":
        assert err <= TOL_F32_MAXABS, f"max abs err {err}"
    else:
        rr = rel_rms(out, ref)
        assert rr <= TOL_BF16_RELRMS, f"rel-RMS {rr}"
        assert err <= TOL_BF16_MAXABS, f"max abs err {err}"


def oracle_step(x, cu, cp, r, s, mode, tf=(0, 0)):
    """Per-step expectation: rank r's queries vs the keys of rank (r-s) mod cp."""
    _, l2g, qpos, qseq = oracle.local_rows(cu, cp, r)
    _, k2g, kpos, kseq = oracle.local_rows(cu, cp, oracle.step_source(cp, r, s))
    return oracle.attention(x["q"][l2g], x["k"][k2g], x["v"][k2g], qseq, qpos, kseq, kpos, mode,
                            tf_chunk=tf[0], tf_num=tf[1])


def oracle_rank_full(x, cu, cp, r, mode, tf=(0, 0), rows=None):
    """Merged expectation: rank r's query rows (or a subset given as local row
    indices) against every key of their sequence."""
    _, l2g, qpos, qseq = oracle.local_rows(cu, cp, r)
    if rows is not None:
        l2g, qpos, qseq = l2g[rows], qpos[rows], qseq[rows]
    T = int(cu[-1])
    seq = np.repeat(np.arange(len(cu) - 1), np.diff(cu))
    pos = np.arange(T) - np.asarray(cu)[seq]
    keep = np.isin(seq, np.unique(qseq))
    return oracle.attention(x["q"][l2g], x["k"][keep], x["v"][keep], qseq, qpos, seq[keep], pos[keep], mode,
                            tf_chunk=tf[0], tf_num=tf[1])
