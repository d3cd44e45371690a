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


def _pool_size():
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_by_head(fn, q, k, v, *args, **kw):
    """Call an oracle routine once per q-head, in a thread pool, and stitch the
    results: O_i and LSE_i of head h depend only on q-head h and its kv-head
    h // (Hq/Hkv), and dK/dV of a kv-head are the sums over its q-heads.  BLAS
    runs one thread per call inside the pool.  fn is oracle.attention
    (returns O, LSE) or oracle.attention_backward (returns dQ, dK, dV; pass
    dout, lse, delta as the first three extra arguments, full-head arrays)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    hq, hkv = q.shape[1], k.shape[1]
    grp = hq // hkv
    backward = fn is oracle.attention_backward

    def one(h):
        g = h // grp
        if backward:
            dout, lse, delta = args[:3]
            rest = args[3:]
            return fn(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], dout[:, h:h + 1], lse[h:h + 1],
                      delta[h:h + 1], *rest, **kw)
        return fn(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], *args, **kw)

    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(_pool_size()) as ex:
            res = list(ex.map(one, range(hq)))
    if backward:
        dq = np.concatenate([r[0] for r in res], axis=1)
        dk = np.zeros(k.shape, np.float64)
        dv = np.zeros(v.shape, np.float64)
        for h, r in enumerate(res):
            dk[:, h // grp] += r[1][:, 0]
            dv[:, h // grp] += r[2][:, 0]
        return dq, dk, dv
    return np.concatenate([r[0] for r in res], axis=1), np.concatenate([r[1] for r in res], axis=0)


def stratified_offsets(n, count, rng, tiles=(64, 128)):
    """About `count` distinct offsets in [0, n): the first two and last two,
    offsets next to tile edges (multiples of 64 and 128, +-1), and uniform
    ones; the draw is fixed by rng."""
    if n <= count:
        return np.arange(n)
    picks = {0, 1, n - 2, n - 1}
    edges = []
    for t in tiles:
        for m in range(t, n, t):
            edges += [m - 1, m, m + 1]
    edges = np.unique(np.clip(np.asarray(edges, np.int64), 0, n - 1))
    take = min(len(edges), count // 2)
    picks.update(int(x) for x in rng.choice(edges, size=take, replace=False))
    while len(picks) < count:
        picks.update(int(x) for x in rng.integers(0, n, size=count - len(picks)))
    return np.sort(np.fromiter(picks, np.int64))
