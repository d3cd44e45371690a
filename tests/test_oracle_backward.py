"""Pins of the backward oracle: torch fp64 autograd (library routine), central
finite differences, and invariants that follow from sum_j P_ij = 1."""
import numpy as np
import pytest
import torch

import oracle
from tests._tiny import tiny_inputs


def _full(x, mode, tf=(0, 0)):
    o, l = oracle.attention(x["q"], x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"], mode,
                            tf_chunk=tf[0], tf_num=tf[1])
    delta = oracle.bwd_delta(o, x["dout"])
    g = oracle.attention_backward(x["q"], x["k"], x["v"], x["dout"], l, delta, x["seq"], x["pos"],
                                  x["seq"], x["pos"], mode, tf_chunk=tf[0], tf_num=tf[1])
    return o, l, g


@pytest.mark.parametrize("lens,hq,hkv,mode,tf", [([12, 7], 4, 2, 0, (0, 0)), ([10], 2, 1, 1, (0, 0)),
                                                  ([18], 3, 3, 2, (3, 3))])
def test_backward_matches_torch_autograd(lens, hq, hkv, mode, tf):
    x = tiny_inputs(21, lens, hq, hkv, 6, dout=True)
    _, _, (dq, dk, dv) = _full(x, mode, tf)
    m = torch.from_numpy(oracle.seq_mask(mode, x["seq"], x["pos"], x["seq"], x["pos"], *tf))
    q = torch.tensor(x["q"], requires_grad=True)
    k = torch.tensor(x["k"], requires_grad=True)
    v = torch.tensor(x["v"], requires_grad=True)
    g = hq // hkv
    qt = q.permute(1, 0, 2)
    kt = k.permute(1, 0, 2).repeat_interleave(g, 0)
    vt = v.permute(1, 0, 2).repeat_interleave(g, 0)
    s = (qt @ kt.transpose(1, 2)) / np.sqrt(6)
    p = torch.softmax(s.masked_fill(~m, -np.inf), -1)
    o = (p @ vt).permute(1, 0, 2)
    (o * torch.from_numpy(x["dout"])).sum().backward()
    np.testing.assert_allclose(dq, q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, k.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, v.grad.numpy(), atol=1e-12)


def test_backward_finite_differences():
    x = tiny_inputs(22, [6, 5], 2, 1, 3, dout=True)
    _, _, (dq, dk, dv) = _full(x, oracle.CAUSAL)
    h = 1e-6

    def loss(xx):
        o, _ = oracle.attention(xx["q"], xx["k"], xx["v"], xx["seq"], xx["pos"], xx["seq"], xx["pos"],
                                oracle.CAUSAL)
        return float((o * xx["dout"]).sum())

    rng = np.random.default_rng(0)
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(6):
            idx = tuple(rng.integers(0, n) for n in x[name].shape)
            xp = {kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in x.items()}
            xm = {kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            fd = (loss(xp) - loss(xm)) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-7, (name, idx, fd, grad[idx])


def test_backward_invariants():
    """sum_j dV_j = sum_i dO_i (per sequence and kv group) and sum_j dK_j = 0."""
    lens = [20, 12]
    x = tiny_inputs(23, lens, 4, 2, 5, dout=True)
    _, _, (_, dk, dv) = _full(x, oracle.CAUSAL)
    for b in range(2):
        sel = x["seq"] == b
        for g in range(2):
            np.testing.assert_allclose(dv[sel, g].sum(0), x["dout"][sel][:, 2 * g:2 * g + 2].sum((0, 1)),
                                       atol=1e-12)
            np.testing.assert_allclose(dk[sel, g].sum(0), 0.0, atol=1e-12)


@pytest.mark.parametrize("lens,cp", [([32], 4), ([16, 48], 2)])
def test_ring_backward_sums_to_full(lens, cp):
    """Per-step contributions from the final LSE, summed over steps (dQ) and
    over ranks (dK/dV of each source), equal the unsplit gradient."""
    x = tiny_inputs(24, lens, 4, 2, 6, dout=True)
    cu = x["cu"]
    _, _, (dq_f, dk_f, dv_f) = _full(x, oracle.CAUSAL)
    o_f, l_f = oracle.attention(x["q"], x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"], oracle.CAUSAL)
    dk_sum = np.zeros_like(dk_f)
    dv_sum = np.zeros_like(dv_f)
    for r in range(cp):
        _, l2g, qpos, qseq = oracle.local_rows(cu, cp, r)
        delta = oracle.bwd_delta(o_f[l2g], x["dout"][l2g])
        dq = np.zeros((len(l2g),) + x["q"].shape[1:])
        for s in range(cp):
            j = oracle.step_source(cp, r, s)
            _, k2g, kpos, kseq = oracle.local_rows(cu, cp, j)
            a, b, c = oracle.attention_backward(x["q"][l2g], x["k"][k2g], x["v"][k2g], x["dout"][l2g],
                                                l_f[:, l2g], delta, qseq, qpos, kseq, kpos, oracle.CAUSAL)
            dq += a
            dk_sum[k2g] += b
            dv_sum[k2g] += c
        np.testing.assert_allclose(dq, dq_f[l2g], atol=1e-12)
    np.testing.assert_allclose(dk_sum, dk_f, atol=1e-12)
    np.testing.assert_allclose(dv_sum, dv_f, atol=1e-12)
