"""Pins of the merge and of ring exactness: merging the per-step partial
results of every rank over every step reproduces attention over the unsplit
sequence ("Scaling Video Training with Parallelism", section 1: splitting
must not change what is computed)."""
import numpy as np
import pytest

import oracle
from tests._tiny import tiny_inputs


def _ring_forward(x, cp, r, mode, cu, tf=(0, 0)):
    _, l2g, qpos, qseq = oracle.local_rows(cu, cp, r)
    hq, d = x["q"].shape[1:]
    out = np.zeros((len(l2g), hq, d))
    lse = np.full((hq, len(l2g)), -np.inf)
    for s in range(cp):
        j = oracle.step_source(cp, r, s)
        _, k2g, kpos, kseq = oracle.local_rows(cu, cp, j)
        op, lp = oracle.attention(x["q"][l2g], x["k"][k2g], x["v"][k2g], qseq, qpos, kseq, kpos, mode,
                                  tf_chunk=tf[0], tf_num=tf[1])
        out, lse = oracle.merge(out, lse, op, lp)
    return l2g, out, lse


@pytest.mark.parametrize("lens,cp,hq,hkv", [([64], 4, 2, 2), ([32, 48, 16], 2, 4, 2), ([24, 40], 4, 3, 1)])
@pytest.mark.parametrize("mode", [0, 1])
def test_ring_merge_equals_full(lens, cp, hq, hkv, mode):
    x = tiny_inputs(11, lens, hq, hkv, 8)
    full_o, full_l = oracle.attention(x["q"], x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"], mode)
    for r in range(cp):
        l2g, o, l = _ring_forward(x, cp, r, mode, x["cu"])
        np.testing.assert_allclose(o, full_o[l2g], atol=1e-12)
        np.testing.assert_allclose(l, full_l[:, l2g], atol=1e-12)


def test_tf_split_keys_merge_equals_full():
    """Teacher forcing at cp = 1 with keys split into arbitrary disjoint
    blocks, merged in a shuffled order."""
    B, N = 3, 4
    x = tiny_inputs(12, [2 * N * B], 2, 2, 8)
    full_o, full_l = oracle.attention(x["q"], x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"],
                                      oracle.TF_BLOCK, tf_chunk=B, tf_num=N)
    perm = np.random.default_rng(1).permutation(2 * N * B)
    blocks = np.array_split(perm, 5)
    out = np.zeros_like(full_o)
    lse = np.full_like(full_l, -np.inf)
    for blk in blocks[::-1]:
        op, lp = oracle.attention(x["q"], x["k"][blk], x["v"][blk], x["seq"], x["pos"], x["seq"][blk],
                                  x["pos"][blk], oracle.TF_BLOCK, tf_chunk=B, tf_num=N)
        out, lse = oracle.merge(out, lse, op, lp)
    np.testing.assert_allclose(out, full_o, atol=1e-12)
    np.testing.assert_allclose(lse, full_l, atol=1e-12)


def test_merge_commutative_associative():
    rng = np.random.default_rng(3)
    parts = [(rng.standard_normal((5, 2, 4)), rng.standard_normal((2, 5)) * 3) for _ in range(3)]
    parts[1][1][0, 2] = -np.inf
    a = oracle.merge(*parts[0], *parts[1])
    b = oracle.merge(*parts[1], *parts[0])
    np.testing.assert_allclose(a[0], b[0], atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], atol=1e-14)
    ab_c = oracle.merge(*a, *parts[2])
    bc = oracle.merge(*parts[1], *parts[2])
    a_bc = oracle.merge(*parts[0], *bc)
    np.testing.assert_allclose(ab_c[0], a_bc[0], atol=1e-13)
    np.testing.assert_allclose(ab_c[1], a_bc[1], atol=1e-13)


def test_merge_closed_form_equal_halves():
    """Two partials with equal LSE: the result is their mean and LSE + ln 2."""
    rng = np.random.default_rng(4)
    o1, o2 = rng.standard_normal((3, 2, 4)), rng.standard_normal((3, 2, 4))
    l = rng.standard_normal((2, 3))
    o, lm = oracle.merge(o1, l, o2, l)
    np.testing.assert_allclose(o, (o1 + o2) / 2, atol=1e-15)
    np.testing.assert_allclose(lm, l + np.log(2.0), atol=1e-15)


def test_merge_minus_inf_passthrough_is_bit_exact():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((4, 2, 8))
    l = rng.standard_normal((2, 4))
    op = rng.standard_normal((4, 2, 8))
    lp = np.full((2, 4), -np.inf)
    no, nl = oracle.merge(o, l, op, lp)
    assert np.array_equal(no, o) and np.array_equal(nl, l)
    # running at (0, -inf) takes the partial as is; (-inf, -inf) stays (0, -inf)
    z = np.zeros_like(o)
    zl = np.full_like(l, -np.inf)
    no, nl = oracle.merge(z, zl, op, l)
    assert np.array_equal(no, op) and np.array_equal(nl, l)
    no, nl = oracle.merge(z, zl, op, lp)
    assert np.array_equal(no, z) and np.array_equal(nl, zl)
