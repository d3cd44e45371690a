"""Pins of the fp64 attention oracle against things other than itself:
a pure-Python brute force, torch's fp64 scaled_dot_product_attention (a
library routine), closed forms and the softmax normalisation."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.brute import brute_attention
from tests._tiny import make_pred_tf, pred_bidir, pred_causal, tiny_inputs

CASES = [
    # (lens, hq, hkv, d, mode, tf)
    ([7, 12, 5], 2, 1, 4, oracle.CAUSAL, None),
    ([9, 16], 4, 2, 8, oracle.BIDIR, None),
    ([24], 2, 2, 4, oracle.TF_BLOCK, (4, 3)),
    ([16, 8], 3, 1, 5, oracle.TF_BLOCK, (2, 4)),
    ([1, 3, 2], 2, 2, 3, oracle.CAUSAL, None),
]


def _pred(mode, tf):
    if mode == oracle.CAUSAL:
        return pred_causal
    if mode == oracle.BIDIR:
        return pred_bidir
    return make_pred_tf(*tf)


@pytest.mark.parametrize("lens,hq,hkv,d,mode,tf", CASES)
def test_oracle_matches_brute_force(lens, hq, hkv, d, mode, tf):
    x = tiny_inputs(1, lens, hq, hkv, d)
    tfc, tfn = tf or (0, 0)
    scale = 1.0 / math.sqrt(d)
    o, l = oracle.attention(x["q"], x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"],
                            mode, tf_chunk=tfc, tf_num=tfn)
    seqs = []
    cu = x["cu"]
    for b in range(len(lens)):
        rows = list(range(cu[b], cu[b + 1]))
        seqs.append((rows, list(range(lens[b])), rows, list(range(lens[b]))))
    bo, bl = brute_attention(x["q"].tolist(), x["k"].tolist(), x["v"].tolist(), seqs,
                             _pred(mode, tf), scale)
    np.testing.assert_allclose(o, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, np.array(bl), rtol=0, atol=1e-12)


@pytest.mark.parametrize("lens,hq,hkv,d,mode,tf", CASES + [([300, 211], 4, 2, 32, oracle.CAUSAL, None),
                                                            ([2 * 12 * 20], 2, 2, 16, oracle.TF_BLOCK, (20, 12))])
def test_oracle_matches_torch_sdpa_fp64(lens, hq, hkv, d, mode, tf):
    x = tiny_inputs(2, lens, hq, hkv, d)
    tfc, tfn = tf or (0, 0)
    o, l = oracle.attention(x["q"], x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"],
                            mode, tf_chunk=tfc, tf_num=tfn)
    pred = _pred(mode, tf)
    cu = x["cu"]
    g = hq // hkv
    for b in range(len(lens)):
        s0, s1 = cu[b], cu[b + 1]
        n = s1 - s0
        mask = torch.tensor([[bool(pred(i, j)) for j in range(n)] for i in range(n)])
        qt = torch.from_numpy(x["q"][s0:s1]).permute(1, 0, 2)
        kt = torch.from_numpy(x["k"][s0:s1]).permute(1, 0, 2).repeat_interleave(g, 0)
        vt = torch.from_numpy(x["v"][s0:s1]).permute(1, 0, 2).repeat_interleave(g, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
        np.testing.assert_allclose(o[s0:s1], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        # LSE from torch's logsumexp over the masked scores.
        sc = (qt @ kt.transpose(1, 2)) / math.sqrt(d)
        sc = sc.masked_fill(~mask, -math.inf)
        np.testing.assert_allclose(l[:, s0:s1], torch.logsumexp(sc, -1).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode,tf", [(oracle.CAUSAL, None), (oracle.BIDIR, None),
                                     (oracle.TF_BLOCK, (3, 4))])
def test_closed_form_zero_query(mode, tf):
    """q = 0: every allowed score is 0, so O_i is the mean of the allowed v_j
    and LSE_i = ln |A(i)|."""
    lens = [24, 24]
    x = tiny_inputs(3, lens, 2, 2, 4)
    tfc, tfn = tf or (0, 0)
    q0 = np.zeros_like(x["q"])
    o, l = oracle.attention(q0, x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"], mode,
                            tf_chunk=tfc, tf_num=tfn)
    pred = _pred(mode, tf)
    for i in range(sum(lens)):
        b = x["seq"][i]
        keys = [j for j in range(sum(lens)) if x["seq"][j] == b and pred(x["pos"][i], x["pos"][j])]
        for h in range(2):
            np.testing.assert_allclose(o[i, h], x["v"][keys, h].mean(0), atol=1e-13)
            assert abs(l[h, i] - math.log(len(keys))) < 1e-13


def test_closed_form_constant_values_and_single_key():
    x = tiny_inputs(4, [10, 6], 4, 2, 8)
    v = np.full_like(x["v"], 2.5)
    o, _ = oracle.attention(x["q"], x["k"], v, x["seq"], x["pos"], x["seq"], x["pos"], oracle.CAUSAL)
    np.testing.assert_allclose(o, 2.5, atol=1e-13)
    # causal row at position 0 sees exactly one key: O = v_0, LSE = s_00
    o, l = oracle.attention(x["q"], x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"], oracle.CAUSAL)
    for b0 in (0, 10):
        for h in range(4):
            g = h // 2
            np.testing.assert_allclose(o[b0, h], x["v"][b0, g], atol=1e-14)
            s = x["q"][b0, h] @ x["k"][b0, g] / math.sqrt(8)
            assert abs(l[h, b0] - s) < 1e-13


def test_bidir_equals_textbook_softmax():
    from scipy.special import softmax
    x = tiny_inputs(5, [33], 3, 3, 16)
    o, _ = oracle.attention(x["q"], x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"], oracle.BIDIR)
    for h in range(3):
        s = x["q"][:, h] @ x["k"][:, h].T / 4.0
        np.testing.assert_allclose(o[:, h], softmax(s, axis=1) @ x["v"][:, h], atol=1e-13)


@pytest.mark.parametrize("mode,tf", [(oracle.CAUSAL, None), (oracle.TF_BLOCK, (5, 3))])
def test_softmax_rows_sum_to_one(mode, tf):
    x = tiny_inputs(6, [30, 30], 2, 1, 8)
    tfc, tfn = tf or (0, 0)
    _, l = oracle.attention(x["q"], x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"], mode,
                            tf_chunk=tfc, tf_num=tfn)
    m = oracle.seq_mask(mode, x["seq"], x["pos"], x["seq"], x["pos"], tfc, tfn)
    for h in range(2):
        s = x["q"][:, h] @ x["k"][:, 0].T / math.sqrt(8)
        p = np.where(m, np.exp(s - l[h][:, None]), 0.0)
        np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-12)


def test_empty_rows_give_zero_and_minus_inf():
    """A query whose sequence has no key in the given set: O = 0, LSE = -inf."""
    x = tiny_inputs(7, [8, 8], 2, 2, 4)
    ksel = x["seq"] == 0
    o, l = oracle.attention(x["q"], x["k"][ksel], x["v"][ksel], x["seq"], x["pos"],
                            x["seq"][ksel], x["pos"][ksel], oracle.CAUSAL)
    assert np.all(o[8:] == 0) and np.all(l[:, 8:] == -np.inf)
    assert np.all(np.isfinite(l[:, :8]))


def test_tf_mask_streams():
    """Teacher forcing reading: clean never sees noisy; noisy chunk 0 sees only
    its own noisy chunk; pair count is N(N+1) B^2."""
    B, N = 3, 4
    p = np.arange(2 * N * B)
    m = oracle.allowed(oracle.TF_BLOCK, p[:, None], p[None, :], B, N)
    assert not m[: N * B, N * B:].any()
    row = m[N * B]          # first noisy token, chunk 0
    assert set(np.nonzero(row)[0]) == set(range(N * B, N * B + B))
    assert m.sum() == N * (N + 1) * B * B
    pred = make_pred_tf(B, N)
    assert all(m[i, j] == pred(i, j) for i in p for j in p)


def test_tf_permutation_equivariance():
    """Permuting tokens (and their positions) permutes outputs the same way."""
    B, N = 4, 3
    x = tiny_inputs(8, [2 * N * B], 2, 2, 8)
    o, l = oracle.attention(x["q"], x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"],
                            oracle.TF_BLOCK, tf_chunk=B, tf_num=N)
    perm = np.random.default_rng(0).permutation(2 * N * B)
    op, lp = oracle.attention(x["q"][perm], x["k"][perm], x["v"][perm], x["seq"][perm], x["pos"][perm],
                              x["seq"][perm], x["pos"][perm], oracle.TF_BLOCK, tf_chunk=B, tf_num=N)
    np.testing.assert_allclose(op, o[perm], atol=1e-13)
    np.testing.assert_allclose(lp, l[:, perm], atol=1e-13)
