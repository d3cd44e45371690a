"""Pins of the balanced teacher-forcing split (oracle/tf_split.py).

"Scaling Video Training with Parallelism", section 4 (balanced SP): every
rank holds the clean and the noisy chunk of the same time segments and an
even share of the noisy targets; section 1: splitting must not change what
is computed.  The assignment rule is the reading stated in tf_split.py."""
import os

import numpy as np
import pytest

import oracle
from oracle import tf_split
from tests._tiny import make_pred_tf, tiny_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tf_balanced_N12.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            v = [int(x) for x in line.split()]
            rows.append((v[0], v[1], v[2:-1], v[-1]))
    return rows


def test_golden_chunk_table():
    rows = _golden()
    assert len(rows) == 2 + 3 + 4 + 6
    for cp, r, chunks, work in rows:
        assert tf_split.rank_time_chunks(12, cp, r) == chunks
        assert sum(c + 1 for c in chunks) == work


@pytest.mark.parametrize("cp,B,N,nseq", [(2, 3, 4, 1), (2, 2, 8, 2), (3, 2, 6, 3), (4, 1, 12, 1), (6, 2, 12, 2)])
def test_rows_partition_and_pairing(cp, B, N, nseq):
    L = 2 * B * N
    cu = np.arange(nseq + 1, dtype=np.int32) * L
    seen = []
    for r in range(cp):
        cu_l, l2g, pos, seq = tf_split.local_rows(cu, cp, r, B, N)
        assert list(cu_l) == [b * L // cp for b in range(nseq + 1)]
        assert np.array_equal(l2g, cu[seq] + pos)
        seen.append(l2g)
        for b in range(nseq):
            p = pos[seq == b]
            clean = sorted({int(x) // B for x in p if x < N * B})
            noisy = sorted({(int(x) - N * B) // B for x in p if x >= N * B})
            assert clean == noisy                      # clean/noisy pair of the same time chunks
            assert int((p >= N * B).sum()) == N * B // cp  # even share of the noisy targets
            # local order: clean chunks ascending, then noisy chunks ascending
            assert np.array_equal(p[: len(p) // 2], np.concatenate([c * B + np.arange(B) for c in clean]))
    allrows = np.sort(np.concatenate(seen))
    assert np.array_equal(allrows, np.arange(nseq * L))


@pytest.mark.parametrize("cp,B,N", [(2, 2, 4), (2, 3, 8), (3, 2, 6), (3, 1, 12), (4, 2, 8)])
def test_work_is_balanced(cp, B, N):
    """Per-rank pairs summed over the ring steps, by brute force over the mask,
    equal the closed form sum over held chunks of 2*(c+1)*B^2, which is the
    same N(N+1)B^2/cp for every rank when N is a multiple of 2*cp."""
    cu = np.array([0, 2 * B * N], np.int32)
    totals = []
    for r in range(cp):
        t = sum(tf_split.count_pairs(cu, cp, r, s, B, N) for s in range(cp))
        assert t == sum(2 * (c + 1) * B * B for c in tf_split.rank_time_chunks(N, cp, r))
        totals.append(t)
    assert set(totals) == {N * (N + 1) * B * B // cp}


def test_step_pairs_match_plain_predicate():
    """Per-step counts against a pure-Python predicate over the oracle's
    positions (not the oracle's mask)."""
    cp, B, N = 3, 2, 6
    cu = np.array([0, 2 * B * N], np.int32)
    pred = make_pred_tf(B, N)
    for r in range(cp):
        _, _, qpos, _ = tf_split.local_rows(cu, cp, r, B, N)
        for s in range(cp):
            _, _, kpos, _ = tf_split.local_rows(cu, cp, oracle.step_source(cp, r, s), B, N)
            want = sum(1 for pq in qpos for pk in kpos if pred(int(pq), int(pk)))
            assert tf_split.count_pairs(cu, cp, r, s, B, N) == want


@pytest.mark.parametrize("cp,B,N,lens_mult", [(2, 3, 4, 1), (3, 2, 6, 2), (2, 2, 8, 1)])
def test_ring_merge_equals_full(cp, B, N, lens_mult):
    """fp64: for every rank, the merge of its per-step partial results over
    all ring steps equals unsplit teacher-forcing attention on its rows."""
    L = 2 * B * N
    x = tiny_inputs(23, [L] * lens_mult, 3, 1, 8)
    cu = x["cu"]
    full_o, full_l = oracle.attention(x["q"], x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"],
                                      oracle.TF_BLOCK, tf_chunk=B, tf_num=N)
    for r in range(cp):
        _, l2g, qpos, qseq = tf_split.local_rows(cu, cp, r, B, N)
        out = np.zeros((len(l2g), 3, 8))
        lse = np.full((3, len(l2g)), -np.inf)
        for s in range(cp):
            _, k2g, kpos, kseq = tf_split.local_rows(cu, cp, oracle.step_source(cp, r, s), B, N)
            op, lp = oracle.attention(x["q"][l2g], x["k"][k2g], x["v"][k2g], qseq, qpos, kseq, kpos,
                                      oracle.TF_BLOCK, tf_chunk=B, tf_num=N)
            out, lse = oracle.merge(out, lse, op, lp)
        np.testing.assert_allclose(out, full_o[l2g], atol=1e-12)
        np.testing.assert_allclose(lse, full_l[:, l2g], atol=1e-12)


def test_round_robin_dealing_is_caught(monkeypatch):
    """Planted mistake: dealing chunks round-robin (c mod cp) keeps the
    pairing but not the balance; the golden table and the balance pin fail."""
    monkeypatch.setattr(tf_split, "chunk_owners", lambda n, cp: [c % cp for c in range(n)])
    with pytest.raises(AssertionError):
        test_golden_chunk_table()
    with pytest.raises(AssertionError):
        test_work_is_balanced(2, 2, 4)
