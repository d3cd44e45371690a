"""Pins of the oracle's zigzag index plan and pair counting: hand-written
golden tables, partition-of-rows invariants and the closed-form causal pair
counts that make the zigzag split balanced."""
import os

import numpy as np
import pytest

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = {}
    part = 0
    tables = [{}, {}]
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if not line:
            continue
        if line.startswith("#"):
            part = 1 if "pairs" in line else 0
            continue
        k, v = line.split(":")
        tables[part][int(k)] = [int(t) for t in v.split()]
    return tables if rows == {} else rows


def test_zigzag_chunk_table_golden():
    chunks, pairs = _read_table("zigzag_cp4.txt")
    for r in range(4):
        assert oracle.rank_chunks(4, r) == chunks[r]
        got = [oracle.count_pairs([0, 256], 4, r, s, oracle.CAUSAL) for s in range(4)]
        assert got == pairs[r]


def test_tf_mask_golden():
    lines = [l.strip() for l in open(os.path.join(GOLD, "tf_mask_N3_B2.txt")) if not l.startswith("#")]
    want = np.array([[c == "1" for c in l] for l in lines if l])
    p = np.arange(12)
    got = oracle.allowed(oracle.TF_BLOCK, p[:, None], p[None, :], 2, 3)
    assert (got == want).all()


@pytest.mark.parametrize("lens,cp", [([256], 4), ([64, 32, 96], 2), ([48, 16, 80, 8], 4), ([40, 24], 1),
                                     ([7, 3], 1)])
def test_partition_is_a_partition(lens, cp):
    cu = np.concatenate([[0], np.cumsum(lens)])
    seen = []
    for r in range(cp):
        cu_l, l2g, pos, seq = oracle.local_rows(cu, cp, r)
        assert cu_l[-1] == len(l2g) == sum(lens) // cp
        assert np.all(np.diff(cu_l) == np.asarray(lens) // cp)
        for b in range(len(lens)):
            rows = l2g[cu_l[b]:cu_l[b + 1]]
            assert np.all(rows >= cu[b]) and np.all(rows < cu[b + 1])
            np.testing.assert_array_equal(rows - cu[b], pos[cu_l[b]:cu_l[b + 1]])
            assert np.all(seq[cu_l[b]:cu_l[b + 1]] == b)
        seen.append(l2g)
    allr = np.sort(np.concatenate(seen))
    np.testing.assert_array_equal(allr, np.arange(sum(lens)))


def test_partition_rejects_indivisible():
    with pytest.raises(ValueError):
        oracle.local_rows([0, 20], 4, 0)


@pytest.mark.parametrize("lens,cp", [([256], 4), ([64, 32, 96], 2), ([48, 16, 80, 8], 4), ([128, 64], 8)])
def test_causal_pairs_closed_form(lens, cp):
    """Per rank: sum_b (L_b^2 + L_b)/(2cp); per step: 2C^2 + C at s = 0 and
    2C^2 at s >= 1, C = L_b/(2cp).  Equal for every rank (the balance the
    zigzag split exists for)."""
    cu = np.concatenate([[0], np.cumsum(lens)])
    for r in range(cp):
        per_step = [oracle.count_pairs(cu, cp, r, s, oracle.CAUSAL) for s in range(cp)]
        want = [sum(2 * (l // (2 * cp)) ** 2 + (l // (2 * cp) if s == 0 else 0) for l in lens)
                for s in range(cp)]
        assert per_step == want
        assert sum(per_step) == sum((l * l + l) // (2 * cp) for l in lens)


def test_config_pair_counts_closed_form():
    """The per-head pair counts of the five workloads, from closed forms
    (causal: sum L(L+1)/2 / cp; teacher forcing: N(N+1) B^2)."""
    W = workloads.WORKLOADS
    c2 = sum(l * (l + 1) // 2 for l in W["packed_varlen"].seqlens)
    assert c2 == 22_395_656
    c3 = sum((l * l + l) // 16 for l in W["long_video"].seqlens)
    assert c3 == 4_294_983_680
    B, N = W["tf_dit"].tf_chunk, W["tf_dit"].tf_num
    assert N * (N + 1) * B * B == 1_518_566_400
    c5 = sum((l * l + l) // 8 for l in W["long_tail"].seqlens)
    assert c5 == 304_747_728
    # brute-force count on the two cheap ones
    assert oracle.count_pairs(W["packed_varlen"].cu_seqlens, 1, 0, 0, oracle.CAUSAL) == c2
    assert sum(oracle.count_pairs(W["tiny_fp32"].cu_seqlens, 4, 0, s, oracle.CAUSAL)
               for s in range(4)) == 8224


def test_tf_pair_count_scaled():
    for B, N in [(3, 4), (13, 12), (8, 1)]:
        assert oracle.count_pairs([0, 2 * N * B], 1, 0, 0, oracle.TF_BLOCK, B, N) == N * (N + 1) * B * B


def test_workload_lengths():
    """Lengths are the seeded draws described in the workloads module."""
    W = workloads.WORKLOADS
    assert W["packed_varlen"].seqlens == (1397, 1079, 2337, 1368, 721, 1768, 4538, 3176)
    lt = W["long_tail"].seqlens
    assert lt[0] == 49152 and sum(lt) == 65536 and all(l % 8 == 0 for l in lt)
    assert all(256 <= l <= 2048 for l in lt[1:])
    assert W["tf_dit"].tokens == 74880 and W["long_video"].tokens == 262144
