"""Pins of the height/width token split (oracle/hw_split.py; LongCat-Video
context-parallel page, split_tensor_in_cp_2d / get_optimal_split, with the
readings stated in hw_split.py)."""
import itertools
import os

import numpy as np
import pytest

import oracle
from oracle import hw_split
from tests._tiny import tiny_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hw_split.txt")


def test_golden_splits():
    n = 0
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        H, W, cp, sh, sw = (int(v) for v in line.split()[:5])
        th, tw = (float(v) for v in line.split()[5:])
        assert hw_split.optimal_split(H, W, cp) == (sh, sw)
        assert (H / sh, W / sw) == (th, tw)
        n += 1
    assert n == 8


@pytest.mark.parametrize("H,W,cp", [(12, 20, 4), (9, 16, 6), (30, 32, 8), (7, 14, 2), (24, 36, 12)])
def test_split_is_the_squarest_even_split(H, W, cp):
    """Brute force over every (a, b) with a*b = cp, written independently."""
    cands = [(a, b) for a, b in itertools.product(range(1, cp + 1), repeat=2)
             if a * b == cp and H % a == 0 and W % b == 0]
    sh, sw = hw_split.optimal_split(H, W, cp)
    assert (sh, sw) in cands
    for a, b in cands:
        assert abs(H / sh - W / sw) <= abs(H / a - W / b)


def test_no_even_split_is_rejected():
    with pytest.raises(ValueError):
        hw_split.optimal_split(30, 30, 8)     # neither 4 nor 8 divides 30


@pytest.mark.parametrize("frames,H,W,cp,nseq", [(2, 4, 6, 4, 1), (3, 6, 4, 6, 2), (1, 8, 8, 8, 1), (2, 5, 6, 2, 2)])
def test_rows_partition_and_tiles(frames, H, W, cp, nseq):
    L = frames * H * W
    cu = np.arange(nseq + 1, dtype=np.int32) * L
    split = hw_split.optimal_split(H, W, cp)
    th, tw = H // split[0], W // split[1]
    seen = []
    for r in range(cp):
        cu_l, l2g, pos, seq = hw_split.local_rows(cu, frames, H, W, split, r)
        assert list(cu_l) == [b * L // cp for b in range(nseq + 1)]
        f, rem = pos // (H * W), pos % (H * W)
        h, w = rem // W, rem % W
        # one rectangular cell per frame, rows top to bottom and left to right
        assert set(np.unique(h // th)) == {r // split[1]} and set(np.unique(w // tw)) == {r % split[1]}
        assert np.all(np.diff(pos[seq == 0]) > 0)
        assert np.bincount(f[seq == 0], minlength=frames).tolist() == [th * tw] * frames
        seen.append(l2g)
    assert np.array_equal(np.sort(np.concatenate(seen)), np.arange(nseq * L))


def test_ring_merge_equals_full_bidir():
    frames, H, W, cp = 2, 4, 6, 4
    L = frames * H * W
    x = tiny_inputs(31, [L, L], 2, 1, 8)
    cu = x["cu"]
    split = hw_split.optimal_split(H, W, cp)
    full_o, full_l = oracle.attention(x["q"], x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"], oracle.BIDIR)
    for r in range(cp):
        _, l2g, qpos, qseq = hw_split.local_rows(cu, frames, H, W, split, r)
        out = np.zeros((len(l2g), 2, 8))
        lse = np.full((2, len(l2g)), -np.inf)
        for s in range(cp):
            _, k2g, kpos, kseq = hw_split.local_rows(cu, frames, H, W, split, oracle.step_source(cp, r, s))
            op, lp = oracle.attention(x["q"][l2g], x["k"][k2g], x["v"][k2g], qseq, qpos, kseq, kpos, oracle.BIDIR)
            out, lse = oracle.merge(out, lse, op, lp)
        np.testing.assert_allclose(out, full_o[l2g], atol=1e-12)
        np.testing.assert_allclose(lse, full_l[:, l2g], atol=1e-12)


def test_width_major_cells_are_caught(monkeypatch):
    """Planted mistake: numbering grid cells width-outer breaks the cell
    check of the partition test."""
    real = hw_split.local_rows

    def swapped(cu, frames, H, W, split, r):
        sh, sw = split
        return real(cu, frames, H, W, split, (r % sh) * sw + r // sh)
    monkeypatch.setattr(hw_split, "local_rows", swapped)
    with pytest.raises(AssertionError):
        test_rows_partition_and_tiles(2, 4, 6, 4, 1)
