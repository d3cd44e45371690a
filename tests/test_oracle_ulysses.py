"""Pins of the one-device Ulysses exchange (oracle/ulysses.py): exact round
trip, equality with the head slice of the unsharded tensor, and that
attention on a gathered head group equals that head group of attention on
the whole batch (heads are independent; GQA groups stay aligned when the
group size divides the kv-head count)."""
import numpy as np
import pytest

import oracle
from oracle import ulysses
from tests._tiny import tiny_inputs


@pytest.mark.parametrize("lens,n,H", [([8, 8, 8, 8], 4, 8), ([5, 11, 3], 3, 6), ([16], 1, 4), ([7, 9], 2, 2)])
def test_round_trip_bit_exact(lens, n, H):
    rng = np.random.default_rng(5)
    shards = [rng.standard_normal((t, H, 4)).astype(np.float32) for t in lens]
    blank = [np.zeros_like(s) for s in shards]
    for g in range(n):
        x = ulysses.seq_to_head(shards, g, n)
        assert x.shape == (sum(lens), H // n, 4)
        blank = ulysses.head_to_seq(x, g, n, blank)
    for a, b in zip(blank, shards):
        assert np.array_equal(a, b)


def test_gather_is_the_global_head_slice():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((48, 12, 8))
    for n in (2, 3, 4, 6):
        shards = ulysses.contiguous_shards(x, n)
        for g in range(n):
            hg = 12 // n
            assert np.array_equal(ulysses.seq_to_head(shards, g, n), x[:, g * hg:(g + 1) * hg])


@pytest.mark.parametrize("mode", [oracle.CAUSAL, oracle.BIDIR])
def test_head_group_attention_equals_full(mode):
    lens = [24, 40]
    n, hq, hkv = 2, 4, 2
    x = tiny_inputs(9, lens, hq, hkv, 8)
    full_o, full_l = oracle.attention(x["q"], x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"], mode)
    for g in range(n):
        q = ulysses.seq_to_head(ulysses.contiguous_shards(x["q"], n), g, n)
        k = ulysses.seq_to_head(ulysses.contiguous_shards(x["k"], n), g, n)
        v = ulysses.seq_to_head(ulysses.contiguous_shards(x["v"], n), g, n)
        o, l = oracle.attention(q, k, v, x["seq"], x["pos"], x["seq"], x["pos"], mode)
        hg = hq // n
        np.testing.assert_allclose(o, full_o[:, g * hg:(g + 1) * hg], atol=1e-12)
        np.testing.assert_allclose(l, full_l[g * hg:(g + 1) * hg], atol=1e-12)


def test_indivisible_heads_rejected():
    with pytest.raises(ValueError):
        ulysses.seq_to_head([np.zeros((4, 6, 2))], 0, 4)
