"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
catch each one: a wrong scale, an off-by-one causal mask, a wrong GQA head
map, a dropped delta term in the backward and a wrong merge weight."""
import math

import numpy as np
import pytest

import oracle
import oracle.lse_merge as omerge
import oracle.masks as omask
import oracle.softmax_attention as oatt
from oracle.brute import brute_attention
from tests._tiny import pred_causal, tiny_inputs


def _brute_ok(lens=(9, 6), hq=4, hkv=2, d=4):
    x = tiny_inputs(31, list(lens), hq, hkv, d)
    o, l = oatt.attention(x["q"], x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"], 0)
    cu = x["cu"]
    seqs = [(list(range(cu[b], cu[b + 1])), list(range(n)), list(range(cu[b], cu[b + 1])), list(range(n)))
            for b, n in enumerate(lens)]
    bo, bl = brute_attention(x["q"].tolist(), x["k"].tolist(), x["v"].tolist(), seqs, pred_causal,
                             1 / math.sqrt(d))
    return np.allclose(o, bo, atol=1e-12) and np.allclose(l, bl, atol=1e-12)


def test_unplanted_passes():
    assert _brute_ok()


def test_wrong_scale_is_caught(monkeypatch):
    monkeypatch.setattr(oatt, "default_scale", lambda d: 1.0 / d)
    assert not _brute_ok()


def test_off_by_one_causal_is_caught(monkeypatch):
    orig = omask.allowed

    def bad(mode, pq, pk, *a):
        if mode == 0:
            return np.asarray(pk) < np.asarray(pq)
        return orig(mode, pq, pk, *a)
    monkeypatch.setattr(oatt, "allowed", bad)
    assert not _brute_ok()


def test_wrong_gqa_map_is_caught(monkeypatch):
    # interleaved instead of contiguous groups
    monkeypatch.setattr(oatt, "kv_head", lambda h, hq, hkv: h % hkv)
    assert not _brute_ok()


def test_dropped_delta_is_caught():
    x = tiny_inputs(32, [8], 2, 2, 4, dout=True)
    o, l = oracle.attention(x["q"], x["k"], x["v"], x["seq"], x["pos"], x["seq"], x["pos"], 0)
    good = oracle.attention_backward(x["q"], x["k"], x["v"], x["dout"], l, oracle.bwd_delta(o, x["dout"]),
                                     x["seq"], x["pos"], x["seq"], x["pos"], 0)
    bad = oracle.attention_backward(x["q"], x["k"], x["v"], x["dout"], l, np.zeros_like(l),
                                    x["seq"], x["pos"], x["seq"], x["pos"], 0)
    # the invariant sum_j dK_j = 0 holds for the good one and fails for the bad one
    assert np.allclose(good[1].sum(0), 0.0, atol=1e-12)
    assert not np.allclose(bad[1].sum(0), 0.0, atol=1e-6)


def test_wrong_merge_weight_is_caught(monkeypatch):
    rng = np.random.default_rng(0)
    o1, o2 = rng.standard_normal((3, 2, 4)), rng.standard_normal((3, 2, 4))
    l1 = rng.standard_normal((2, 3))
    # a merge that forgets to renormalise the weights
    monkeypatch.setattr(omerge.np, "log", lambda x: np.zeros_like(x))
    o, lm = omerge.merge(o1, l1, o2, l1)
    assert not np.allclose(o, (o1 + o2) / 2)
