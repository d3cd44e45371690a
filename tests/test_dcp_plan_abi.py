"""Parity of the native Dynamic-CP planner (cpattn_dcp_plan_batch,
cpattn_dcp_quotas; host code, no GPU) with the oracle
(oracle/dynamic_cp.py): every integer decision bit-exact, doubles equal to
the correctly rounded exact values.  "Speeding up Variable-Length Training
with Dynamic Context Parallelism and NVIDIA Megatron Core", sections A2 and
A7."""
import numpy as np
import pytest

import context_attention_varlen_amd as cpa
from oracle import dynamic_cp as dc
import workloads


def _compare(lengths, gpus, max_cp, pp, vpp, mem, a, b, m_min, m_max, radius):
    L = [int(x) for x in lengths]
    o = dc.plan(L, gpus, max_cp, pp, vpp, mem, a, b, m_min, m_max, radius)
    if o is None:
        with pytest.raises(cpa.CpattnError) as e:
            cpa.cpattn_dcp_plan_batch(L, gpus, max_cp, pp, vpp, mem, a, b, m_min, m_max, radius)
        assert e.value.status == cpa.ERR_INFEASIBLE
        return None
    r = cpa.cpattn_dcp_plan_batch(L, gpus, max_cp, pp, vpp, mem, a, b, m_min, m_max, radius)
    assert r["m"] == o["m"] and r["knee"] == o["knee"]
    assert r["step_time"] == float(o["time"]) / max_cp
    bks = o["buckets"]
    assert r["num_buckets"] == len(bks)
    assert list(r["cp"]) == [bk.cp for bk in bks]
    assert list(r["slot"]) == [bk.slot for bk in bks]
    assert list(r["rank"]) == [bk.gpu for bk in bks]
    assert list(r["tokens"]) == [bk.tokens for bk in bks]
    assert list(r["load"]) == [float(bk.load) for bk in bks]
    own = np.full(len(L), -1)
    for j, bk in enumerate(bks):
        own[bk.samples] = j
    assert np.array_equal(r["sample_bucket"], own)
    ms = range(m_min, m_max + 1)
    want_t = [(-2.0 if m not in o["times"] else -1.0 if o["times"][m] is None else float(o["times"][m]) / max_cp)
              for m in ms]
    assert list(r["times"]) == want_t
    assert list(r["budget"]) == dc.budget_curve(L, gpus, max_cp, a, b, m_min, m_max)
    return r


CASES = [
    # gpus, max_cp, pp, vpp, mem, a, b, m_min, m_max, radius
    (8, 4, 2, 2, 16384, 1, 2000, 2, 8, -1),
    (16, 8, 4, 1, 8192, 1, 0, 4, 16, 2),
    (4, 4, 1, 1, 32768, 3, 100000, 1, 6, -1),
    (64, 8, 4, 2, 16384, 1, 4096, 4, 16, 1),
    (2, 1, 2, 3, 10**6, 0, 1, 1, 4, -1),          # linear workload, no split
    (32, 32, 8, 1, 4096, 1, 0, 8, 24, 0),           # knee only
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("seed", range(4))
def test_plan_matches_oracle(case, seed):
    rng = np.random.default_rng(seed * 31 + case)
    n = int(rng.integers(1, 400))
    lengths = np.minimum(rng.lognormal(7.0, 1.4, n).astype(np.int64) + 1, 200000)
    _compare(lengths, *CASES[case])


def test_plan_long_tail_batch():
    """A batch drawn like the long-tail microbatch workload (one long sample
    plus many short ones), repeated eight times."""
    w = workloads.WORKLOADS["long_tail"]
    lens = np.diff(np.asarray(w.cu_seqlens)).tolist() * 8
    r = _compare(lens, 32, 8, 4, 2, 16384, 1, 8192, 4, 16, -1)
    assert r is not None and max(r["cp"]) == 8


@pytest.mark.parametrize("mem,gpus,lo,hi", [(16384, 64, 4, 16), (32768, 64, 2, 12), (20000, 128, 2, 10)])
def test_plan_larger_batch(mem, gpus, lo, hi):
    """1500 long-tail samples (9.1M tokens): infeasible and feasible m side by
    side, memory-bound cp = 1 microbatches (the least-loaded one often lacks
    room), many split microbatches of every size."""
    lens = workloads.global_batch_lengths(seed=3, n=1500)
    r = _compare(lens, gpus, 8, 2, 1, mem, 1, 0, lo, hi, -1)
    assert r is not None and set(r["cp"]) == {1, 2, 4, 8}


@pytest.mark.parametrize("lengths,cfg", [
    ([1], (1, 1, 1, 1, 1, 1, 0, 1, 1, -1)),                    # smallest problem
    ([5, 5, 5, 5], (2, 2, 1, 1, 10, 1, 0, 1, 3, -1)),          # ties everywhere
    ([100000, 10], (4, 4, 1, 1, 1000, 1, 0, 1, 4, -1)),        # over the cap even at max_cp
    ([64] * 10, (4, 4, 2, 2, 16, 1, 0, 1, 2, -1)),             # memory forces every sample to split
    ([3, 3, 2, 2, 2], (1, 1, 2, 1, 100, 0, 1, 2, 2, -1)),      # Graham's tight instance
])
def test_plan_edge_cases(lengths, cfg):
    _compare(lengths, *cfg)


@pytest.mark.parametrize("bad", [
    dict(gpus=6, max_cp=4), dict(max_cp=3), dict(max_cp=16), dict(pp=0), dict(vpp=0), dict(mem=0),
    dict(a=0, b=0), dict(a=-1), dict(m_min=0), dict(m_min=5, m_max=4), dict(m_max=5000),
])
def test_plan_rejects_bad_config(bad):
    cfg = dict(gpus=8, max_cp=4, pp=2, vpp=2, mem=4096, a=1, b=0, m_min=1, m_max=4)
    cfg.update(bad)
    with pytest.raises(cpa.CpattnError) as e:
        cpa.cpattn_dcp_plan_batch([100, 200], cfg["gpus"], cfg["max_cp"], cfg["pp"], cfg["vpp"], cfg["mem"],
                                  cfg["a"], cfg["b"], cfg["m_min"], cfg["m_max"])
    assert e.value.status == cpa.ERR_INVALID_ARG


def test_plan_rejects_bad_lengths():
    for L in ([0, 5], [-3], [1 << 23]):
        with pytest.raises(cpa.CpattnError) as e:
            cpa.cpattn_dcp_plan_batch(L, 4, 2, 1, 1, 10**6, 1, 0, 1, 2)
        assert e.value.status == cpa.ERR_INVALID_ARG


@pytest.mark.parametrize("seed", range(5))
def test_quotas_match_oracle(seed):
    """Double-precision Eq. 1-3 against the exact fractions: n + 3 rounded
    operations per quota bound the relative error by (n + 3) 2^-53."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 64))
    m = rng.integers(1, 32, n)
    V, p, total = int(rng.integers(1, 4)), int(rng.integers(1, 9)), float(rng.integers(1, 10**12))
    got = cpa.cpattn_dcp_quotas(m, V, p, total)
    want = np.array([float(x) for x in dc.quotas([int(v) for v in m], V, p, int(total))])
    np.testing.assert_allclose(got, want, rtol=(n + 3) * 2.0**-53, atol=0)


def test_quotas_reject_bad_args():
    for m, V, p, t in (([0, 1], 1, 1, 1.0), ([1], 0, 1, 1.0), ([1], 1, 0, 1.0), ([1], 1, 1, -1.0),
                       ([1], 1, 1, float("nan"))):
        with pytest.raises(cpa.CpattnError):
            cpa.cpattn_dcp_quotas(m, V, p, t)
