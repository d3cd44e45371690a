"""A Dynamic-CP plan executed on the attention path ("Speeding up
Variable-Length Training with Dynamic Context Parallelism and NVIDIA Megatron
Core", sections A2 and A7: every microbatch runs with its own cp size).

A small long-tail batch is planned by cpattn_dcp_plan_batch; every
microbatch is then run at its cp size through the C ABI, rank by rank of its
group (partition, ring forward with merges, ring backward), the rank shares
are scattered back, and every sample's output, LSE and gradients must equal
the fp64 oracle's unsplit causal attention of that sample alone."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads  # noqa: E402
from tests._gpu import TOL_GRAD_RELRMS, check_lse, check_out, dev, rel_rms  # noqa: E402


@pytest.fixture(scope="module")
def cpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_varlen_amd as c
    return c


def _run_microbatch(cpa, lens, cp, x):
    """Out [T,Hq,d], LSE [Hq,T], dQ, dK, dV of one microbatch (global row
    order) computed as cp ranks."""
    from context_attention_varlen_amd.ring import RankPlan, partition, ring_backward, ring_forward
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    hq, d = x["q"].shape[1:]
    hkv = x["k"].shape[1]
    out = np.zeros((T, hq, d))
    lse = np.zeros((hq, T))
    dq = np.zeros((T, hq, d))
    dk = np.zeros((T, hkv, d))
    dv = np.zeros((T, hkv, d))
    maps = [cpa.cpattn_partition_index(cu, cp, j)[1] for j in range(cp)]
    for r in range(cp):
        plan = RankPlan.make(cu, cp, r)
        q = partition(g["q"], plan)
        do = partition(g["dout"], plan)
        ks = [partition(g["k"], plan, j) for j in range(cp)]
        vs = [partition(g["v"], plan, j) for j in range(cp)]
        bufs, _ = ring_forward(q, ks, vs, plan, oracle.CAUSAL)
        gq, gk, gv, _ = ring_backward(q, ks, vs, do, bufs, plan, oracle.CAUSAL)
        torch.cuda.synchronize()
        l2g = maps[r]
        out[l2g] = bufs.out.cpu().numpy()
        lse[:, l2g] = bufs.lse.cpu().numpy()
        dq[l2g] = gq.cpu().numpy()
        for j in range(cp):
            dk[maps[j]] += gk[j].cpu().numpy()
            dv[maps[j]] += gv[j].cpu().numpy()
    return out, lse, dq, dk, dv


@pytest.mark.parametrize("seed", [0, 2])
def test_planned_batch_equals_oracle(cpa, seed):
    rng = np.random.default_rng(seed)
    lens = workloads.global_batch_lengths(seed=seed, n=14, mu=6.0, sigma=0.9, cap=3072, quantum=16)
    hq, hkv, d = 4, 2, 64
    plan = cpa.cpattn_dcp_plan_batch(lens, 4, 4, 1, 1, 1024, 1, 0, 1, 8)
    assert plan["cp"].max() > 1 and plan["cp"].min() == 1       # both split and unsplit microbatches
    seen = 0
    for b in range(plan["num_buckets"]):
        idx = np.flatnonzero(plan["sample_bucket"] == b)
        if len(idx) == 0:
            continue
        blens = [lens[i] for i in idx]
        cp = int(plan["cp"][b])
        T = sum(blens)
        x = {k: workloads.round_bf16(rng.standard_normal((T, h, d), dtype=np.float32))
             for k, h in (("q", hq), ("k", hkv), ("v", hkv), ("dout", hq))}
        out, lse, dq, dk, dv = _run_microbatch(cpa, blens, cp, x)
        start = 0
        for L in blens:
            sl = slice(start, start + L)
            pos = np.arange(L)
            seq = np.zeros(L, np.int64)
            o_r, l_r = oracle.attention(x["q"][sl], x["k"][sl], x["v"][sl], seq, pos, seq, pos, oracle.CAUSAL)
            check_out(out[sl], o_r, "bf16")
            check_lse(lse[:, sl], l_r)
            delta = oracle.bwd_delta(o_r, x["dout"][sl])
            gq, gk, gv = oracle.attention_backward(x["q"][sl], x["k"][sl], x["v"][sl], x["dout"][sl], l_r, delta,
                                                   seq, pos, seq, pos, oracle.CAUSAL)
            assert rel_rms(dq[sl], gq) <= TOL_GRAD_RELRMS
            assert rel_rms(dk[sl], gk) <= TOL_GRAD_RELRMS
            assert rel_rms(dv[sl], gv) <= TOL_GRAD_RELRMS
            start += L
            seen += 1
    assert seen == len(lens)
