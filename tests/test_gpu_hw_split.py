"""GPU parity of the height/width token split (LongCat-Video context-parallel
page; readings in oracle/hw_split.py) through the C ABI: the gather/scatter
round trip is bit-exact against the oracle's index plan, and BIDIR ring
attention over the split shares (forward steps, merge, backward) equals the
fp64 oracle, including shares of odd length."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads  # noqa: E402
from oracle import hw_split  # noqa: E402
from tests._gpu import TOL_GRAD_RELRMS, check_lse, check_out, dev, rel_rms  # noqa: E402


@pytest.fixture(scope="module")
def cpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_varlen_amd as c
    return c


def test_hw_partition_round_trip(cpa):
    frames, H, W, cp, nseq = 3, 6, 10, 4, 2
    split = cpa.cpattn_split_hw(H, W, cp)
    L = frames * H * W
    cu = np.arange(nseq + 1, dtype=np.int32) * L
    rng = np.random.default_rng(2)
    g = dev(rng.standard_normal((nseq * L, 3, 64), dtype=np.float32), torch.bfloat16)
    back = torch.zeros_like(g)
    cu_dev = torch.from_numpy(cu).cuda()
    for r in range(cp):
        loc = torch.empty((nseq * L // cp, 3, 64), dtype=torch.bfloat16, device="cuda")
        cpa.cpattn_partition_hw(g, loc, cu_dev, nseq, frames, H, W, split, r)
        _, l2g, _, _ = hw_split.local_rows(cu, frames, H, W, split, r)
        assert torch.equal(loc.cpu(), g.cpu()[torch.from_numpy(l2g)])
        cpa.cpattn_unpartition_hw(loc, back, cu_dev, nseq, frames, H, W, split, r)
    torch.cuda.synchronize()
    assert torch.equal(back.cpu(), g.cpu())


@pytest.mark.parametrize("frames,H,W,cp,nseq,hq,hkv,d", [(3, 6, 10, 4, 1, 2, 2, 128),     # 45-row shares (odd)
                                                         (4, 8, 8, 8, 2, 4, 2, 128),
                                                         (2, 12, 20, 6, 1, 2, 1, 64)])
def test_hw_split_ring_forward_backward(cpa, frames, H, W, cp, nseq, hq, hkv, d):
    split = cpa.cpattn_split_hw(H, W, cp)
    L = frames * H * W
    cu = np.arange(nseq + 1, dtype=np.int32) * L
    T = nseq * L
    rng = np.random.default_rng(8)
    x = {k: workloads.round_bf16(rng.standard_normal((T, h, d), dtype=np.float32))
         for k, h in (("q", hq), ("k", hkv), ("v", hkv), ("dout", hq))}
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    cu_dev = torch.from_numpy(cu).cuda()
    loc = {}
    for r in range(cp):
        for k in g:
            t = torch.empty((T // cp,) + tuple(g[k].shape[1:]), dtype=torch.bfloat16, device="cuda")
            cpa.cpattn_partition_hw(g[k], t, cu_dev, nseq, frames, H, W, split, r)
            loc[(k, r)] = t
    seq = np.repeat(np.arange(nseq), L)
    pos = np.tile(np.arange(L), nseq)
    from context_attention_varlen_amd.ring import ForwardBuffers, RankPlan, ring_backward, ring_forward
    for r in sorted({0, cp - 1}):
        cu_l, _ = cpa.cpattn_partition_index_hw(cu, frames, H, W, split, r, with_map=False)
        plan = RankPlan(cp, r, cu, cu_l, cu_dev, torch.from_numpy(cu_l).cuda(), nseq, int(cu_l[-1]))
        ks = [loc[("k", j)] for j in range(cp)]
        vs = [loc[("v", j)] for j in range(cp)]
        bufs, _ = ring_forward(loc[("q", r)], ks, vs, plan, oracle.BIDIR)
        dq, dk, dv, _ = ring_backward(loc[("q", r)], ks, vs, loc[("dout", r)], bufs, plan, oracle.BIDIR)
        torch.cuda.synchronize()
        _, l2g, qpos, qseq = hw_split.local_rows(cu, frames, H, W, split, r)
        o_ref, l_ref = oracle.attention(x["q"][l2g], x["k"], x["v"], qseq, qpos, seq, pos, oracle.BIDIR)
        check_out(bufs.out.cpu().numpy(), o_ref, "bf16")
        check_lse(bufs.lse.cpu().numpy(), l_ref)
        delta = oracle.bwd_delta(o_ref, x["dout"][l2g])
        dq_ref = np.zeros_like(o_ref)
        for s in range(cp):
            j = oracle.step_source(cp, r, s)
            _, k2g, kpos, kseq = hw_split.local_rows(cu, frames, H, W, split, j)
            a, b, c = oracle.attention_backward(x["q"][l2g], x["k"][k2g], x["v"][k2g], x["dout"][l2g], l_ref, delta,
                                                qseq, qpos, kseq, kpos, oracle.BIDIR)
            dq_ref += a
            assert rel_rms(dk[j].cpu().numpy(), b) <= TOL_GRAD_RELRMS, j
            assert rel_rms(dv[j].cpu().numpy(), c) <= TOL_GRAD_RELRMS, j
        assert rel_rms(dq.cpu().numpy(), dq_ref) <= TOL_GRAD_RELRMS
