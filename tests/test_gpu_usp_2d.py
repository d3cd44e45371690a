"""Ulysses x ring (the 2D-Attention / USP mesh) composed on one GPU
("Scaling Video Training with Parallelism", SP landscape: USP / LoongTrain
run Ulysses inside a group and the ring across groups).

The sequence is zigzag-split over the ring ranks; inside a ring rank, its
local tokens are further split into contiguous Ulysses shards (all heads).
Member g of the Ulysses group gathers head group g of every shard
(cpattn_seq_to_head), runs the ring over the ring ranks for those heads,
and the output goes back into the token shards (cpattn_head_to_seq).  The
reassembled output and LSE of every ring rank must equal the fp64 oracle's
attention over that rank's rows, all heads."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads  # noqa: E402
from tests._gpu import check_lse, check_out, dev  # noqa: E402


@pytest.fixture(scope="module")
def cpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_varlen_amd as c
    return c


@pytest.mark.parametrize("lens,ring,u,hq,hkv", [([512, 256], 2, 2, 4, 2), ([384, 128, 256], 2, 4, 8, 4),
                                                 ([768], 3, 2, 6, 2)])
def test_ulysses_times_ring(cpa, lens, ring, u, hq, hkv):
    from context_attention_varlen_amd.ring import RankPlan, partition, ring_forward
    d = 128
    rng = np.random.default_rng(31)
    T = sum(lens)
    x = {k: workloads.round_bf16(rng.standard_normal((T, h, d), dtype=np.float32))
         for k, h in (("q", hq), ("k", hkv), ("v", hkv))}
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    seq = np.repeat(np.arange(len(lens)), lens)
    pos = np.arange(T) - cu[seq]
    plans = [RankPlan.make(cu, ring, j) for j in range(ring)]
    loc = {k: [partition(g[k], plans[j]) for j in range(ring)] for k in ("q", "k", "v")}
    for rho in range(ring):
        tl = plans[rho].tokens_local
        assert tl % u == 0
        # every ring rank's local tokens as u contiguous Ulysses shards, all heads
        shards = {k: [list(loc[k][j].split(tl // u)) for j in range(ring)] for k in ("q", "k", "v")}
        out_shards = [torch.zeros((tl // u, hq, d), dtype=torch.float32, device="cuda") for _ in range(u)]
        lse = torch.empty((hq, tl), dtype=torch.float32, device="cuda")
        for grp in range(u):
            def gather(k, j, h):
                t = torch.empty((tl, h // u, d), dtype=torch.bfloat16, device="cuda")
                cpa.cpattn_seq_to_head(shards[k][j], grp, t)
                return t
            q = gather("q", rho, hq)
            ks = [gather("k", j, hkv) for j in range(ring)]
            vs = [gather("v", j, hkv) for j in range(ring)]
            bufs, _ = ring_forward(q, ks, vs, plans[rho], oracle.CAUSAL)
            cpa.cpattn_head_to_seq(bufs.out, grp, out_shards)
            lse[grp * (hq // u):(grp + 1) * (hq // u)] = bufs.lse
        torch.cuda.synchronize()
        _, l2g, qpos, qseq = oracle.local_rows(cu, ring, rho)
        o_ref, l_ref = oracle.attention(x["q"][l2g], x["k"], x["v"], qseq, qpos, seq, pos, oracle.CAUSAL)
        check_out(torch.cat(out_shards).cpu().numpy(), o_ref, "bf16")
        check_lse(lse.cpu().numpy(), l_ref)
