"""The ring step under HIP graph capture.

Every call of the hot path only enqueues kernels on the caller's stream: no
allocation, no memset, no host synchronisation.  So a whole rank step
(cp forward steps with their merges, the backward preprocess and cp backward
steps, plus the torch fills that reset the buffers) can be captured once and
replayed.  Replays are interleaved with unrelated eager work and host
synchronisation, and every replay must reproduce the eager results bit for
bit (the kernels use no atomics, so the result does not depend on timing)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads  # noqa: E402
from tests._gpu import dev  # noqa: E402


@pytest.fixture(scope="module")
def cpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_varlen_amd as c
    return c


@pytest.mark.parametrize("lens,cp,mode", [([512, 96, 160], 2, oracle.CAUSAL), ([384, 128], 4, oracle.CAUSAL),
                                          ([300, 77], 1, oracle.BIDIR)])
def test_graph_replay_matches_eager(cpa, lens, cp, mode):
    from context_attention_varlen_amd.ring import ForwardBuffers, RankPlan, partition, ring_backward, ring_forward
    hq, hkv, d = 4, 2, 128
    rng = np.random.default_rng(5)
    T = sum(lens)
    x = {k: dev(workloads.round_bf16(rng.standard_normal((T, h, d), dtype=np.float32)), torch.bfloat16)
         for k, h in (("q", hq), ("k", hkv), ("v", hkv), ("dout", hq))}
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    plan = RankPlan.make(cu, cp, 0)
    q = partition(x["q"], plan)
    do = partition(x["dout"], plan)
    ks = [partition(x["k"], plan, j) for j in range(cp)]
    vs = [partition(x["v"], plan, j) for j in range(cp)]
    bufs = ForwardBuffers.make(q, ks[0].shape[0], plan.num_seqs)
    grads = (torch.zeros((q.shape[0], hq, d), dtype=torch.float32, device="cuda"),
             [torch.zeros(k.shape, dtype=torch.float32, device="cuda") for k in ks],
             [torch.zeros(k.shape, dtype=torch.float32, device="cuda") for k in ks],
             torch.empty((hq, q.shape[0]), dtype=torch.float32, device="cuda"))

    def step():
        bufs.reset()
        ring_forward(q, ks, vs, plan, mode, bufs=bufs)
        ring_backward(q, ks, vs, do, bufs, plan, mode, grads=grads)

    def snapshot():
        return [t.clone() for t in (bufs.out, bufs.lse, grads[0], *grads[1], *grads[2], grads[3])]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # eager run on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    want = snapshot()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (bufs.out, grads[0], *grads[1], *grads[2]):
            t.fill_(123.0)                       # stale values the replay must overwrite / reset
        g.replay()
        noise = torch.randn(1 << 20, device="cuda").mul_(2.0)   # unrelated eager work
        torch.cuda.synchronize()
        got = snapshot()
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager run"
        del noise


@pytest.mark.parametrize("lens,cp,mode,tf", [([512, 96, 160], 2, oracle.CAUSAL, (0, 0)),
                                             ([384, 128, 0, 64], 4, oracle.CAUSAL, (0, 0)),
                                             ([300, 77], 1, oracle.BIDIR, (0, 0)),
                                             ([2 * 40 * 6], 3, oracle.TF_BLOCK, (40, 6))])
def test_overlapped_rank_step(cpa, lens, cp, mode, tf):
    """ring.rank_step with its second stream (K/V gathers, dO gather, fills and
    merges beside the forward steps) gives bit for bit what the same call on
    one stream gives, eagerly and as a graph replayed three times; the one-
    stream call is checked against the oracle."""
    from context_attention_varlen_amd.ring import RankPlan, StepBuffers, rank_step
    from tests._gpu import check_lse, check_out
    from tests.test_gpu_bwd import _check_grad, oracle_grads
    hq, hkv, d = 4, 2, 128
    rng = np.random.default_rng(11)
    T = sum(lens)
    xs = {k: workloads.round_bf16(rng.standard_normal((T, h, d), dtype=np.float32))
          for k, h in (("q", hq), ("k", hkv), ("v", hkv), ("dout", hq))}
    x = {k: dev(v, torch.bfloat16) for k, v in xs.items()}
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    plan = RankPlan.make(cu, cp, cp - 1, tf=tf if tf[0] else None)
    b = StepBuffers.make(plan, hq, hkv, d, torch.bfloat16, backward=True)

    def snapshot():
        return [t.clone() for t in (b.fwd.out, b.fwd.lse, b.dq, *b.dk, *b.dv, b.delta)]

    rank_step(x["q"], x["k"], x["v"], x["dout"], plan, mode, b)
    torch.cuda.synchronize()
    want = snapshot()
    if not tf[0]:
        _, l2g, qpos, qseq = oracle.local_rows(cu, cp, cp - 1)
        seq = np.repeat(np.arange(len(cu) - 1), np.diff(cu))
        pos = np.arange(T) - cu[seq]
        o_ref, l_ref = oracle.attention(xs["q"][l2g], xs["k"], xs["v"], qseq, qpos, seq, pos, mode)
        check_out(want[0].cpu().numpy(), o_ref, "bf16")
        check_lse(want[1].cpu().numpy(), l_ref)
        dq_r, dk_r, dv_r, _ = oracle_grads(xs, cu, cp, cp - 1, mode, (0, 0))
        _check_grad(b.dq.cpu().numpy(), dq_r, "dq")
        for j in range(cp):
            _check_grad(b.dk[j].cpu().numpy(), dk_r[j], f"dk[{j}]")
            _check_grad(b.dv[j].cpu().numpy(), dv_r[j], f"dv[{j}]")

    side = torch.cuda.Stream()
    for t in (b.fwd.out, b.dq, *b.dk, *b.dv):
        t.fill_(7.0)
    rank_step(x["q"], x["k"], x["v"], x["dout"], plan, mode, b, side=side)
    torch.cuda.synchronize()
    for a, w_ in zip(snapshot(), want):
        assert torch.equal(a, w_), "the overlapped step differs from the one-stream step"

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        rank_step(x["q"], x["k"], x["v"], x["dout"], plan, mode, b, side=side)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rank_step(x["q"], x["k"], x["v"], x["dout"], plan, mode, b, side=side)
    for rep in range(3):
        for t in (b.fwd.out, b.fwd.lse, b.dq, *b.dk, *b.dv):
            t.fill_(123.0)
        g.replay()
        noise = torch.randn(1 << 20, device="cuda").mul_(2.0)   # unrelated eager work
        torch.cuda.synchronize()
        for a, w_ in zip(snapshot(), want):
            assert torch.equal(a, w_), f"replay {rep} of the overlapped step differs"
        del noise
