"""GPU parity of the balanced teacher-forcing split at cp > 1 ("Scaling Video
Training with Parallelism", section 4, balanced SP) through the C ABI: the
partition round trip (bit-exact), every ring step's partial result, the
merged result, and the backward, against the fp64 oracle with its own split
(oracle/tf_split.py)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads  # noqa: E402
from oracle import tf_split  # noqa: E402
from tests._gpu import TOL_GRAD_RELRMS, check_lse, check_out, dev, rel_rms, tdtype  # noqa: E402


@pytest.fixture(scope="module")
def cpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_varlen_amd as c
    return c


def _inputs(seed, nseq, B, N, hq, hkv, d, dtype):
    rng = np.random.default_rng(seed)
    T = nseq * 2 * B * N
    x = {"q": rng.standard_normal((T, hq, d), dtype=np.float32),
         "k": rng.standard_normal((T, hkv, d), dtype=np.float32),
         "v": rng.standard_normal((T, hkv, d), dtype=np.float32),
         "dout": rng.standard_normal((T, hq, d), dtype=np.float32)}
    if dtype == "bf16":
        x = {k: workloads.round_bf16(v) for k, v in x.items()}
    cu = np.arange(nseq + 1, dtype=np.int32) * (2 * B * N)
    return x, cu


def _oracle_rank(x, cu, cp, r, B, N):
    """Per-step partials, merged (out, lse) from unsplit attention, and the
    per-source gradients of rank r."""
    _, l2g, qpos, qseq = tf_split.local_rows(cu, cp, r, B, N)
    T = int(cu[-1])
    seq = np.repeat(np.arange(len(cu) - 1), np.diff(cu))
    pos = np.arange(T) - cu[seq]
    o, lse = oracle.attention(x["q"][l2g], x["k"], x["v"], qseq, qpos, seq, pos, oracle.TF_BLOCK,
                              tf_chunk=B, tf_num=N)
    delta = oracle.bwd_delta(o, x["dout"][l2g])
    steps, dks, dvs = [], {}, {}
    dq = np.zeros((len(l2g),) + x["q"].shape[1:])
    for s in range(cp):
        j = oracle.step_source(cp, r, s)
        _, k2g, kpos, kseq = tf_split.local_rows(cu, cp, j, B, N)
        steps.append(oracle.attention(x["q"][l2g], x["k"][k2g], x["v"][k2g], qseq, qpos, kseq, kpos,
                                      oracle.TF_BLOCK, tf_chunk=B, tf_num=N))
        a, b, c = oracle.attention_backward(x["q"][l2g], x["k"][k2g], x["v"][k2g], x["dout"][l2g], lse, delta,
                                            qseq, qpos, kseq, kpos, oracle.TF_BLOCK, tf_chunk=B, tf_num=N)
        dq += a
        dks[j], dvs[j] = b, c
    return steps, (o, lse), dq, dks, dvs, delta


CASES = [
    # nseq, B, N, cp, hq, hkv, d, dtype
    (1, 64, 4, 2, 2, 2, 128, "bf16"),
    (2, 96, 6, 3, 4, 2, 128, "bf16"),
    (1, 37 + 27, 12, 4, 2, 1, 128, "bf16"),     # N not a multiple of 2cp: a partial dealing round
    (1, 80, 6, 3, 2, 2, 64, "bf16"),
    (1, 48, 4, 2, 2, 1, 64, "f32"),
]


@pytest.mark.parametrize("nseq,B,N,cp,hq,hkv,d,dtype", CASES)
def test_tf_split_forward_backward(cpa, nseq, B, N, cp, hq, hkv, d, dtype):
    from context_attention_varlen_amd.ring import RankPlan, partition, ring_backward, ring_forward
    x, cu = _inputs(7, nseq, B, N, hq, hkv, d, dtype)
    td = tdtype(dtype)
    g = {k: dev(v, td) for k, v in x.items()}
    for r in sorted({0, cp - 1}):
        plan = RankPlan.make(cu, cp, r, tf=(B, N))
        q = partition(g["q"], plan)
        do = partition(g["dout"], plan)
        ks = [partition(g["k"], plan, j) for j in range(cp)]
        vs = [partition(g["v"], plan, j) for j in range(cp)]
        bufs, parts = ring_forward(q, ks, vs, plan, oracle.TF_BLOCK, tf=(B, N), keep_partials=True)
        dq, dk, dv, delta = ring_backward(q, ks, vs, do, bufs, plan, oracle.TF_BLOCK, tf=(B, N))
        torch.cuda.synchronize()
        steps, (o, lse), dq_r, dk_r, dv_r, delta_r = _oracle_rank(x, cu, cp, r, B, N)
        for s in range(cp):
            op, lp = parts[s]
            check_out(op.float().cpu().numpy(), steps[s][0], dtype)
            check_lse(lp.cpu().numpy(), steps[s][1])
        check_out(bufs.out.cpu().numpy(), o, dtype)
        check_lse(bufs.lse.cpu().numpy(), lse)
        tol = 1e-4 if dtype == "f32" else TOL_GRAD_RELRMS
        assert rel_rms(delta.cpu().numpy(), delta_r) <= tol
        assert rel_rms(dq.cpu().numpy(), dq_r) <= tol
        for j in range(cp):
            assert rel_rms(dk[j].cpu().numpy(), dk_r[j]) <= tol, j
            assert rel_rms(dv[j].cpu().numpy(), dv_r[j]) <= tol, j
        # every pair the step computed is the closed count the library reports
        pairs = sum(cpa.cpattn_count_pairs(cu, oracle.TF_BLOCK, cpa.make_step(cp, r, s, B, N)) for s in range(cp))
        assert pairs == sum(tf_split.count_pairs(cu, cp, r, s, B, N) for s in range(cp))


def test_tf_partition_round_trip_bit_exact(cpa):
    B, N, cp, nseq = 40, 6, 3, 2
    x, cu = _inputs(3, nseq, B, N, 3, 3, 64, "bf16")
    g = dev(x["q"], torch.bfloat16)
    back = torch.zeros_like(g)
    for r in range(cp):
        from context_attention_varlen_amd.ring import RankPlan, partition
        plan = RankPlan.make(cu, cp, r, tf=(B, N))
        loc = partition(g, plan)
        _, l2g, _, _ = tf_split.local_rows(cu, cp, r, B, N)
        assert torch.equal(loc.cpu(), g.cpu()[torch.from_numpy(l2g)])
        cpa.cpattn_unpartition_tf(loc, back, plan.cu_global_dev, nseq, cp, r, B, N)
    torch.cuda.synchronize()
    assert torch.equal(back.cpu(), g.cpu())
