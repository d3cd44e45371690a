"""GPU parity of the backward ring steps (dQ, and dK/dV per source rank)
against the fp64 oracle, through the C ABI.  The GPU backward runs from the
GPU forward's merged (out, lse); the oracle uses its own exact ones."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads  # noqa: E402
from tests._gpu import TOL_GRAD_RELRMS, check_lse, check_out, dev, rel_rms, tdtype  # noqa: E402


@pytest.fixture(scope="module")
def cpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_varlen_amd as c
    return c


def _inputs(seed, lens, hq, hkv, d, dtype):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    x = {"q": rng.standard_normal((T, hq, d), dtype=np.float32),
         "k": rng.standard_normal((T, hkv, d), dtype=np.float32),
         "v": rng.standard_normal((T, hkv, d), dtype=np.float32),
         "dout": rng.standard_normal((T, hq, d), dtype=np.float32)}
    if dtype == "bf16":
        x = {k: workloads.round_bf16(v) for k, v in x.items()}
    return x, np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def run_gpu(x, cu, cp, r, mode, dtype, tf=(0, 0)):
    from context_attention_varlen_amd.ring import RankPlan, partition, ring_backward, ring_forward
    plan = RankPlan.make(cu, cp, r)
    td = tdtype(dtype)
    g = {k: dev(v, td) for k, v in x.items()}
    q = partition(g["q"], plan)
    do = partition(g["dout"], plan)
    ks = [partition(g["k"], plan, j) for j in range(cp)]
    vs = [partition(g["v"], plan, j) for j in range(cp)]
    bufs, _ = ring_forward(q, ks, vs, plan, mode, tf=tf)
    dq, dk, dv, delta = ring_backward(q, ks, vs, do, bufs, plan, mode, tf=tf)
    torch.cuda.synchronize()
    return (dq.cpu().numpy(), [t.cpu().numpy() for t in dk], [t.cpu().numpy() for t in dv],
            delta.cpu().numpy(), bufs)


def oracle_grads(x, cu, cp, r, mode, tf=(0, 0)):
    """Per-source dK/dV and summed dQ of rank r, from the exact final LSE/O."""
    _, l2g, qpos, qseq = oracle.local_rows(cu, cp, r)
    T = int(cu[-1])
    seq = np.repeat(np.arange(len(cu) - 1), np.diff(cu))
    pos = np.arange(T) - cu[seq]
    o, lse = oracle.attention(x["q"][l2g], x["k"], x["v"], qseq, qpos, seq, pos, mode,
                              tf_chunk=tf[0], tf_num=tf[1])
    delta = oracle.bwd_delta(o, x["dout"][l2g])
    dq = np.zeros((len(l2g),) + x["q"].shape[1:])
    dks, dvs = [], []
    for s in range(cp):
        j = oracle.step_source(cp, r, s)
        _, k2g, kpos, kseq = oracle.local_rows(cu, cp, j)
        a, b, c = oracle.attention_backward(x["q"][l2g], x["k"][k2g], x["v"][k2g], x["dout"][l2g], lse, delta,
                                            qseq, qpos, kseq, kpos, mode, tf_chunk=tf[0], tf_num=tf[1])
        dq += a
        dks.append((j, b))
        dvs.append((j, c))
    return dq, dict(dks), dict(dvs), delta


def _check_grad(x, ref, name, tol=TOL_GRAD_RELRMS):
    assert np.all(np.isfinite(x)), f"{name}: non-finite"
    rr = rel_rms(x, ref)
    assert rr <= tol, f"{name}: rel-RMS {rr}"


CASES = [
    ([256], 4, 2, 2, 64, "f32", oracle.CAUSAL, (0, 0)),
    ([512], 2, 4, 2, 128, "bf16", oracle.CAUSAL, (0, 0)),
    ([384, 128, 64], 4, 4, 1, 128, "bf16", oracle.CAUSAL, (0, 0)),
    ([200, 56, 336], 4, 8, 2, 128, "bf16", oracle.CAUSAL, (0, 0)),
    ([333, 1, 70], 1, 3, 3, 128, "bf16", oracle.CAUSAL, (0, 0)),
    ([300, 77], 1, 4, 2, 128, "bf16", oracle.BIDIR, (0, 0)),
    ([96, 160], 2, 2, 2, 128, "bf16", oracle.BIDIR, (0, 0)),
    ([2 * 3 * 37], 1, 2, 2, 128, "bf16", oracle.TF_BLOCK, (37, 3)),
    ([2 * 4 * 100, 2 * 4 * 100], 1, 4, 2, 128, "bf16", oracle.TF_BLOCK, (100, 4)),
    ([256, 128], 2, 4, 4, 64, "bf16", oracle.CAUSAL, (0, 0)),
    ([200], 1, 2, 1, 64, "bf16", oracle.TF_BLOCK, (25, 4)),
    ([96, 32], 2, 2, 1, 128, "f32", oracle.CAUSAL, (0, 0)),
]


@pytest.mark.parametrize("lens,cp,hq,hkv,d,dtype,mode,tf", CASES)
def test_backward_against_oracle(cpa, lens, cp, hq, hkv, d, dtype, mode, tf):
    x, cu = _inputs(11, lens, hq, hkv, d, dtype)
    tol = 1e-4 if dtype == "f32" else TOL_GRAD_RELRMS
    for r in sorted({0, cp - 1}):
        dq, dk, dv, delta, _ = run_gpu(x, cu, cp, r, mode, dtype, tf)
        dq_r, dk_r, dv_r, delta_r = oracle_grads(x, cu, cp, r, mode, tf)
        _check_grad(delta, delta_r, "delta", tol)
        _check_grad(dq, dq_r, "dq", tol)
        for j in range(cp):
            _check_grad(dk[j], dk_r[j], f"dk[{j}]", tol)
            _check_grad(dv[j], dv_r[j], f"dv[{j}]", tol)


def test_backward_invariants_long_tail_scaled(cpa):
    """Long-tail structure scaled down 8x: sum over every source's key rows of
    dV equals sum of the rank's dO per (sequence, kv-group), and dK sums to
    zero (sum_j P_ij = 1, sum_j dS_ij = 0)."""
    w = workloads.WORKLOADS["long_tail"]
    lens = [l // 8 - (l // 8) % 8 for l in w.seqlens]
    x, cu = _inputs(12, lens, 8, 2, 128, "bf16")
    dq, dk, dv, _, _ = run_gpu(x, cu, 4, 0, oracle.CAUSAL, "bf16")
    cu_l, l2g, _, qseq = oracle.local_rows(cu, 4, 0)
    grp = 4
    for b in range(len(lens)):
        rows = slice(cu_l[b], cu_l[b + 1])
        dv_sum = sum(dv[j][rows].sum(0) for j in range(4))   # [Hkv, d]
        dk_sum = sum(dk[j][rows].sum(0) for j in range(4))
        do_loc = x["dout"][l2g][rows]
        for g in range(2):
            want = do_loc[:, g * grp:(g + 1) * grp].sum((0, 1))
            scale = np.abs(do_loc).sum() / max(1, do_loc.size) * np.sqrt(do_loc.shape[0] * grp)
            assert np.max(np.abs(dv_sum[g] - want)) <= 2e-2 * max(1.0, scale)
            assert np.max(np.abs(dk_sum[g])) <= 2e-2 * max(1.0, scale)


@pytest.mark.parametrize("bad", ["q", "k"])
def test_bad_device_cu_seqlens_backward(cpa, bad):
    """A non-monotone device cu_seqlens array (query or key side) schedules no
    work in either list of the backward: the gradients are left as they were
    and the workspace status reports INVALID_ARG; a valid call clears it."""
    q = torch.randn(64, 4, 128, device="cuda").bfloat16()
    kv = torch.randn(64, 2, 128, device="cuda").bfloat16()
    do = torch.randn(64, 4, 128, device="cuda").bfloat16()
    lse = torch.zeros(4, 64, device="cuda")
    delta = torch.zeros(4, 64, device="cuda")
    dq = torch.full((64, 4, 128), 7.0, device="cuda")
    dk = torch.full((64, 2, 128), 7.0, device="cuda")
    dv = torch.full((64, 2, 128), 7.0, device="cuda")
    ws = torch.empty(cpa.cpattn_workspace_size(64, 64, 3), dtype=torch.uint8, device="cuda")
    cu_ok = torch.tensor([0, 20, 40, 64], dtype=torch.int32, device="cuda")
    cu_bad = torch.tensor([0, 40, 20, 64], dtype=torch.int32, device="cuda")
    cu_q, cu_k = (cu_bad, cu_ok) if bad == "q" else (cu_ok, cu_bad)
    st = cpa.make_step(1, 0, 0)
    cpa.cpattn_bwd_step(q, kv, kv, do, lse, delta, cu_q, cu_k, 3, cpa.CAUSAL, st, 0.0, dq, dk, dv, ws)
    assert cpa.cpattn_workspace_status(ws) == cpa.ERR_INVALID_ARG
    assert torch.all(dq == 7.0) and torch.all(dk == 7.0) and torch.all(dv == 7.0)
    cpa.cpattn_bwd_step(q, kv, kv, do, lse, delta, cu_ok, cu_ok, 3, cpa.CAUSAL, st, 0.0, dq, dk, dv, ws)
    assert cpa.cpattn_workspace_status(ws) == cpa.OK


def test_many_sequences_global_schedule_path(cpa):
    """Over 2048 sequences and over 8192 work items per tile list: the
    scheduler keeps per-sequence offsets, cu_seqlens and item cost bins in
    workspace memory instead of LDS.  5000 short sequences (some empty) at
    cp = 2, forward and backward of rank 1 against the oracle."""
    rng = np.random.default_rng(77)
    lens = [int(4 * rng.integers(1, 11)) for _ in range(5000)]
    for i in rng.choice(5000, size=40, replace=False):
        lens[int(i)] = 0
    assert len(lens) > 2048 and 2 * sum(1 for L in lens if L) > 8192
    x, cu = _inputs(78, lens, 2, 1, 64, "bf16")
    mode = oracle.CAUSAL
    dq, dk, dv, delta, bufs = run_gpu(x, cu, 2, 1, mode, "bf16")
    _, l2g, qpos, qseq = oracle.local_rows(cu, 2, 1)
    seq = np.repeat(np.arange(len(cu) - 1), np.diff(cu))
    pos = np.arange(int(cu[-1])) - cu[seq]
    o_ref, l_ref = oracle.attention(x["q"][l2g], x["k"], x["v"], qseq, qpos, seq, pos, mode)
    check_out(bufs.out.cpu().numpy(), o_ref, "bf16")
    check_lse(bufs.lse.cpu().numpy(), l_ref)
    dq_r, dk_r, dv_r, _ = oracle_grads(x, cu, 2, 1, mode)
    _check_grad(dq, dq_r, "dq")
    for j in range(2):
        _check_grad(dk[j], dk_r[j], f"dk[{j}]")
        _check_grad(dv[j], dv_r[j], f"dv[{j}]")
