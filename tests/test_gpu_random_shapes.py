"""Seeded random shapes through the whole rank step (partition, forward steps
with merges, backward) against the fp64 oracle.

Each case draws a packed batch (1-6 sequences, ragged lengths, some tiny or
empty), a cp size and rank, a GQA head split, head_dim 64 or 128 and a causal
or bidirectional mask, or teacher forcing with a random chunk size and
count, so that tile counts, partial tiles, the two-tiles-per-trip forward
loop and both backward workgroup kinds meet shapes no hand-picked case
names.  The draw is fixed by the seed."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads  # noqa: E402
from tests._gpu import TOL_GRAD_RELRMS, check_lse, check_out, dev, rel_rms  # noqa: E402
from tests.test_gpu_bwd import _check_grad, _inputs, oracle_grads, run_gpu  # noqa: E402


@pytest.fixture(scope="module")
def cpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_varlen_amd as c
    return c


def _draw(seed, long=False):
    """One case.  long: fewer, longer sequences (700-4000 tokens), so that
    items run tens of key tiles and dK/dV workgroups sweep ~100 query tiles,
    element by element against the oracle."""
    rng = np.random.default_rng((60000 if long else 20000) + seed)
    hq, hkv = [(2, 1), (4, 2), (3, 3), (8, 2), (6, 3)][int(rng.integers(0, 5))]
    d = int(rng.choice([64, 128]))
    if rng.random() < 0.2:
        # teacher forcing at cp = 1 (cp > 1 has its own tests): 1-2 sequences
        # of [clean ; noisy] with random chunk size B and count N
        B, N = int(rng.integers(1, 600 if long else 120)), int(rng.integers(1, 6))
        return [2 * B * N] * int(rng.integers(1, 3)), 1, 0, hq, hkv, d, oracle.TF_BLOCK, (B, N)
    cp = int(rng.choice([1, 2, 3, 4]))
    mode = oracle.CAUSAL if rng.random() < 0.7 else oracle.BIDIR
    nseq = int(rng.integers(1, 4 if long else 7))
    quantum = 2 * cp
    lens = []
    for _ in range(nseq):
        kind = rng.random()
        if kind < 0.15:
            n = 0
        elif kind < 0.35:
            n = int(rng.integers(1, 40))
        else:
            n = int(rng.integers(700, 4000)) if long else int(rng.integers(40, 700))
        lens.append(n - n % quantum if cp > 1 else n)
    if sum(lens) == 0:
        lens[0] = 8 * quantum
    rank = int(rng.integers(0, cp))
    return lens, cp, rank, hq, hkv, d, mode, (0, 0)


def _check_case(lens, cp, r, hq, hkv, d, mode, tf, seed):
    print(f"seed {seed}: lens {lens} cp {cp} rank {r} heads {hq}/{hkv} d {d} mode {mode} tf {tf}", flush=True)
    x, cu = _inputs(300 + seed, lens, hq, hkv, d, "bf16")
    dq, dk, dv, delta, bufs = run_gpu(x, cu, cp, r, mode, "bf16", tf)
    _, l2g, qpos, qseq = oracle.local_rows(cu, cp, r)
    T = int(cu[-1])
    seq = np.repeat(np.arange(len(cu) - 1), np.diff(cu))
    pos = np.arange(T) - cu[seq]
    o_ref, l_ref = oracle.attention(x["q"][l2g], x["k"], x["v"], qseq, qpos, seq, pos, mode,
                                    tf_chunk=tf[0], tf_num=tf[1])
    check_out(bufs.out.cpu().numpy(), o_ref, "bf16")
    check_lse(bufs.lse.cpu().numpy(), l_ref)
    dq_r, dk_r, dv_r, delta_r = oracle_grads(x, cu, cp, r, mode, tf)
    _check_grad(dq, dq_r, "dq")
    for j in range(cp):
        _check_grad(dk[j], dk_r[j], f"dk[{j}]")
        _check_grad(dv[j], dv_r[j], f"dv[{j}]")


@pytest.mark.parametrize("seed", range(400))
def test_random_shape(cpa, seed):
    _check_case(*_draw(seed), seed)


@pytest.mark.parametrize("seed", range(24))
def test_random_shape_long(cpa, seed):
    _check_case(*_draw(seed, long=True), 1000 + seed)


@pytest.mark.parametrize("seed", range(16))
def test_random_shape_f32(cpa, seed):
    """The fp32 path on the same kind of draws (fp32 inputs, no bf16
    anywhere), to its tolerance."""
    lens, cp, r, hq, hkv, d, mode, tf = _draw(100 + seed)
    lens = [min(L, 300 - 300 % (2 * cp)) for L in lens]       # the fp32 kernels are slow
    if sum(lens) == 0:
        lens[0] = 8 * cp
    print(f"seed {seed}: lens {lens} cp {cp} rank {r} heads {hq}/{hkv} d {d} mode {mode} tf {tf}", flush=True)
    if tf[0]:
        lens = [2 * tf[0] * tf[1]] * len(lens)
    x, cu = _inputs(500 + seed, lens, hq, hkv, d, "f32")
    dq, dk, dv, delta, bufs = run_gpu(x, cu, cp, r, mode, "f32", tf)
    _, l2g, qpos, qseq = oracle.local_rows(cu, cp, r)
    T = int(cu[-1])
    seq = np.repeat(np.arange(len(cu) - 1), np.diff(cu))
    pos = np.arange(T) - cu[seq]
    o_ref, l_ref = oracle.attention(x["q"][l2g], x["k"], x["v"], qseq, qpos, seq, pos, mode,
                                    tf_chunk=tf[0], tf_num=tf[1])
    check_out(bufs.out.cpu().numpy(), o_ref, "f32")
    check_lse(bufs.lse.cpu().numpy(), l_ref, tol=1e-5)
    dq_r, dk_r, dv_r, _ = oracle_grads(x, cu, cp, r, mode, tf)
    _check_grad(dq, dq_r, "dq", tol=1e-4)
    for j in range(cp):
        _check_grad(dk[j], dk_r[j], f"dk[{j}]", tol=1e-4)
        _check_grad(dv[j], dv_r[j], f"dv[{j}]", tol=1e-4)


@pytest.mark.parametrize("seed", range(16))
def test_random_balanced_tf_split(cpa, seed):
    """Teacher forcing at cp > 1 under the balanced split: random B >= 32,
    N a multiple of cp (a partial last dealing round included), every rank's
    merged result and gradients against the oracle's own split."""
    from context_attention_varlen_amd.ring import RankPlan, partition, ring_backward, ring_forward
    from tests.test_gpu_tf_split import _oracle_rank
    rng = np.random.default_rng(40000 + seed)
    cp = int(rng.integers(2, 5))
    N = cp * int(rng.integers(1, 4))
    B = int(rng.integers(32, 90))
    nseq = int(rng.integers(1, 3))
    hq, hkv = [(2, 1), (4, 2), (3, 3)][int(rng.integers(0, 3))]
    d = int(rng.choice([64, 128]))
    r = int(rng.integers(0, cp))
    print(f"seed {seed}: nseq {nseq} B {B} N {N} cp {cp} rank {r} heads {hq}/{hkv} d {d}", flush=True)
    rs = np.random.default_rng(600 + seed)
    T = nseq * 2 * B * N
    x = {k: workloads.round_bf16(rs.standard_normal((T, h, d), dtype=np.float32))
         for k, h in (("q", hq), ("k", hkv), ("v", hkv), ("dout", hq))}
    cu = np.arange(nseq + 1, dtype=np.int32) * (2 * B * N)
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    plan = RankPlan.make(cu, cp, r, tf=(B, N))
    q = partition(g["q"], plan)
    do = partition(g["dout"], plan)
    ks = [partition(g["k"], plan, j) for j in range(cp)]
    vs = [partition(g["v"], plan, j) for j in range(cp)]
    bufs, _ = ring_forward(q, ks, vs, plan, oracle.TF_BLOCK, tf=(B, N))
    dq, dk, dv, _ = ring_backward(q, ks, vs, do, bufs, plan, oracle.TF_BLOCK, tf=(B, N))
    torch.cuda.synchronize()
    _, (o, lse), dq_r, dk_r, dv_r, _ = _oracle_rank(x, cu, cp, r, B, N)
    check_out(bufs.out.cpu().numpy(), o, "bf16")
    check_lse(bufs.lse.cpu().numpy(), lse)
    assert rel_rms(dq.cpu().numpy(), dq_r) <= TOL_GRAD_RELRMS
    for j in range(cp):
        assert rel_rms(dk[j].cpu().numpy(), dk_r[j]) <= TOL_GRAD_RELRMS, j
        assert rel_rms(dv[j].cpu().numpy(), dv_r[j]) <= TOL_GRAD_RELRMS, j


@pytest.mark.parametrize("seed", range(40))
def test_random_shape_overlapped_step(cpa, seed):
    """ring.rank_step with its second stream on the random draws gives bit
    for bit what the one-stream ring calls give (same kernels, same order
    on every buffer)."""
    from context_attention_varlen_amd.ring import RankPlan, StepBuffers, rank_step
    lens, cp, r, hq, hkv, d, mode, tf = _draw(seed)
    print(f"seed {seed}: lens {lens} cp {cp} rank {r} heads {hq}/{hkv} d {d} mode {mode} tf {tf}", flush=True)
    x, cu = _inputs(300 + seed, lens, hq, hkv, d, "bf16")
    dq, dk, dv, delta, bufs = run_gpu(x, cu, cp, r, mode, "bf16", tf)
    g = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    plan = RankPlan.make(cu, cp, r, tf=tf if tf[0] else None)
    b = StepBuffers.make(plan, hq, hkv, d, torch.bfloat16, backward=True)
    rank_step(g["q"], g["k"], g["v"], g["dout"], plan, mode, b, side=torch.cuda.Stream(), tf=tf)
    torch.cuda.synchronize()
    assert torch.equal(b.fwd.out, bufs.out) and torch.equal(b.fwd.lse, bufs.lse)
    assert np.array_equal(b.dq.cpu().numpy(), dq) and np.array_equal(b.delta.cpu().numpy(), delta)
    for j in range(cp):
        assert np.array_equal(b.dk[j].cpu().numpy(), dk[j]) and np.array_equal(b.dv[j].cpu().numpy(), dv[j])
