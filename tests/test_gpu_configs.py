"""Full-size workloads through the C ABI, in the launch configuration bench.py
times, checked against the fp64 oracle on seeded samples of rows (the oracle
computes each sampled row against every key it may attend) and, for the
backward, with invariants that hold at any size."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads  # noqa: E402
from tests._gpu import (TOL_GRAD_RELRMS, check_lse, check_out, oracle_by_head, rel_rms,  # noqa: E402
                        stratified_offsets, tdtype)


@pytest.fixture(scope="module")
def cpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_varlen_amd as c
    return c


def _seq_pos(cu):
    T = int(cu[-1])
    seq = np.repeat(np.arange(len(cu) - 1), np.diff(cu))
    return seq, np.arange(T) - np.asarray(cu)[seq]


def _sample_local_rows(w, r, count, seed):
    """Stratified seeded sample of a rank's local rows: first/last row of every
    local chunk, rows next to 64/128/256 tile edges, plus uniform rows."""
    cu_l, l2g, _, _ = oracle.local_rows(w.cu_seqlens, w.cp, r)
    edges = []
    for b in range(len(cu_l) - 1):
        n = cu_l[b + 1] - cu_l[b]
        halves = [(cu_l[b], n)] if w.cp == 1 else [(cu_l[b], n // 2), (cu_l[b] + n // 2, n // 2)]
        for s0, m in halves:
            if m == 0:
                continue
            edges += [s0, s0 + m - 1]
            for t in (64, 128, 256):
                if m > t:
                    edges += [s0 + t - 1, s0 + t]
    rng = np.random.default_rng(1000 + r)
    base = workloads.sample_rows(rng, len(l2g), count)
    edges = np.unique(np.asarray(edges))
    extra = rng.choice(edges, size=min(len(edges), count), replace=False) if len(edges) else []
    return np.unique(np.concatenate([base, np.asarray(extra, dtype=np.int64)]))


def _stratified_local_rows(w, r, per_chunk, seed):
    """At least `per_chunk` rows of every local chunk of rank r (each zigzag
    half of each sequence): its first two and last two rows, rows next to
    64- and 128-row tile edges (+-1), and uniform rows, seeded."""
    cu_l, _, _, _ = oracle.local_rows(w.cu_seqlens, w.cp, r)
    rng = np.random.default_rng(2000 + 10 * r + seed)
    out = []
    for b in range(len(cu_l) - 1):
        n = int(cu_l[b + 1] - cu_l[b])
        halves = [(int(cu_l[b]), n)] if w.cp == 1 else [(int(cu_l[b]), n // 2), (int(cu_l[b]) + n // 2, n // 2)]
        for s0, m in halves:
            if m:
                out.append(s0 + stratified_offsets(m, per_chunk, rng))
    return np.unique(np.concatenate(out))


def _oracle_rows(w, x, r, rows, step=None):
    """Oracle output/LSE of a rank's sampled local rows: against every key of
    their sequence (merged result) or only the keys of one ring step.  Under
    the causal mask only keys up to the last sampled position can be allowed,
    so the others are left out of the call (the result is the same).  Heads
    run in parallel threads."""
    _, l2g, qpos, qseq = oracle.local_rows(w.cu_seqlens, w.cp, r)
    if step is None:
        seq, pos = _seq_pos(w.cu_seqlens)
        kidx = np.nonzero(np.isin(seq, np.unique(qseq[rows])))[0]
        kseq, kpos = seq[kidx], pos[kidx]
    else:
        _, kidx, kpos, kseq = oracle.local_rows(w.cu_seqlens, w.cp, oracle.step_source(w.cp, r, step))
    if w.mask == oracle.CAUSAL:
        keep = kpos <= qpos[rows].max()
        kidx, kpos, kseq = kidx[keep], kpos[keep], kseq[keep]
    return oracle_by_head(oracle.attention, x["q"][l2g[rows]], x["k"][kidx], x["v"][kidx], qseq[rows], qpos[rows],
                          kseq, kpos, w.mask, tf_chunk=w.tf_chunk, tf_num=w.tf_num)


def _gpu_ring(w, x, r, keep=False, backward=False):
    from context_attention_varlen_amd.ring import RankPlan, partition, ring_backward, ring_forward
    td = tdtype(w.dtype)
    plan = RankPlan.make(w.cu_seqlens, w.cp, r, tf=(w.tf_chunk, w.tf_num) if w.tf_chunk else None)
    q = partition(torch.from_numpy(x["q"]).to(td).cuda(), plan)
    kg = torch.from_numpy(x["k"]).to(td).cuda()
    vg = torch.from_numpy(x["v"]).to(td).cuda()
    ks = [partition(kg, plan, j) for j in range(w.cp)]
    vs = [partition(vg, plan, j) for j in range(w.cp)]
    del kg, vg
    torch.cuda.empty_cache()
    tf = (w.tf_chunk, w.tf_num)
    bufs, parts = ring_forward(q, ks, vs, plan, w.mask, tf=tf, keep_partials=keep)
    grads = None
    if backward:
        do = partition(torch.from_numpy(x["dout"]).to(td).cuda(), plan)
        grads = ring_backward(q, ks, vs, do, bufs, plan, w.mask, tf=tf)
    torch.cuda.synchronize()
    return plan, bufs, parts, grads


@pytest.fixture(scope="module")
def long_video_inputs():
    return workloads.draw(workloads.WORKLOADS["long_video"])


@pytest.mark.parametrize("rank", [0, 7])
def test_long_video_rank(cpa, long_video_inputs, rank):
    """262144 tokens, cp=8 zigzag, 28/4 heads: all 8 forward steps and merges
    of one rank; at least 256 stratified rows of each of its two local chunks
    (chunk edges, tile edges +-1, uniform) of the merged result and of three
    step partials."""
    w = workloads.WORKLOADS["long_video"]
    x = long_video_inputs
    plan, bufs, parts, _ = _gpu_ring(w, x, rank, keep=True)
    rows = _stratified_local_rows(w, rank, 256, 0)
    assert len(rows) >= 512
    o_ref, l_ref = _oracle_rows(w, x, rank, rows)
    t = torch.from_numpy(rows).cuda()
    check_out(bufs.out[t].cpu().numpy(), o_ref, "bf16")
    check_lse(bufs.lse[:, t].cpu().numpy(), l_ref)
    for s in (0, 1, 7):
        o_ref, l_ref = _oracle_rows(w, x, rank, rows, step=s)
        op, lp = parts[s]
        check_out(op[t].float().cpu().numpy(), o_ref, "bf16")
        check_lse(lp[:, t].cpu().numpy(), l_ref)
    # balance of the zigzag split: the exact pair count is rank-independent
    assert sum(cpa.cpattn_count_pairs(w.cu_seqlens, w.mask, cpa.make_step(8, rank, s)) for s in range(8)) \
        == 4_294_983_680


@pytest.fixture(scope="module")
def two_million():
    """One 2,097,152-token sequence (the >2M-token contexts of the long-video
    pages), zigzag cp = 8, GQA 2/1, d = 128, bf16 0.5 N(0,1)."""
    w = workloads.Workload("two_million_tokens", (1 << 21,), heads_q=2, heads_kv=1, head_dim=128, dtype="bf16",
                           mask=oracle.CAUSAL, cp=8, rank=0, value_scale=0.5, seed=7)
    return w, workloads.draw(w)


@pytest.mark.parametrize("rank", [0, 7])
def test_two_million_token_sequence(cpa, two_million, rank):
    """The largest shape in the suite: positions up to 2^21 and 262144 local
    rows per rank; all 8 forward steps and merges, sampled merged rows and
    step partials against the oracle, and the exact per-rank pair count."""
    w, x = two_million
    plan, bufs, parts, _ = _gpu_ring(w, x, rank, keep=True)
    rows = _sample_local_rows(w, rank, 12, 0)
    o_ref, l_ref = _oracle_rows(w, x, rank, rows)
    t = torch.from_numpy(rows).cuda()
    check_out(bufs.out[t].cpu().numpy(), o_ref, "bf16")
    check_lse(bufs.lse[:, t].cpu().numpy(), l_ref)
    for s in (0, 5):
        o_ref, l_ref = _oracle_rows(w, x, rank, rows, step=s)
        op, lp = parts[s]
        check_out(op[t].float().cpu().numpy(), o_ref, "bf16")
        check_lse(lp[:, t].cpu().numpy(), l_ref)
    L = 1 << 21
    assert sum(cpa.cpattn_count_pairs(w.cu_seqlens, w.mask, cpa.make_step(8, rank, s)) for s in range(8)) \
        == L * L // 16 + L // 16


def test_tf_dit_sampled(cpa):
    """Teacher-forced DiT, 74880 tokens, block mask: sampled rows stratified
    over both streams and the chunk edges (B = 3120 is not a tile multiple)."""
    w = workloads.WORKLOADS["tf_dit"]
    x = workloads.draw(w)
    plan, bufs, _, _ = _gpu_ring(w, x, 0)
    B, N = w.tf_chunk, w.tf_num
    edges = []
    for c in range(2 * N):
        edges += [c * B, c * B + 1, c * B + B - 1]
    rng = np.random.default_rng(1003)
    rows = workloads.sample_rows(rng, w.tokens, 40, edges)
    o_ref, l_ref = _oracle_rows(w, x, 0, rows)
    t = torch.from_numpy(rows).cuda()
    check_out(bufs.out[t].cpu().numpy(), o_ref, "bf16")
    check_lse(bufs.lse[:, t].cpu().numpy(), l_ref)


def _oracle_rank_forward(w, x, r):
    """fp64 O and LSE of every local row of rank r against every key of its
    sequence, one local chunk at a time (under the causal mask a chunk's rows
    can only see keys up to its last position, so later keys are left out of
    the call); heads in parallel threads."""
    cu = w.cu_seqlens
    cu_l, l2g, qpos, qseq = oracle.local_rows(cu, w.cp, r)
    seq, pos = _seq_pos(cu)
    n = len(l2g)
    o = np.zeros((n, w.heads_q, w.head_dim))
    lse = np.full((w.heads_q, n), -np.inf)
    for b in range(len(cu_l) - 1):
        L = int(cu_l[b + 1] - cu_l[b])
        for c0, m in ((int(cu_l[b]), L // 2), (int(cu_l[b]) + L // 2, L // 2)):
            if m == 0:
                continue
            rows = np.arange(c0, c0 + m)
            keys = np.nonzero((seq == b) & (pos <= qpos[rows].max()))[0]
            o[rows], lse[:, rows] = oracle_by_head(oracle.attention, x["q"][l2g[rows]], x["k"][keys], x["v"][keys],
                                                   qseq[rows], qpos[rows], seq[keys], pos[keys], w.mask)
    return o, lse


def test_long_tail_forward_backward(cpa):
    """65536 tokens (49152 + 15 short), cp=4 zigzag, 32/8 heads, rank 0, in
    the launch configuration bench.py times.  The oracle computes the merged
    forward of all 16384 local rows (so every row's output and LSE is
    compared, and the exact LSE and delta feed the gradient checks); dQ on
    512 stratified rows against every key; dK/dV of every source rank on at
    least 256 stratified key rows of the 49152-token sequence (both chunk
    halves, chunk and tile edges +-1, keys near the causal diagonal) and on
    stratified keys of every short sequence, each summed over all of rank
    0's queries; the gradient sums over all keys as an extra check."""
    w = workloads.WORKLOADS["long_tail"]
    x = workloads.draw(w)
    r = 0
    plan, bufs, _, grads = _gpu_ring(w, x, r, backward=True)
    dq, dk, dv, _ = grads
    cu = w.cu_seqlens
    cu_l, l2g, qpos, qseq = oracle.local_rows(cu, w.cp, r)
    seq, pos = _seq_pos(cu)

    # merged forward, every local row
    o_ref, l_ref = _oracle_rank_forward(w, x, r)
    check_out(bufs.out.cpu().numpy(), o_ref, "bf16")
    check_lse(bufs.lse.cpu().numpy(), l_ref)
    dout_l = x["dout"][l2g]
    delta_ref = oracle.bwd_delta(o_ref, dout_l)

    # dQ (summed over the 4 ring steps = every key) on stratified rows
    rng = np.random.default_rng(3005)
    rows = np.unique(np.concatenate([stratified_offsets(len(l2g), 384, rng),
                                     _stratified_local_rows(w, r, 4, 1)]))
    kidx = np.nonzero(np.isin(seq, np.unique(qseq[rows])))[0]
    dq_ref, _, _ = oracle_by_head(oracle.attention_backward, x["q"][l2g[rows]], x["k"][kidx], x["v"][kidx],
                                  dout_l[rows], l_ref[:, rows], delta_ref[:, rows], qseq[rows], qpos[rows],
                                  seq[kidx], pos[kidx], w.mask)
    t = torch.from_numpy(rows).cuda()
    assert rel_rms(dq[t].cpu().numpy(), dq_ref) <= TOL_GRAD_RELRMS

    # dK/dV per source rank, each sampled key summed over all rank-0 queries
    # of its sequence
    long_len = int(w.seqlens[0])
    C = long_len // (2 * w.cp)
    for j in range(w.cp):
        _, k2g, kpos, kseq = oracle.local_rows(cu, w.cp, j)
        krng = np.random.default_rng(4000 + j)
        for b in range(len(w.seqlens)):
            kb = np.nonzero(kseq == b)[0]
            if b == 0:
                half = len(kb) // 2
                # both chunk halves: chunk / tile edges +-1 and uniform keys,
                # plus keys next to rank 0's query-chunk boundaries (the
                # causal diagonal of its chunks 0 and 2cp-1)
                sel = [kb[:half][stratified_offsets(half, 160, krng)],
                       kb[half:][stratified_offsets(half, 160, krng)]]
                diag = np.nonzero(np.isin(kpos[kb], [C - 2, C - 1, C, (2 * w.cp - 1) * C - 1,
                                                     (2 * w.cp - 1) * C, (2 * w.cp - 1) * C + 1,
                                                     long_len - 2, long_len - 1]))[0]
                ksel = np.unique(np.concatenate(sel + [kb[diag]]))
                assert len(ksel) >= 256
            else:
                ksel = kb[stratified_offsets(len(kb), 24, krng)]
            qrows = np.nonzero(qseq == b)[0]
            _, dk_ref, dv_ref = oracle_by_head(
                oracle.attention_backward, x["q"][l2g[qrows]], x["k"][k2g[ksel]], x["v"][k2g[ksel]], dout_l[qrows],
                l_ref[:, qrows], delta_ref[:, qrows], qseq[qrows], qpos[qrows], kseq[ksel], kpos[ksel], w.mask)
            kt = torch.from_numpy(ksel).cuda()
            assert rel_rms(dk[j][kt].cpu().numpy(), dk_ref) <= TOL_GRAD_RELRMS, ("dk", b, j)
            assert rel_rms(dv[j][kt].cpu().numpy(), dv_ref) <= TOL_GRAD_RELRMS, ("dv", b, j)

    # extra: sum_j dV_j = sum_i dO_i and sum_j dK_j = 0 over every key
    do_loc = torch.from_numpy(dout_l).cuda()
    grp = w.heads_q // w.heads_kv
    for b in range(len(w.seqlens)):
        rs = slice(int(cu_l[b]), int(cu_l[b + 1]))
        dv_sum = sum(dv[j][rs].double().sum(0) for j in range(w.cp))
        dk_sum = sum(dk[j][rs].double().sum(0) for j in range(w.cp))
        want = do_loc[rs].double().sum(0).view(w.heads_kv, grp, w.head_dim).sum(1)
        scale = float(do_loc[rs].double().norm()) / np.sqrt(w.head_dim * w.heads_kv)
        assert float((dv_sum - want).abs().max()) <= 1e-2 * max(1.0, scale), b
        assert float(dk_sum.abs().max()) <= 1e-2 * max(1.0, scale), b


def test_tf_dit_split_sampled(cpa):
    """Teacher-forced DiT under the balanced split, cp = 3, rank 0 (time
    chunks 0, 5, 6, 11; 24960 local rows): merged forward and dQ on rows
    stratified over both streams and every chunk edge; the gradient sums
    over every key row (sum_j dV_j = sum_i dO_i, sum_j dK_j = 0 per head)."""
    from oracle import tf_split
    w = workloads.WORKLOADS["tf_dit_split"]
    x = workloads.draw(w)
    r = 0
    plan, bufs, _, grads = _gpu_ring(w, x, r, backward=True)
    dq, dk, dv, _ = grads
    B, N, cu = w.tf_chunk, w.tf_num, w.cu_seqlens
    _, l2g, qpos, qseq = tf_split.local_rows(cu, w.cp, r, B, N)
    m = N // w.cp
    edges = []
    for blk in range(2 * m):
        edges += [blk * B, blk * B + 1, blk * B + B - 1]
    rng = np.random.default_rng(1005)
    rows = workloads.sample_rows(rng, len(l2g), 32, edges)
    seq, pos = _seq_pos(cu)
    o_ref, l_ref = oracle.attention(x["q"][l2g[rows]], x["k"], x["v"], qseq[rows], qpos[rows], seq, pos,
                                    oracle.TF_BLOCK, tf_chunk=B, tf_num=N)
    t = torch.from_numpy(rows).cuda()
    check_out(bufs.out[t].cpu().numpy(), o_ref, "bf16")
    check_lse(bufs.lse[:, t].cpu().numpy(), l_ref)
    delta = oracle.bwd_delta(o_ref, x["dout"][l2g[rows]])
    dq_ref, _, _ = oracle.attention_backward(x["q"][l2g[rows]], x["k"], x["v"], x["dout"][l2g[rows]], l_ref, delta,
                                             qseq[rows], qpos[rows], seq, pos, oracle.TF_BLOCK, tf_chunk=B, tf_num=N)
    assert rel_rms(dq[t].cpu().numpy(), dq_ref) <= TOL_GRAD_RELRMS
    do_loc = torch.from_numpy(x["dout"][l2g]).cuda().double()
    dv_sum = sum(dv[j].double().sum(0) for j in range(w.cp))
    dk_sum = sum(dk[j].double().sum(0) for j in range(w.cp))
    want = do_loc.sum(0)
    scale = float(do_loc.norm()) / np.sqrt(w.head_dim * w.heads_kv)
    assert float((dv_sum - want).abs().max()) <= 1e-2 * max(1.0, scale)
    assert float(dk_sum.abs().max()) <= 1e-2 * max(1.0, scale)
