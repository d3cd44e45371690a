"""The varlen tile scheduler's work lists, read back from the workspace after
cpattn_fwd_step and cpattn_bwd_step and checked by brute force over the mask.

The scheduler is what makes the attention kernels skip fully masked tiles
and the element mask inside fully allowed ranges, so the forward/backward
parity tests alone would not notice a list that visits masked tiles twice or
skips nothing.  What is checked, for every list (forward query tiles; the
backward's query tiles and key tiles):
  * the items' primary rows partition the local rows (the forward's list
    also covers rows past the last sequence, with no segments);
  * every item stays inside one sequence and one zigzag chunk, and its
    positions and its segments' positions are those of the oracle's index
    plan (consecutive rows, consecutive positions);
  * segments of one item are disjoint and cover every secondary row that
    has an allowed pair with the item, so every allowed (query, key) pair
    is visited exactly once;
  * the allowed pairs inside the emitted segments add up to the closed-form
    count cpattn_count_pairs gives (and the oracle's brute-force count);
  * no 64-row block of an emitted segment is fully masked for the item
    (tiles with no allowed pair are skipped), and the [full_lo, full_hi)
    range of a segment is allowed for every row of the item (the element
    mask may be skipped there);
  * an item's cost is the number of 64-row secondary tiles it visits times
    the GQA group size (key-tile list), and the order array is a
    permutation sorting the costs longest first.
Pair counts follow "Speeding up Variable-Length Training with Dynamic
Context Parallelism and NVIDIA Megatron Core", section A2 (work counted from
real sequence lengths); the skipped work is the O(S^2) masked half that the
same page's data-scheduling model is about.

The workspace layout read here is the library's: two regions (query tiles,
then key tiles), each a 256-byte header (status, item count), 64-byte items
(seq, row0, nrows, pos0, cost, nseg, then two segments of row, pos, n,
full_lo, full_hi), the sorted order and per-sequence bases, with
(tokens + 15) / 16 + 2 * num_seqs + 1 item slots per region, every part
aligned to 256 bytes."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from oracle import tf_split  # noqa: E402

KBINS = 2048
SEC_TILE = 64


@pytest.fixture(scope="module")
def cpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_varlen_amd as c
    return c


def _align(x, a=256):
    return (x + a - 1) // a * a


def _region(base, tokens, nseq):
    cap = (tokens + 15) // 16 + 2 * nseq + 1
    items = base + 256
    order = _align(items + cap * 64)
    seq_base = _align(order + cap * 4)
    return {"hdr": base, "items": items, "order": order, "end": _align(seq_base + (nseq + 1) * 4)}


def _read_list(ws_bytes, region):
    w = ws_bytes.view(np.int32)
    status, n = int(w[region["hdr"] // 4]), int(w[region["hdr"] // 4 + 1])
    items = w[region["items"] // 4: region["items"] // 4 + 16 * n].reshape(n, 16)
    order = w[region["order"] // 4: region["order"] // 4 + n]
    return status, items.copy(), order.copy()


def _plan(cu, cp, r, mode, tf):
    """(cu_local, positions) of rank r's local rows, from the oracle's index
    code.  Under BIDIR at cp > 1 positions do not matter and the scheduler
    numbers each local sequence's rows from 0, which is what is compared."""
    if mode == oracle.TF_BLOCK and cp > 1:
        cu_l, _, pos, _ = tf_split.local_rows(cu, cp, r, tf[0], tf[1])
    else:
        cu_l, _, pos, seq = oracle.local_rows(cu, cp, r)
        if mode == oracle.BIDIR and cp > 1:
            pos = np.arange(len(pos)) - np.asarray(cu_l)[seq]
    return np.asarray(cu_l, np.int64), np.asarray(pos, np.int64)


def check_list(status, items, order, prim_is_q, cu_p, pos_p, cu_s, pos_s, T_p, tail, mode, tf, cost_mult,
               want_pairs, seg_pos_consecutive=True):
    """seg_pos_consecutive: False under the balanced teacher-forcing split,
    where a segment spans several local chunk blocks whose positions jump
    (the kernels run those segments unmasked, so only rows matter)."""
    assert status == 0, f"scheduler status {status}"
    nseq = len(cu_p) - 1
    covered = np.zeros(T_p, np.int64)
    total = 0

    def pred(pp, ps):       # allowed matrix [primary rows, secondary rows]
        if prim_is_q:
            return oracle.allowed(mode, pp[:, None], ps[None, :], tf[0], tf[1])
        return oracle.allowed(mode, ps[None, :], pp[:, None], tf[0], tf[1])

    for it in items:
        seq, row0, nrows, pos0, cost, nseg = (int(v) for v in it[:6])
        assert nrows > 0 and 0 <= row0 and row0 + nrows <= T_p, it
        covered[row0:row0 + nrows] += 1
        if seq == nseq:                     # rows past the last sequence
            assert tail and nseg == 0 and cost == 0 and row0 >= cu_p[nseq], it
            continue
        assert 0 <= seq < nseq and cu_p[seq] <= row0 and row0 + nrows <= cu_p[seq + 1], it
        pp = pos_p[row0:row0 + nrows]
        assert np.array_equal(pp, pos0 + np.arange(nrows)), ("primary positions", it)
        s0, s1 = int(cu_s[seq]), int(cu_s[seq + 1])
        want_rows = pred(pp, pos_s[s0:s1]).any(axis=0)      # secondary rows with an allowed pair
        cover = np.zeros(s1 - s0, np.int64)
        tiles = 0
        assert 0 <= nseg <= 2, it
        for g in range(nseg):
            row, pos, n, flo, fhi = (int(v) for v in it[6 + 5 * g: 11 + 5 * g])
            assert n > 0 and s0 <= row and row + n <= s1, ("segment rows", it)
            ps = pos_s[row:row + n]
            if seg_pos_consecutive:
                assert np.array_equal(ps, pos + np.arange(n)), ("segment positions", it)
            else:
                assert ps[0] == pos, ("segment start position", it)
            cover[row - s0: row - s0 + n] += 1
            M = pred(pp, ps)
            total += int(M.sum())
            if fhi > flo:
                assert 0 <= flo and fhi <= n and M[:, flo:fhi].all(), ("full range holds a masked pair", it)
            for b0 in range(0, n, SEC_TILE):
                assert M[:, b0:b0 + SEC_TILE].any(), ("fully masked tile emitted", it, b0)
            tiles += -(-n // SEC_TILE)
        assert cost == tiles * cost_mult, ("cost", it)
        assert cover.max(initial=0) <= 1, ("overlapping segments", it)
        assert not np.any(want_rows & (cover == 0)), ("allowed rows outside the segments", it)
    inside = np.zeros(T_p, bool)
    inside[:int(cu_p[nseq])] = True
    if tail:
        inside[:] = True
    assert np.all(covered[inside] == 1) and np.all(covered[~inside] == 0), "primary rows not partitioned"
    assert total == want_pairs, (total, want_pairs)
    n = len(items)
    assert np.array_equal(np.sort(order), np.arange(n)), "order is not a permutation"
    costs = np.minimum(items[order, 4], KBINS - 1)
    assert np.all(np.diff(costs) <= 0), "order is not longest first"


def _run_case(c, lens, cp, r, s, mode, tf, hq, hkv, pad=0):
    from context_attention_varlen_amd.ring import RankPlan
    d = 128
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    split = tf if (mode == oracle.TF_BLOCK and cp > 1) else None
    plan = RankPlan.make(cu, cp, r, tf=split)
    j = c.cpattn_step_source(c.make_step(cp, r, s))
    plan_k = RankPlan.make(cu, cp, j, tf=split)
    Tq = plan.tokens_local + pad
    Tk = plan_k.tokens_local
    gen = torch.Generator(device="cuda").manual_seed(1)
    q = torch.randn((Tq, hq, d), device="cuda", generator=gen).bfloat16()
    k = torch.randn((Tk, hkv, d), device="cuda", generator=gen).bfloat16()
    v = torch.randn_like(k)
    do = torch.randn_like(q)
    op = torch.empty_like(q)
    lsep = torch.empty((hq, Tq), device="cuda")
    ws = torch.zeros(c.cpattn_workspace_size(Tq, Tk, len(lens)), dtype=torch.uint8, device="cuda")
    st = c.make_step(cp, r, s, *tf)
    c.cpattn_fwd_step(q, k, v, plan.cu_local_dev, plan_k.cu_local_dev, len(lens), mode, st, 0.0, op, lsep, ws)
    torch.cuda.synchronize()
    fwd_ws = ws.cpu().numpy()
    lse = torch.full((hq, Tq), 30.0, device="cuda")     # any finite LSE: only the lists are read
    delta = torch.zeros((hq, Tq), device="cuda")
    dq = torch.zeros((Tq, hq, d), device="cuda")
    dk = torch.zeros((Tk, hkv, d), device="cuda")
    dv = torch.zeros_like(dk)
    c.cpattn_bwd_step(q, k, v, do, lse, delta, plan.cu_local_dev, plan_k.cu_local_dev, len(lens), mode, st, 0.0,
                      dq, dk, dv, ws)
    torch.cuda.synchronize()
    bwd_ws = ws.cpu().numpy()

    cu_q, pos_q = _plan(cu, cp, r, mode, tf)
    cu_k, pos_k = _plan(cu, cp, j, mode, tf)
    pos_q = np.concatenate([pos_q, np.zeros(pad, np.int64)])
    if split:
        want = tf_split.count_pairs(cu, cp, r, s, tf[0], tf[1])
    else:
        want = oracle.count_pairs(cu, cp, r, s, mode, tf[0], tf[1])
    assert c.cpattn_count_pairs(cu, mode, st) == want
    ra = _region(0, Tq, len(lens))
    rb = _region(ra["end"], Tk, len(lens))
    lists = [(fwd_ws, ra, True, True, 1, Tq), (bwd_ws, ra, True, False, 1, Tq), (bwd_ws, rb, False, False, hq // hkv, Tk)]
    for wsb, reg, prim_q, tail, mult, T_p in lists:
        status, items, order = _read_list(wsb, reg)
        if prim_q:
            check_list(status, items, order, True, cu_q, pos_q, cu_k, pos_k, T_p, tail, mode, tf, mult, want,
                       not split)
        else:
            check_list(status, items, order, False, cu_k, pos_k, cu_q, pos_q, T_p, tail, mode, tf, mult, want,
                       not split)
    return op, lsep


def _draw(seed):
    rng = np.random.default_rng(70000 + seed)
    kind = seed % 4
    hq, hkv = [(2, 1), (4, 4), (8, 2)][int(rng.integers(0, 3))]
    if kind == 2:       # teacher forcing at cp = 1, chunk sizes off the tile grid
        B, N = int(rng.integers(5, 150)), int(rng.integers(1, 6))
        return [2 * B * N] * int(rng.integers(1, 3)), 1, 0, oracle.TF_BLOCK, (B, N), hq, hkv
    if kind == 3:       # balanced teacher-forcing split
        cp = int(rng.integers(2, 5))
        B, N = int(rng.integers(32, 150)), cp * int(rng.integers(1, 4))
        return [2 * B * N] * int(rng.integers(1, 3)), cp, int(rng.integers(0, cp)), oracle.TF_BLOCK, (B, N), hq, hkv
    cp = int(rng.integers(1, 5))
    mode = oracle.CAUSAL if kind == 0 else oracle.BIDIR
    lens = []
    for _ in range(int(rng.integers(1, 7))):
        u = rng.random()
        n = 0 if u < 0.15 else int(rng.integers(1, 60)) if u < 0.35 else int(rng.integers(60, 1500))
        lens.append(n - n % (2 * cp) if cp > 1 else n)
    if sum(lens) == 0:
        lens[0] = 16 * cp
    return lens, cp, int(rng.integers(0, cp)), mode, (0, 0), hq, hkv


@pytest.mark.parametrize("seed", range(40))
def test_work_lists(cpa, seed):
    lens, cp, r, mode, tf, hq, hkv = _draw(seed)
    for s in range(cp):
        print(f"seed {seed}: lens {lens} cp {cp} rank {r} step {s} mode {mode} tf {tf} heads {hq}/{hkv}",
              flush=True)
        _run_case(cpa, lens, cp, r, s, mode, tf, hq, hkv)


@pytest.mark.parametrize("name", ["long_tail", "packed_varlen"])
def test_work_lists_config_shapes(cpa, name):
    """The work lists of two full-size workloads' sequence layouts (every ring
    step of rank 0), with few heads so that the brute force stays small."""
    import workloads
    w = workloads.WORKLOADS[name]
    for s in range(w.cp):
        print(f"{name}: step {s}", flush=True)
        _run_case(cpa, list(w.seqlens), w.cp, 0, s, w.mask, (0, 0), 4, 1)


def test_padded_query_rows_are_written(cpa):
    """A query buffer longer than its sequences: the forward writes every row
    (0 and lse = -inf past the last sequence), so the merge that follows
    reads no stale partial."""
    from context_attention_varlen_amd.ring import RankPlan
    lens, cp, r = [96, 40], 2, 1
    pad = 77
    cu = np.array([0, 96, 136], np.int32)
    plan = RankPlan.make(cu, cp, r)
    Tq = plan.tokens_local + pad
    q = torch.randn((Tq, 2, 128), device="cuda").bfloat16()
    k = torch.randn((plan.tokens_local, 1, 128), device="cuda").bfloat16()
    op = torch.full_like(q, float("nan"))
    lsep = torch.full((2, Tq), float("nan"), device="cuda")
    ws = torch.empty(cpa.cpattn_workspace_size(Tq, plan.tokens_local, 2), dtype=torch.uint8, device="cuda")
    out = torch.full((Tq, 2, 128), float("nan"), device="cuda")
    lse = torch.full((2, Tq), -float("inf"), device="cuda")
    for s in range(cp):
        st = cpa.make_step(cp, r, s)
        cpa.cpattn_fwd_step(q, k, k, plan.cu_local_dev, plan.cu_local_dev, 2, oracle.CAUSAL, st, 0.0, op, lsep, ws)
        cpa.cpattn_merge(out, lse, op, lsep)
    torch.cuda.synchronize()
    T = plan.tokens_local
    assert torch.all(op[T:].float() == 0) and torch.all(lsep[:, T:] == -float("inf"))
    assert torch.all(out[T:] == 0) and torch.all(lse[:, T:] == -float("inf"))
    assert torch.isfinite(out[:T]).all() and torch.isfinite(lse[:, :T]).all()
    # the work list itself, with the padded rows as items without segments
    _run_case(cpa, lens, cp, r, 0, oracle.CAUSAL, (0, 0), 2, 1, pad=pad)
