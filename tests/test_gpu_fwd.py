"""GPU parity of the zigzag partition, the forward ring steps and the LSE
merge against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads  # noqa: E402
from tests._gpu import (check_lse, check_out, dev, oracle_rank_full, oracle_step,  # noqa: E402
                        tdtype)


@pytest.fixture(scope="module")
def cpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_varlen_amd as c
    return c


def _inputs(seed, lens, hq, hkv, d, dtype, scale=1.0, dout=False):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    x = {"q": rng.standard_normal((T, hq, d), dtype=np.float32) * scale,
         "k": rng.standard_normal((T, hkv, d), dtype=np.float32) * scale,
         "v": rng.standard_normal((T, hkv, d), dtype=np.float32) * scale}
    if dout:
        x["dout"] = rng.standard_normal((T, hq, d), dtype=np.float32)
    if dtype == "bf16":
        x = {k: workloads.round_bf16(v) for k, v in x.items()}
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return x, cu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("lens,cp", [([256], 4), ([64, 0, 192, 16], 4), ([40, 24, 8], 2), ([37, 5], 1)])
def test_partition_bitexact_and_roundtrip(cpa, dtype, lens, cp):
    from context_attention_varlen_amd.ring import RankPlan, partition
    x, cu = _inputs(1, lens, 3, 3, 64, dtype)
    g = dev(x["q"], tdtype(dtype))
    back = torch.zeros_like(g)
    for r in range(cp):
        plan = RankPlan.make(cu, cp, r)
        cu_l_or, l2g, _, _ = oracle.local_rows(cu, cp, r)
        assert np.array_equal(plan.cu_local, cu_l_or)
        _, l2g_lib = cpa.cpattn_partition_index(cu, cp, r)
        assert np.array_equal(l2g_lib, l2g)
        loc = partition(g, plan)
        assert torch.equal(loc.cpu(), g.cpu()[torch.from_numpy(l2g)])
        cpa.cpattn_unpartition(loc, back, plan.cu_global_dev, plan.num_seqs, cp, r)
    torch.cuda.synchronize()
    assert torch.equal(back.cpu(), g.cpu())


@pytest.mark.parametrize("count", [0, 1, 3, 4, 5, 1023, (1 << 20) + 3])
def test_fill_f32(cpa, count):
    """Exact fill of count values (16-byte stores plus a ragged tail), the
    ring's -inf and 0 included; nothing past count is written."""
    for value in (0.0, -float("inf"), 1.5):
        buf = torch.full((count + 64,), 7.0, device="cuda")
        cpa.cpattn_fill_f32(buf[:count], value)
        torch.cuda.synchronize()
        head, rest = buf[:count].cpu(), buf[count:].cpu()
        assert torch.equal(head, torch.full((count,), value))
        assert torch.all(rest == 7.0)


def test_device_info(cpa):
    cus, khz = cpa.cpattn_device_info(0)
    assert cus == torch.cuda.get_device_properties(0).multi_processor_count
    assert 100_000 < khz < 10_000_000


@pytest.mark.parametrize("dtype,heads,d", [("bf16", 28, 128), ("f32", 80, 128), ("bf16", 1, 64), ("f32", 7, 64)])
def test_partition_rows_per_workgroup(cpa, dtype, heads, d):
    """Gather and scatter where a workgroup holds one row (80 fp32 heads: 2560
    16-byte chunks, two passes), a few rows (28 heads) or many (1 head), with
    a partial last workgroup: bit-exact against the index map."""
    from context_attention_varlen_amd.ring import RankPlan, partition
    lens = [392, 0, 56, 8 * 37]
    cp = 4
    rng = np.random.default_rng(5)
    T = sum(lens)
    g = dev(rng.standard_normal((T, heads, d), dtype=np.float32), tdtype(dtype))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    back = torch.zeros_like(g)
    for r in range(cp):
        plan = RankPlan.make(cu, cp, r)
        _, l2g, _, _ = oracle.local_rows(cu, cp, r)
        loc = partition(g, plan)
        assert torch.equal(loc.cpu(), g.cpu()[torch.from_numpy(l2g)])
        cpa.cpattn_unpartition(loc, back, plan.cu_global_dev, plan.num_seqs, cp, r)
    torch.cuda.synchronize()
    assert torch.equal(back.cpu(), g.cpu())


def _run_ring(cpa, x, cu, cp, r, mode, dtype, hq, hkv, tf=(0, 0), keep=True):
    from context_attention_varlen_amd.ring import RankPlan, partition, ring_forward
    plan = RankPlan.make(cu, cp, r)
    td = tdtype(dtype)
    qg, kg, vg = dev(x["q"], td), dev(x["k"], td), dev(x["v"], td)
    q = partition(qg, plan)
    ks = [partition(kg, plan, j) for j in range(cp)]
    vs = [partition(vg, plan, j) for j in range(cp)]
    bufs, parts = ring_forward(q, ks, vs, plan, mode, tf=tf, keep_partials=keep)
    torch.cuda.synchronize()
    return plan, bufs, parts


def test_tiny_fp32_all_ranks_all_steps(cpa):
    """One causal 256-token sequence, 2 heads, d=64, fp32, cp=4: every rank,
    every step, then the merge; compared to full unsplit attention."""
    w = workloads.WORKLOADS["tiny_fp32"]
    x = workloads.draw(w)
    cu = w.cu_seqlens
    full_o, full_l = oracle.attention(x["q"], x["k"], x["v"], np.zeros(256, int), np.arange(256),
                                      np.zeros(256, int), np.arange(256), oracle.CAUSAL)
    for r in range(w.cp):
        plan, bufs, parts = _run_ring(cpa, x, cu, w.cp, r, oracle.CAUSAL, "f32", 2, 2)
        for s, (op, lp) in enumerate(parts):
            o_ref, l_ref = oracle_step(x, cu, w.cp, r, s, oracle.CAUSAL)
            check_out(op.cpu().numpy(), o_ref, "f32")
            check_lse(lp.cpu().numpy(), l_ref, tol=1e-5)
        _, l2g, _, _ = oracle.local_rows(cu, w.cp, r)
        check_out(bufs.out.cpu().numpy(), full_o[l2g], "f32")
        check_lse(bufs.lse.cpu().numpy(), full_l[:, l2g], tol=1e-5)


SMALL = [
    # lens, cp, hq, hkv, d, mask, tf
    ([512], 2, 4, 2, 128, oracle.CAUSAL, (0, 0)),
    ([384, 128, 64], 4, 4, 1, 128, oracle.CAUSAL, (0, 0)),
    ([200, 56, 336], 4, 2, 2, 128, oracle.CAUSAL, (0, 0)),
    ([333, 1, 70], 1, 3, 3, 128, oracle.CAUSAL, (0, 0)),
    ([300, 77], 1, 4, 2, 128, oracle.BIDIR, (0, 0)),
    ([96, 160], 2, 2, 2, 128, oracle.BIDIR, (0, 0)),
    ([2 * 3 * 37], 1, 2, 2, 128, oracle.TF_BLOCK, (37, 3)),
    ([2 * 4 * 100, 2 * 4 * 100], 1, 4, 2, 128, oracle.TF_BLOCK, (100, 4)),
    ([256, 128], 2, 4, 4, 64, oracle.CAUSAL, (0, 0)),
    ([200], 1, 2, 1, 64, oracle.TF_BLOCK, (25, 4)),
    # tile counts around the two-tiles-per-trip loop of the pipelined forward:
    # 16 key tiles with a partial last one, 3 + 3, and 1 + 11 at d = 64
    ([1000, 24], 1, 2, 1, 128, oracle.CAUSAL, (0, 0)),
    ([192, 130], 1, 2, 2, 128, oracle.BIDIR, (0, 0)),
    ([64, 704], 1, 2, 2, 64, oracle.CAUSAL, (0, 0)),
]


@pytest.mark.parametrize("lens,cp,hq,hkv,d,mode,tf", SMALL)
def test_bf16_steps_and_merge(cpa, lens, cp, hq, hkv, d, mode, tf):
    x, cu = _inputs(7, lens, hq, hkv, d, "bf16")
    for r in sorted({0, cp - 1}):
        plan, bufs, parts = _run_ring(cpa, x, cu, cp, r, mode, "bf16", hq, hkv, tf)
        for s, (op, lp) in enumerate(parts):
            o_ref, l_ref = oracle_step(x, cu, cp, r, s, mode, tf)
            check_out(op.float().cpu().numpy(), o_ref, "bf16")
            check_lse(lp.cpu().numpy(), l_ref)
        o_ref, l_ref = oracle_rank_full(x, cu, cp, r, mode, tf)
        check_out(bufs.out.cpu().numpy(), o_ref, "bf16")
        check_lse(bufs.lse.cpu().numpy(), l_ref)


def test_packed_varlen_full(cpa):
    """8 lognormal-length causal sequences (16384 tokens), 16 heads, d=128,
    cp=1: every output row against the fp64 oracle."""
    w = workloads.WORKLOADS["packed_varlen"]
    x = workloads.draw(w)
    cu = w.cu_seqlens
    plan, bufs, parts = _run_ring(cpa, x, cu, 1, 0, oracle.CAUSAL, "bf16", 16, 16, keep=False)
    seq = np.repeat(np.arange(8), np.diff(cu))
    pos = np.arange(w.tokens) - cu[seq]
    o_ref, l_ref = oracle.attention(x["q"], x["k"], x["v"], seq, pos, seq, pos, oracle.CAUSAL)
    check_out(bufs.out.cpu().numpy(), o_ref, "bf16")
    check_lse(bufs.lse.cpu().numpy(), l_ref)


def test_bad_device_cu_seqlens_sets_status(cpa):
    """Non-monotone cu_seqlens on the device: no item is scheduled, nothing is
    written, and the workspace status reports INVALID_ARG."""
    from context_attention_varlen_amd.ring import ForwardBuffers
    q = torch.randn(64, 2, 128, device="cuda").bfloat16()
    cu_bad = torch.tensor([0, 40, 20, 64], dtype=torch.int32, device="cuda")
    bufs = ForwardBuffers.make(q, 64, 3)
    bufs.out_partial.fill_(7.0)
    cpa.cpattn_fwd_step(q, q, q, cu_bad, cu_bad, 3, cpa.CAUSAL, cpa.make_step(1, 0, 0), 0.0,
                        bufs.out_partial, bufs.lse_partial, bufs.workspace)
    assert cpa.cpattn_workspace_status(bufs.workspace) == cpa.ERR_INVALID_ARG
    assert torch.all(bufs.out_partial == 7.0)
    cu_ok = torch.tensor([0, 20, 40, 64], dtype=torch.int32, device="cuda")
    cpa.cpattn_fwd_step(q, q, q, cu_ok, cu_ok, 3, cpa.CAUSAL, cpa.make_step(1, 0, 0), 0.0,
                        bufs.out_partial, bufs.lse_partial, bufs.workspace)
    assert cpa.cpattn_workspace_status(bufs.workspace) == cpa.OK


def test_merge_passthrough_bit_exact(cpa):
    T, H, d = 300, 3, 128
    out = torch.randn(T, H, d, device="cuda")
    lse = torch.randn(H, T, device="cuda")
    lse[1, 5:50] = -float("inf")
    o0, l0 = out.clone(), lse.clone()
    part = torch.randn(T, H, d, device="cuda").bfloat16()
    lp = torch.full((H, T), -float("inf"), device="cuda")
    cpa.cpattn_merge(out, lse, part, lp)
    torch.cuda.synchronize()
    # finite running rows pass through bit-exact; rows never merged (running
    # lse -inf) become the result over no keys, 0
    o0[5:50, 1, :] = 0.0
    assert torch.equal(out, o0) and torch.equal(lse, l0)
    # running rows at -inf take the partial exactly
    lp2 = torch.randn(H, T, device="cuda")
    out.zero_()
    lse.fill_(-float("inf"))
    cpa.cpattn_merge(out, lse, part, lp2)
    torch.cuda.synchronize()
    assert torch.equal(out.permute(1, 0, 2), part.float().permute(1, 0, 2)) and torch.equal(lse, lp2)


def test_merge_first_needs_no_output_init(cpa):
    """From the starting state lse = -inf the running output's old contents
    do not matter: rows with a finite partial LSE take the partial exactly,
    rows whose partial is -inf too become 0 (the result over no keys)."""
    T, H, d = 300, 3, 128
    out = torch.full((T, H, d), float("nan"), device="cuda")
    lse = torch.full((H, T), -float("inf"), device="cuda")
    part = torch.randn(T, H, d, device="cuda").bfloat16()
    lp = torch.randn(H, T, device="cuda")
    lp[0, 7:90] = -float("inf")
    lp[2, 250:] = -float("inf")
    cpa.cpattn_merge(out, lse, part, lp)
    torch.cuda.synchronize()
    live = torch.isfinite(lp).t()                    # [T, H]
    ref = torch.where(live[..., None], part.float(), torch.zeros_like(out))
    assert torch.equal(out, ref) and torch.equal(lse, lp)


def test_merge_against_oracle(cpa):
    rng = np.random.default_rng(3)
    T, H, d = 257, 2, 128
    o = rng.standard_normal((T, H, d)).astype(np.float32)
    l = (rng.standard_normal((H, T)) * 4).astype(np.float32)
    op = workloads.round_bf16(rng.standard_normal((T, H, d)).astype(np.float32))
    lp = (rng.standard_normal((H, T)) * 4).astype(np.float32)
    lp[0, :20] = -np.inf
    l[1, 30:40] = -np.inf
    o_ref, l_ref = oracle.merge(o, l, op, lp)
    out, lse = dev(o, torch.float32), dev(l, torch.float32)
    cpa.cpattn_merge(out, lse, dev(op, torch.bfloat16), dev(lp, torch.float32))
    torch.cuda.synchronize()
    np.testing.assert_allclose(out.cpu().numpy(), o_ref, atol=2e-6, rtol=2e-6)
    check_lse(lse.cpu().numpy(), l_ref, tol=2e-6)
