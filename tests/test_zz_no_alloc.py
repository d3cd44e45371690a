"""The allocation-free forward step (schedule workspace in the library's own
device array) against cpattn_fwd_step with a caller workspace, through the C
ABI: bit-identical partial output and LSE on two calls in a row, the second
on a smaller batch, so whatever the first call left in the array cannot leak
into the second."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402


@pytest.fixture(scope="module")
def cpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_varlen_amd as c
    return c


def _case(c, lens, cp, r, s, hq, hkv, seed):
    from context_attention_varlen_amd.ring import RankPlan
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    plan = RankPlan.make(cu, cp, r)
    gen = torch.Generator(device="cuda").manual_seed(seed)
    T = plan.tokens_local
    q = torch.randn((T, hq, 128), device="cuda", generator=gen).bfloat16()
    k = torch.randn((T, hkv, 128), device="cuda", generator=gen).bfloat16()
    v = torch.randn((T, hkv, 128), device="cuda", generator=gen).bfloat16()
    st = c.make_step(cp, r, s)
    ws = torch.empty(c.cpattn_workspace_size(T, T, len(lens)), dtype=torch.uint8, device="cuda")
    o_ref = torch.empty_like(q)
    l_ref = torch.empty((hq, T), device="cuda")
    c.cpattn_fwd_step(q, k, v, plan.cu_local_dev, plan.cu_local_dev, len(lens), oracle.CAUSAL, st, 0.0,
                      o_ref, l_ref, ws)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((hq, T), float("nan"), device="cuda")
    c.cpattn_fwd_step_noalloc(q, k, v, plan.cu_local_dev, plan.cu_local_dev, len(lens), oracle.CAUSAL, st, 0.0,
                              o, lse)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "partial output differs"
    assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32)), "partial LSE differs"
    return int(len(lens))


def test_noalloc_matches_workspace_call_twice(cpa):
    # first call: a long-tail batch (49152 + short sequences at cp = 4),
    # second: a smaller batch with fewer sequences and another rank / step
    big = [12288, 1784, 1400, 1176, 736, 808, 328, 384]
    print("noalloc call 1: long-tail batch, cp 4, rank 0, step 1", flush=True)
    _case(cpa, big, 4, 0, 1, 8, 2, 0)
    print("noalloc call 2: small batch, cp 2, rank 1, step 0", flush=True)
    _case(cpa, [512, 96], 2, 1, 0, 4, 4, 1)


def test_noalloc_rejects_shapes_beyond_the_array(cpa):
    """A shape whose workspace exceeds the array is refused with
    CPATTN_ERR_WORKSPACE before anything is enqueued."""
    T = 4_000_000
    assert cpa.cpattn_workspace_size(T, T, 1) > (16 << 20)
    q = torch.empty((T, 1, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, T), device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    with pytest.raises(cpa.CpattnError) as e:
        cpa.cpattn_fwd_step_noalloc(q, q, q, cu, cu, 1, oracle.CAUSAL, cpa.make_step(1, 0, 0), 0.0, q, lse)
    assert e.value.status == cpa.ERR_WORKSPACE
