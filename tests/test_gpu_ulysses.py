"""GPU parity of the one-device Ulysses exchange ("Scaling Video Training with
Parallelism", SP landscape: DeepSpeed-Ulysses, USP / LoongTrain) through the
C ABI: the sequence->head gather and head->sequence scatter are bit-exact
against the oracle, and a whole Ulysses forward (gather each head group,
attention over all tokens with cp = 1, scatter the output back into the
shards) equals the oracle's attention over the unsharded batch."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads  # noqa: E402
from oracle import ulysses  # noqa: E402
from tests._gpu import check_lse, check_out, dev  # noqa: E402


@pytest.fixture(scope="module")
def cpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_varlen_amd as c
    return c


@pytest.mark.parametrize("lens,H,d,dtype", [([96, 160, 32, 224], 8, 128, torch.bfloat16),
                                             ([64, 64, 64], 6, 64, torch.float32),
                                             ([1, 255], 4, 128, torch.bfloat16)])
def test_exchange_bit_exact(cpa, lens, H, d, dtype):
    n = len(lens)
    H = H - H % n if H % n else H
    rng = np.random.default_rng(4)
    shards_np = [rng.standard_normal((t, H, d)).astype(np.float32) for t in lens]
    shards = [dev(s, dtype) for s in shards_np]
    ref_shards = [s.cpu().numpy() if dtype == torch.float32 else s.float().cpu().numpy() for s in shards]
    back = [torch.zeros_like(s) for s in shards]
    for g in range(n):
        # strided destination view: a slice of a wider tensor
        wide = torch.zeros((sum(lens) + 3, 2 * (H // n), d), dtype=dtype, device="cuda")
        out = wide[:, : H // n]
        cpa.cpattn_seq_to_head(shards, g, out)
        torch.cuda.synchronize()
        want = ulysses.seq_to_head(ref_shards, g, n)
        assert np.array_equal(out[: sum(lens)].float().cpu().numpy(), want)
        assert torch.count_nonzero(wide[:, H // n:]) == 0
        cpa.cpattn_head_to_seq(out, g, back)
    torch.cuda.synchronize()
    for a, b in zip(back, shards):
        assert torch.equal(a, b)


@pytest.mark.parametrize("lens,n,hq,hkv,mode", [([300, 212], 4, 8, 4, oracle.CAUSAL),
                                                ([256, 256, 128, 128], 2, 4, 2, oracle.BIDIR),
                                                ([512], 2, 6, 2, oracle.CAUSAL)])
def test_ulysses_forward_equals_oracle(cpa, lens, n, hq, hkv, mode):
    d = 128
    rng = np.random.default_rng(12)
    T = sum(lens)
    x = {k: workloads.round_bf16(rng.standard_normal((T, h, d), dtype=np.float32))
         for k, h in (("q", hq), ("k", hkv), ("v", hkv))}
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    seq = np.repeat(np.arange(len(lens)), lens)
    pos = np.arange(T) - cu[seq]
    o_ref, l_ref = oracle.attention(x["q"], x["k"], x["v"], seq, pos, seq, pos, mode)
    sh = {k: [dev(s, torch.bfloat16) for s in ulysses.contiguous_shards(v, n)] for k, v in x.items()}
    out_shards = [torch.zeros((T // n, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    cu_dev = torch.from_numpy(cu).cuda()
    for g in range(n):
        q = torch.empty((T, hq // n, d), dtype=torch.bfloat16, device="cuda")
        k = torch.empty((T, hkv // n, d), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        cpa.cpattn_seq_to_head(sh["q"], g, q)
        cpa.cpattn_seq_to_head(sh["k"], g, k)
        cpa.cpattn_seq_to_head(sh["v"], g, v)
        o = torch.empty_like(q)
        lse = torch.empty((hq // n, T), dtype=torch.float32, device="cuda")
        ws = torch.empty(cpa.cpattn_workspace_size(T, T, len(lens)), dtype=torch.uint8, device="cuda")
        cpa.cpattn_fwd_step(q, k, v, cu_dev, cu_dev, len(lens), mode, cpa.make_step(1, 0, 0), 0.0, o, lse, ws)
        cpa.cpattn_head_to_seq(o, g, out_shards)
        torch.cuda.synchronize()
        hg = hq // n
        check_lse(lse.cpu().numpy(), l_ref[g * hg:(g + 1) * hg])
    got = torch.cat(out_shards).float().cpu().numpy()
    check_out(got, o_ref, "bf16")
