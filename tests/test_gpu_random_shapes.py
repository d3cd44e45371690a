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
from tests._gpu import check_lse, check_out  # noqa: E402
from tests.test_gpu_bwd import _check_grad, _inputs, oracle_grads, run_gpu  # noqa: E402


@pytest.fixture(scope="module")
def cpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_varlen_amd as c
    return c


def _draw(seed):
    rng = np.random.default_rng(20000 + seed)
    hq, hkv = [(2, 1), (4, 2), (3, 3), (8, 2), (6, 3)][int(rng.integers(0, 5))]
    d = int(rng.choice([64, 128]))
    if rng.random() < 0.2:
        # teacher forcing at cp = 1 (cp > 1 has its own tests): 1-2 sequences
        # of [clean ; noisy] with random chunk size B and count N
        B, N = int(rng.integers(1, 120)), int(rng.integers(1, 6))
        return [2 * B * N] * int(rng.integers(1, 3)), 1, 0, hq, hkv, d, oracle.TF_BLOCK, (B, N)
    cp = int(rng.choice([1, 2, 3, 4]))
    mode = oracle.CAUSAL if rng.random() < 0.7 else oracle.BIDIR
    nseq = int(rng.integers(1, 7))
    quantum = 2 * cp
    lens = []
    for _ in range(nseq):
        kind = rng.random()
        if kind < 0.15:
            n = 0
        elif kind < 0.35:
            n = int(rng.integers(1, 40))
        else:
            n = int(rng.integers(40, 700))
        lens.append(n - n % quantum if cp > 1 else n)
    if sum(lens) == 0:
        lens[0] = 8 * quantum
    rank = int(rng.integers(0, cp))
    return lens, cp, rank, hq, hkv, d, mode, (0, 0)


@pytest.mark.parametrize("seed", range(48))
def test_random_shape(cpa, seed):
    lens, cp, r, hq, hkv, d, mode, tf = _draw(seed)
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
