"""Seeded synthetic inputs for the blockwise context-parallel attention path.

This module only draws numbers and shapes.  It holds none of the method's
arithmetic: no partitioning, masking, attention or merging.  Both the CPU
oracle (through the tests and the benchmark) and the HIP library are fed from
the arrays produced here, so both sides always see identical inputs.

Workloads (the five shapes the library is measured and checked on):

  tiny_fp32     one causal sequence S=256, Hq=Hkv=2, d=64, fp32 N(0,1),
                zigzag cp=4, all 4 ranks x 4 steps.
  packed_varlen 8 causal sequences, lognormal(7.5, 1.0) lengths rescaled to
                sum to 16384, Hq=Hkv=16, d=128, bf16 N(0,1), cp=1.
  long_video    one causal sequence of 262144 tokens, zigzag cp=8, one rank's
                share (32768 local tokens), Hq=28/Hkv=4, d=128,
                bf16 0.5*N(0,1).
  tf_dit        teacher-forced video DiT: 12 time chunks x 2 streams x 3120
                tokens = 74880, Hq=Hkv=24, d=128, bf16 N(0,1), block mask.
  long_tail     65536 tokens: one 49152-token sequence plus short sequences
                with lengths uniform over multiples of 8 in [256, 2048];
                causal, zigzag cp=4 on every sequence, Hq=32/Hkv=8, d=128,
                bf16 q/k/v/dO N(0,1); forward and backward.
  tf_dit_split  the tf_dit sequence under the balanced teacher-forcing split
                over cp=3 ranks (4 time chunks per rank, 24960 local tokens),
                rank 0; forward and backward.

Dynamic-CP global batch (global_batch_lengths): 256 samples with
lognormal(8.0, 1.2) lengths (median ~3000 tokens, a tail capped at 131072),
rounded up to multiples of 16; it is planned into microbatches of per-sample
cp size and each microbatch's rank share is timed on the attention path
(Hq=32/Hkv=8, d=128, causal).

Page context: the long-tail length mix stands in for the variable-length
datasets of "Speeding up Variable-Length Training with Dynamic Context
Parallelism and NVIDIA Megatron Core" (section A3, long-tail distribution);
the 262144-token sequence stands in for the ~274K-token 1400-frame LongVILA
sample ("Scaling Video Training with Parallelism", section 1); the
teacher-forcing layout [clean history ; noisy target] follows the same blog's
section 4.  No dataset is used.

Random draws.  Each tensor gets its own child of ``SeedSequence(seed)`` (draw
order: lengths, q, k, v, dout), and is filled in fixed blocks of
``_BLOCK`` elements with one PCG64 stream per block, so the values do not
depend on the number of threads.  bf16 inputs are drawn as fp32 and rounded
to bf16 with round-to-nearest-even; the returned fp32 arrays hold exactly the
rounded values (the oracle upcasts those).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

CAUSAL, BIDIR, TF_BLOCK = 0, 1, 2
_BLOCK = 1 << 22


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seqlens: tuple            # global per-sequence lengths
    heads_q: int
    heads_kv: int
    head_dim: int
    dtype: str                # "f32" or "bf16"
    mask: int                 # CAUSAL / BIDIR / TF_BLOCK
    cp: int
    rank: int                 # primary rank evaluated
    value_scale: float = 1.0
    tf_chunk: int = 0         # teacher forcing: tokens per chunk (B)
    tf_num: int = 0           # teacher forcing: number of time chunks (N)
    backward: bool = False
    seed: int = 0

    @property
    def tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    def scaled(self, factor: int, name: Optional[str] = None) -> "Workload":
        """Same structure with every length divided by ``factor`` (test sizes)."""
        lens = tuple(int(l) // factor for l in self.seqlens)
        kw = dataclasses.asdict(self)
        kw.update(seqlens=lens, name=name or f"{self.name}/{factor}")
        if self.tf_chunk:
            kw["tf_chunk"] = self.tf_chunk // factor
        return Workload(**kw)


def lognormal_lengths(rng: np.random.Generator, n: int, total: int,
                      mu: float, sigma: float) -> list:
    """n lengths ~ lognormal(mu, sigma), rescaled to sum exactly to ``total``.

    floor(total * x / sum x); the remainder goes +1 to the largest fractional
    parts (stable by index); every length is at least 1.
    """
    x = rng.lognormal(mu, sigma, n)
    exact = total * x / x.sum()
    lens = np.floor(exact).astype(np.int64)
    order = np.argsort(-(exact - lens), kind="stable")
    lens[order[: total - int(lens.sum())]] += 1
    lens = np.maximum(lens, 1)
    return [int(v) for v in lens]


def long_tail_lengths(rng: np.random.Generator, total: int, long_len: int,
                      lo: int = 256, hi: int = 2048, quantum: int = 8) -> list:
    """One long sequence, then short ones uniform over multiples of
    ``quantum`` in [lo, hi] until ``total`` is filled exactly."""
    lens = [long_len]
    rem = total - long_len
    while rem > 0:
        length = quantum * int(rng.integers(lo // quantum, hi // quantum + 1))
        if rem - length < lo:
            length = rem if rem <= hi else rem - lo
        lens.append(length)
        rem -= length
    return lens


def global_batch_lengths(seed: int = 0, n: int = 256, mu: float = 8.0, sigma: float = 1.2,
                         cap: int = 131072, quantum: int = 16) -> list:
    """A global batch of n sample lengths with a long tail: lognormal(mu,
    sigma) tokens, rounded up to a multiple of ``quantum`` (so every sample
    can be zigzag-split up to cp = quantum / 2) and capped at ``cap``."""
    x = np.random.default_rng(seed).lognormal(mu, sigma, n)
    lens = np.minimum(np.ceil(x / quantum).astype(np.int64) * quantum, cap)
    return [int(v) for v in np.maximum(lens, quantum)]


def _c2_lengths() -> tuple:
    return tuple(lognormal_lengths(np.random.default_rng(0), 8, 16384, 7.5, 1.0))


def _c5_lengths() -> tuple:
    return tuple(long_tail_lengths(np.random.default_rng(0), 65536, 49152))


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", (256,), 2, 2, 64, "f32", CAUSAL, 4, 0),
    "packed_varlen": Workload("packed_varlen", _c2_lengths(), 16, 16, 128, "bf16", CAUSAL, 1, 0),
    "long_video": Workload("long_video", (262144,), 28, 4, 128, "bf16", CAUSAL, 8, 0,
                           value_scale=0.5),
    "tf_dit": Workload("tf_dit", (74880,), 24, 24, 128, "bf16", TF_BLOCK, 1, 0,
                       tf_chunk=3120, tf_num=12),
    "long_tail": Workload("long_tail", _c5_lengths(), 32, 8, 128, "bf16", CAUSAL, 4, 0,
                          backward=True),
    "tf_dit_split": Workload("tf_dit_split", (74880,), 24, 24, 128, "bf16", TF_BLOCK, 3, 0,
                             tf_chunk=3120, tf_num=12, backward=True),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(seed_seq: np.random.SeedSequence, shape) -> np.ndarray:
    """Standard normal fp32 array, filled block-wise with spawned PCG64 streams."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    nblk = (n + _BLOCK - 1) // _BLOCK
    children = seed_seq.spawn(nblk)

    def fill(i):
        g = np.random.Generator(np.random.PCG64(children[i]))
        g.standard_normal(out=out[i * _BLOCK:(i + 1) * _BLOCK], dtype=np.float32)

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest even); returns fp32 holding
    exactly the bf16 values.  Inputs are finite."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def draw(w: Workload, names=("q", "k", "v", "dout"), scale_override: Optional[float] = None) -> dict:
    """Draw the global THD tensors of a workload.

    Returns fp32 numpy arrays [T, H, d] (bf16-representable when w.dtype is
    bf16).  ``dout`` is drawn only for backward workloads.
    """
    root = np.random.SeedSequence(w.seed)
    kids = dict(zip(("q", "k", "v", "dout"), root.spawn(4)))
    scale = w.value_scale if scale_override is None else scale_override
    out = {}
    for nm in names:
        if nm == "dout" and not w.backward:
            continue
        h = w.heads_q if nm in ("q", "dout") else w.heads_kv
        x = normal_f32(kids[nm], (w.tokens, h, w.head_dim))
        if nm != "dout" and scale != 1.0:
            x *= np.float32(scale)
        if w.dtype == "bf16":
            x = round_bf16(x)
        out[nm] = x
    return out


def sample_rows(rng: np.random.Generator, n_rows: int, count: int,
                edges=()) -> np.ndarray:
    """Seeded row sample: the given edge rows (clipped to range) plus uniform
    random rows, sorted and unique."""
    picks = [int(e) for e in edges if 0 <= int(e) < n_rows]
    if count > 0 and n_rows > 0:
        picks.extend(rng.integers(0, n_rows, size=count).tolist())
    return np.unique(np.asarray(picks, dtype=np.int64))
