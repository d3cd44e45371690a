"""CPU fp64 oracle for blockwise (zigzag ring) varlen attention.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plainly written reference
that the HIP library is checked against.  Only the test suite, the smoke check
and the CPU-baseline leg of the benchmark may import it; the library itself
never does, and nothing here imports the library.

What it follows (page titles as given at the top of each page):
  * "Scaling Video Training with Parallelism", section 1: splitting a sample
    over ranks must not change what the model sees or the loss, so chunked,
    merged attention has to equal attention over the unsplit sequence.
  * same page, section 2 (Ring Attention paragraph): blockwise attention while
    key/value blocks stream around the ranks.
  * same page, section 4: the teacher-forcing sequence [clean history ; noisy
    target] and what each stream may see, and the balanced split that gives
    every rank the clean/noisy chunks of the same time segments (tf_split.py).
  * same page, SP landscape (DeepSpeed-Ulysses, USP / LoongTrain): the
    sequence-to-head all-to-all, on one device a gather (ulysses.py).
  * LongCat-Video context-parallel page: the height/width token split with a
    near-square choice of factors (hw_split.py).
  * LongVILA article (ZIGZAG-RINGATTN, "balancing compute"): the zigzag chunk
    assignment (the chunk rule itself is not printed; see zigzag.py).
  * "Speeding up Variable-Length Training with Dynamic Context Parallelism and
    NVIDIA Megatron Core", section A2: packed THD layout with cu_seqlens and
    FLOPs counted from real sequence lengths; same section (Eq. 1-3 and the
    three-stage heuristic) and section A7 (grid search near the knee of the
    budget curve): the Dynamic-CP microbatch planner (dynamic_cp.py).

Pins (what each function is checked against, other than itself) live in
tests/test_oracle_*.py.  Every function here is pinned; none is marked
"parity unpinned".
"""
from .masks import CAUSAL, BIDIR, TF_BLOCK, allowed, seq_mask  # noqa: F401
from .zigzag import (rank_chunks, local_rows, partition, count_pairs,  # noqa: F401
                     step_source)
from .softmax_attention import attention, attention_backward, bwd_delta, default_scale  # noqa: F401
from .lse_merge import merge  # noqa: F401
from . import dynamic_cp, hw_split, tf_split, ulysses  # noqa: F401
