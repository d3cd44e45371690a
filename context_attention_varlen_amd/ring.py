"""Host loop of one context-parallel rank, iterated on one GPU.

"Scaling Video Training with Parallelism" (section 2, Ring Attention
paragraph): each rank attends its local queries to one K/V block at a time
while the blocks travel round the ring.  With one GPU the ring's transport
becomes a choice of which source rank's K/V share to pass at each step; the
shapes per step are the real per-rank shapes.  Everything numeric happens in
libcpattn's kernels; this module only allocates buffers with torch and
orders the calls on one stream.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

from . import (cpattn_bwd_preprocess, cpattn_bwd_step, cpattn_fill_f32, cpattn_fwd_step, cpattn_merge,
               cpattn_partition, cpattn_partition_index, cpattn_partition_index_tf, cpattn_partition_tf,
               cpattn_step_source, cpattn_workspace_size, make_step)


@dataclasses.dataclass
class RankPlan:
    """Index plan and device buffers of rank `rank` out of `cp`."""
    cp: int
    rank: int
    cu_global: np.ndarray
    cu_local: np.ndarray
    cu_global_dev: torch.Tensor
    cu_local_dev: torch.Tensor
    num_seqs: int
    tokens_local: int
    tf: tuple = (0, 0)   # (B, N) for the balanced teacher-forcing split, else zigzag

    @staticmethod
    def make(cu_global, cp: int, rank: int, device="cuda", tf=None) -> "RankPlan":
        """Zigzag plan, or with tf = (B, N) and cp > 1 the balanced
        teacher-forcing split."""
        cu_g = np.ascontiguousarray(cu_global, dtype=np.int32)
        split = (int(tf[0]), int(tf[1])) if tf is not None and cp > 1 and tf[0] > 0 else (0, 0)
        if split[0]:
            cu_l, _ = cpattn_partition_index_tf(cu_g, cp, rank, split[0], split[1], with_map=False)
        else:
            cu_l, _ = cpattn_partition_index(cu_g, cp, rank, with_map=False)
        return RankPlan(cp, rank, cu_g, cu_l, torch.from_numpy(cu_g).to(device),
                        torch.from_numpy(cu_l).to(device), len(cu_g) - 1, int(cu_l[-1]), split)


def partition(x_global: torch.Tensor, plan: RankPlan, rank: Optional[int] = None) -> torch.Tensor:
    """Rank's share of a global THD tensor (device gather) under the plan's
    split."""
    r = plan.rank if rank is None else rank
    out = torch.empty((plan.tokens_local,) + tuple(x_global.shape[1:]), dtype=x_global.dtype,
                      device=x_global.device)
    if plan.tf[0]:
        cpattn_partition_tf(x_global, out, plan.cu_global_dev, plan.num_seqs, plan.cp, r, plan.tf[0], plan.tf[1])
    else:
        cpattn_partition(x_global, out, plan.cu_global_dev, plan.num_seqs, plan.cp, r)
    return out


@dataclasses.dataclass
class ForwardBuffers:
    out: torch.Tensor          # fp32 [T, Hq, d] running output
    lse: torch.Tensor          # fp32 [Hq, T] running LSE
    out_partial: torch.Tensor  # [T, Hq, d] input dtype
    lse_partial: torch.Tensor  # fp32 [Hq, T]
    workspace: torch.Tensor

    @staticmethod
    def make(q_local: torch.Tensor, tokens_k: int, num_seqs: int) -> "ForwardBuffers":
        t, hq, d = q_local.shape
        dev = q_local.device
        ws = torch.empty(cpattn_workspace_size(t, tokens_k, num_seqs), dtype=torch.uint8, device=dev)
        return ForwardBuffers(torch.zeros((t, hq, d), dtype=torch.float32, device=dev),
                              torch.full((hq, t), -float("inf"), dtype=torch.float32, device=dev),
                              torch.empty_like(q_local),
                              torch.empty((hq, t), dtype=torch.float32, device=dev), ws)

    def reset(self):
        """The ring's starting state, lse = -inf (library fill kernel); the merge
        writes every running row whose lse is -inf, so out needs no fill."""
        cpattn_fill_f32(self.lse, -float("inf"))


def ring_forward(q_local: torch.Tensor, k_shares: List[torch.Tensor], v_shares: List[torch.Tensor],
                 plan: RankPlan, mask_mode: int, tf=(0, 0), scale: float = 0.0,
                 bufs: Optional[ForwardBuffers] = None, keep_partials: bool = False):
    """cp forward steps and merges for rank plan.rank.  Returns the buffers
    (and the per-step partials when keep_partials)."""
    if bufs is None:
        bufs = ForwardBuffers.make(q_local, k_shares[0].shape[0], plan.num_seqs)
    else:
        bufs.reset()
    partials = []
    for s in range(plan.cp):
        st = make_step(plan.cp, plan.rank, s, tf[0], tf[1])
        j = cpattn_step_source(st)
        cpattn_fwd_step(q_local, k_shares[j], v_shares[j], plan.cu_local_dev, plan.cu_local_dev,
                        plan.num_seqs, mask_mode, st, scale, bufs.out_partial, bufs.lse_partial,
                        bufs.workspace)
        if keep_partials:
            partials.append((bufs.out_partial.clone(), bufs.lse_partial.clone()))
        cpattn_merge(bufs.out, bufs.lse, bufs.out_partial, bufs.lse_partial)
    return bufs, partials


def ring_backward(q_local, k_shares, v_shares, dout_local, bufs: ForwardBuffers, plan: RankPlan,
                  mask_mode: int, tf=(0, 0), scale: float = 0.0, grads=None):
    """Backward of rank plan.rank from the final merged (out, lse): returns
    (dq [T,Hq,d], dk [cp][Tk,Hkv,d], dv [cp][Tk,Hkv,d]) in fp32, dk/dv indexed
    by source rank."""
    t, hq, d = q_local.shape
    dev = q_local.device
    if grads is None:
        dq = torch.zeros((t, hq, d), dtype=torch.float32, device=dev)
        dk = [torch.zeros(k.shape, dtype=torch.float32, device=dev) for k in k_shares]
        dv = [torch.zeros(v.shape, dtype=torch.float32, device=dev) for v in v_shares]
        delta = torch.empty((hq, t), dtype=torch.float32, device=dev)
    else:
        dq, dk, dv, delta = grads
        for x in [dq] + dk + dv:
            cpattn_fill_f32(x, 0.0)
    cpattn_bwd_preprocess(bufs.out, dout_local, delta)
    for s in range(plan.cp):
        st = make_step(plan.cp, plan.rank, s, tf[0], tf[1])
        j = cpattn_step_source(st)
        cpattn_bwd_step(q_local, k_shares[j], v_shares[j], dout_local, bufs.lse, delta, plan.cu_local_dev,
                        plan.cu_local_dev, plan.num_seqs, mask_mode, st, scale, dq, dk[j], dv[j],
                        bufs.workspace)
    return dq, dk, dv, delta


@dataclasses.dataclass
class StepBuffers:
    """Device buffers of one rank's whole step: the gathered shares, the
    forward state (with a second partial pair, so a merge can overlap the
    next forward step) and the fp32 gradients."""
    q: torch.Tensor
    dout: Optional[torch.Tensor]
    ks: List[torch.Tensor]
    vs: List[torch.Tensor]
    fwd: ForwardBuffers
    partial2: tuple
    dq: Optional[torch.Tensor]
    dk: Optional[List[torch.Tensor]]
    dv: Optional[List[torch.Tensor]]
    delta: Optional[torch.Tensor]

    @staticmethod
    def make(plan: RankPlan, heads_q: int, heads_kv: int, head_dim: int, dtype, backward: bool,
             device="cuda") -> "StepBuffers":
        tl = plan.tokens_local
        q = torch.empty((tl, heads_q, head_dim), dtype=dtype, device=device)
        ks = [torch.empty((tl, heads_kv, head_dim), dtype=dtype, device=device) for _ in range(plan.cp)]
        vs = [torch.empty_like(ks[0]) for _ in range(plan.cp)]
        fb = ForwardBuffers.make(q, tl, plan.num_seqs)
        p2 = (torch.empty_like(fb.out_partial), torch.empty_like(fb.lse_partial))
        if not backward:
            return StepBuffers(q, None, ks, vs, fb, p2, None, None, None, None)
        f32 = dict(dtype=torch.float32, device=device)
        return StepBuffers(q, torch.empty_like(q), ks, vs, fb, p2, torch.empty(q.shape, **f32),
                           [torch.empty(ks[0].shape, **f32) for _ in range(plan.cp)],
                           [torch.empty(ks[0].shape, **f32) for _ in range(plan.cp)],
                           torch.empty((heads_q, tl), **f32))


def _gather(x_global: torch.Tensor, dst: torch.Tensor, plan: RankPlan, rank: int):
    if plan.tf[0]:
        cpattn_partition_tf(x_global, dst, plan.cu_global_dev, plan.num_seqs, plan.cp, rank, plan.tf[0], plan.tf[1])
    else:
        cpattn_partition(x_global, dst, plan.cu_global_dev, plan.num_seqs, plan.cp, rank)


def rank_step(q_g: torch.Tensor, k_g: torch.Tensor, v_g: torch.Tensor, dout_g: Optional[torch.Tensor],
              plan: RankPlan, mask_mode: int, b: StepBuffers, side: Optional[torch.cuda.Stream] = None,
              scale: float = 0.0, tf=None):
    """One rank's whole step from the global THD tensors: gathers of Q (and
    dO) and of every source rank's K/V share, cp forward steps with their LSE
    merges, then (when dout_g is given) the backward preprocess and cp
    backward steps into b.dq / b.dk / b.dv.

    With `side` (a stream of default priority) the work that the ring would
    overlap with compute runs there, ordered by events: the K/V gathers of
    steps 1.. (the ring's transfers), the dO gather, the gradient zero fills
    and the merges, which alternate between two partial buffers so that merge
    s runs beside forward step s + 1.  Every buffer sees the same kernels in
    the same order either way, so the results are bit-identical; the calling
    stream is joined with `side` before the backward and at the end.  Only
    enqueues work, so it can be captured as a graph.  tf = (B, N) gives the
    teacher-forcing mask's chunking (default: the plan's split; needed at
    cp = 1, where the plan has no split)."""
    cp, r = plan.cp, plan.rank
    tf = plan.tf if tf is None else tf
    steps = [make_step(cp, r, s, tf[0], tf[1]) for s in range(cp)]
    src = [cpattn_step_source(st) for st in steps]
    main = torch.cuda.current_stream()
    fb = b.fwd
    parts = [(fb.out_partial, fb.lse_partial), b.partial2] if side is not None else [(fb.out_partial, fb.lse_partial)]
    _gather(q_g, b.q, plan, r)
    _gather(k_g, b.ks[src[0]], plan, src[0])
    _gather(v_g, b.vs[src[0]], plan, src[0])
    fb.reset()
    ready = {}
    if side is not None:
        side.wait_stream(main)
    with torch.cuda.stream(side if side is not None else main):
        for s in range(1, cp):
            _gather(k_g, b.ks[src[s]], plan, src[s])
            _gather(v_g, b.vs[src[s]], plan, src[s])
            if side is not None:
                ready[s] = torch.cuda.Event()
                ready[s].record(side)
        if dout_g is not None:
            _gather(dout_g, b.dout, plan, r)
            for x in [b.dq] + b.dk + b.dv:
                cpattn_fill_f32(x, 0.0)
    merged = {}
    for s in range(cp):
        if s in ready:
            main.wait_event(ready[s])
        if s >= 2 and side is not None:
            main.wait_event(merged[s - 2])    # partial buffer s % 2 is free again
        op, lp = parts[s % len(parts)]
        cpattn_fwd_step(b.q, b.ks[src[s]], b.vs[src[s]], plan.cu_local_dev, plan.cu_local_dev, plan.num_seqs,
                        mask_mode, steps[s], scale, op, lp, fb.workspace)
        if side is None:
            cpattn_merge(fb.out, fb.lse, op, lp)
            continue
        done = torch.cuda.Event()
        done.record(main)
        with torch.cuda.stream(side):
            side.wait_event(done)
            cpattn_merge(fb.out, fb.lse, op, lp)
            merged[s] = torch.cuda.Event()
            merged[s].record(side)
    if side is not None:
        main.wait_stream(side)
    if dout_g is None:
        return
    cpattn_bwd_preprocess(fb.out, b.dout, b.delta)
    for s in range(cp):
        cpattn_bwd_step(b.q, b.ks[src[s]], b.vs[src[s]], b.dout, fb.lse, b.delta, plan.cu_local_dev,
                        plan.cu_local_dev, plan.num_seqs, mask_mode, steps[s], scale, b.dq, b.dk[src[s]],
                        b.dv[src[s]], fb.workspace)
