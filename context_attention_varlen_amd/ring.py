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
