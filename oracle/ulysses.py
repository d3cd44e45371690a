"""Ulysses sequence-to-head exchange on one device (oracle; test infrastructure only).

"Scaling Video Training with Parallelism", section on the SP landscape
(DeepSpeed-Ulysses paragraph): Ulysses shards the input along the sequence
and uses an all-to-all around attention, which works when the head count
divides by the group size; USP / LoongTrain combine it with the ring as a 2D
mesh.  With every shard resident on one device, the all-to-all that gives
group member g all tokens of its head group is a gather: the rows of every
shard, in shard order, restricted to heads [g*Hg, (g+1)*Hg) with
Hg = H / n_groups.  The reverse exchange after attention scatters those
rows back into the shards.  Reading taken where the pages are silent: shards
are contiguous token ranges of the packed THD batch, in rank order.
"""
import numpy as np


def seq_to_head(shards, group, n_groups):
    """[sum of shard tokens, H/n_groups, d]: head group `group` of every shard."""
    H = shards[0].shape[1]
    if H % n_groups:
        raise ValueError(f"{H} heads do not split into {n_groups} groups")
    hg = H // n_groups
    return np.concatenate([np.asarray(s)[:, group * hg:(group + 1) * hg] for s in shards], axis=0)


def head_to_seq(x, group, n_groups, shards):
    """Writes head group `group` of the gathered tensor x back into copies of
    the shards; returns the updated shards."""
    out = [np.array(s, copy=True) for s in shards]
    hg = out[0].shape[1] // n_groups
    row = 0
    for s in out:
        s[:, group * hg:(group + 1) * hg] = x[row:row + len(s)]
        row += len(s)
    return out


def contiguous_shards(x_global, n_shards):
    """Equal contiguous token shards of a global THD tensor (rank order)."""
    x_global = np.asarray(x_global)
    t = x_global.shape[0]
    if t % n_shards:
        raise ValueError(f"{t} tokens do not split into {n_shards} shards")
    n = t // n_shards
    return [x_global[i * n:(i + 1) * n] for i in range(n_shards)]
