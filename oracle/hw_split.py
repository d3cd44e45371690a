"""Two-dimensional height/width token split over cp ranks (oracle; test infrastructure only).

LongCat-Video context-parallel page (split_tensor_in_cp_2d / get_optimal_split):
video latent tokens are split along height and then width, and rank cp_rank
takes its piece; the split factors are chosen automatically as the split
closest to square, to balance the ranks.  The page gives no formula.
Readings taken here:
  * a sample's tokens are frames x H x W in row-major order, token
    t = (f*H + h)*W + w;
  * cp = split_h * split_w with split_h dividing H and split_w dividing W;
    among those, the split whose per-rank tile (H/split_h) x (W/split_w) is
    closest to square (smallest |H/split_h - W/split_w|), ties to the smaller
    split_h;
  * rank r takes grid cell (r // split_w, r % split_w) (height pieces outer,
    width pieces inner) in every frame; its local rows are, frame by frame,
    the cell's rows top to bottom, each row left to right.
Attention over these shares is order-free only under the BIDIR mask (full
spatio-temporal attention), which is what the split is used with here.
"""
import numpy as np


def optimal_split(H, W, cp):
    """(split_h, split_w) by exhaustive search over the factor pairs of cp."""
    best = None
    for sh in range(1, cp + 1):
        if cp % sh:
            continue
        sw = cp // sh
        if H % sh or W % sw:
            continue
        key = (abs(H / sh - W / sw), sh)
        if best is None or key < best[0]:
            best = (key, (sh, sw))
    if best is None:
        raise ValueError(f"no even split of {H}x{W} into {cp} tiles")
    return best[1]


def local_rows(cu_seqlens, frames, H, W, split, r):
    """Index plan of rank r: (cu_local int32, l2g int64, pos int64, seq int64)."""
    sh, sw = split
    th, tw = H // sh, W // sw
    rh, rw = r // sw, r % sw
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    l2g, pos, seq = [], [], []
    cu_local = [0]
    for b in range(len(cu) - 1):
        start, length = int(cu[b]), int(cu[b + 1] - cu[b])
        if length != frames * H * W:
            raise ValueError(f"sequence {b} has {length} tokens, not {frames}x{H}x{W}")
        p = []
        for f in range(frames):
            for h in range(rh * th, (rh + 1) * th):
                for w in range(rw * tw, (rw + 1) * tw):
                    p.append((f * H + h) * W + w)
        p = np.asarray(p, dtype=np.int64)
        pos.append(p)
        l2g.append(start + p)
        seq.append(np.full(len(p), b, dtype=np.int64))
        cu_local.append(cu_local[-1] + len(p))
    cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int64)  # noqa: E731
    return np.asarray(cu_local, np.int32), cat(l2g), cat(pos), cat(seq)
