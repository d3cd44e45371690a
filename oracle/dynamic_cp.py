"""Dynamic-CP microbatch planner (oracle; test infrastructure only).

"Speeding up Variable-Length Training with Dynamic Context Parallelism and
NVIDIA Megatron Core", section A2 (data scheduling model, Eq. 1-3) and
section A7 (zero-overhead runtime, Fig. 7).  The page describes, without
code: a workload model (time grows as S^2 with the sample length, activation
memory as S); per-microbatch workload quotas from Eq. 1-3; a heuristic that
first works on workload (a sample above the quota gets a larger power-of-two
cp size), then on memory (the buckets are topped up with the samples of least
compute), then hands the remaining samples, heaviest first, to the
microbatches; a simulator that scores each candidate under the pipeline
schedule and keeps the fastest plan that fits in memory; and a grid search
over the number of microbatches per rank (the same for all ranks), from PP
up to a small multiple of it, kept near the knee of the budget curve.

The page fixes none of the constants or tie-breaks.  Readings taken here
(each also listed with the design notes of the library):

  * pool: `gpus` ranks share the data- and context-parallel work of one
    pipeline stage; cp groups are aligned blocks of a power-of-two size
    c <= max_cp (max_cp divides gpus); every rank runs m microbatch slots,
    and a microbatch with cp size c fills one slot on each rank of its group;
  * workload w(S) = a*S^2 + b*S (integers a, b >= 0, not both 0);
    per-rank share of a sample under cp size c is w(S)/c; per-rank tokens
    are S for c = 1, else S rounded up to a multiple of 2c, over c (the
    zigzag split needs 2c equal chunks);
  * quota: Eq. 1-3 with every rank at m microbatches gives the same
    per-slot quota W = total / (gpus * m) on every rank;
  * stage 1 (workload): cp(S) = smallest power of two c that fits the
    memory cap and has w(S)/c <= W (or c = max_cp); each sample with
    cp(S) > 1 opens its own microbatch;
  * stage 2 (memory): those microbatches, heaviest first, are topped up with
    the cp = 1 samples of least workload while both quota and cap hold;
  * stage 3: the remaining samples, heaviest first, go to the cp = 1
    microbatch of least workload that still has memory for them; there are
    exactly gpus*m - (sum of the split microbatches' cp sizes) of those, so
    the slot grid is full;
  * placement: split microbatches (largest cp first) take the free aligned
    group of least current load; cp = 1 microbatches (heaviest first) take
    a free slot on the least-loaded rank;
  * simulator: rank time = V * (sum of its slot loads) + (p - 1) * (its
    largest slot load), which is Eq. 1's W * (m V + p - 1) when the loads
    are equal; the step time is the slowest rank's;
  * knee: budget(m) = max(total / (gpus m), max_S w(S) / max_cp) over the
    sweep range; the knee is the point farthest below the chord joining the
    first and last points of the normalised curve (the "Kneedle" rule of
    Satopaa et al., 2011), computed in IEEE double in the order written
    below; the search keeps m within `radius` of it (radius < 0: all m);
  * choice: least step time, ties to the smaller m.

All decisions compare exact integers (Python ints), except the knee, which
compares doubles.  Ties break on the lower index everywhere.
"""
from fractions import Fraction


def workload(S, a, b):
    """Modelled time of one sample of S tokens: compute grows as S^2
    (attention), the linear part as S (section A2, data scheduling model)."""
    return a * S * S + b * S


def rank_tokens(S, c):
    """Tokens one rank of a size-c cp group holds of a sample of S tokens
    (activation memory grows as S, section A2)."""
    if c == 1:
        return S
    chunk = -(-S // (2 * c))          # ceil: zigzag needs 2c equal chunks
    return 2 * chunk


def quotas(m, V, p, total):
    """Eq. 1-3 of section A2: per-microbatch workload quota W_i of every data
    parallel rank i, given its microbatch count m_i, V virtual stages, p
    pipeline stages and the batch's total workload.

    Eq. 1 makes W_i * (m_i V + p - 1) the same constant K on every rank;
    Eq. 3 fixes K through sum_i W_i m_i = total.  Exact fractions."""
    inv = [Fraction(mi, mi * V + p - 1) for mi in m]
    K = Fraction(total) / sum(inv)
    return [K / (mi * V + p - 1) for mi in m]


def pick_cp(S, w, total, gpus, m, max_cp, mem):
    """Stage 1: smallest power-of-two cp size whose per-rank share of the
    sample fits the memory cap and the per-slot quota total/(gpus*m)
    (max_cp is taken when no size meets the quota).  None if even max_cp
    does not fit the cap."""
    c = 1
    while True:
        fits_mem = rank_tokens(S, c) <= mem
        fits_quota = w * gpus * m <= c * total
        if fits_mem and (fits_quota or c == max_cp):
            return c
        if c == max_cp:
            return None
        c *= 2


class Bucket:
    """One microbatch: its cp size and samples; load = sum of w(S)."""

    def __init__(self, cp):
        self.cp = cp
        self.samples = []
        self.load = 0
        self.tokens = 0           # per rank
        self.slot = -1
        self.gpu = -1             # first rank of its group

    def add(self, i, S, w):
        self.samples.append(i)
        self.load += w
        self.tokens += rank_tokens(S, self.cp)


def stage3_order(items, w):
    """Stage 3 hands out the remaining samples heaviest first."""
    return sorted(items, key=lambda i: (-w[i], i))


def plan_for_m(lengths, gpus, max_cp, mem, a, b, m):
    """Stages 1-3 and placement for m slots per rank.  Returns the list of
    buckets (split ones first, then cp = 1 ones) or None if infeasible."""
    n = len(lengths)
    w = [workload(S, a, b) for S in lengths]
    total = sum(w)
    cps = []
    for i in range(n):
        c = pick_cp(lengths[i], w[i], total, gpus, m, max_cp, mem)
        if c is None:
            return None
        cps.append(c)
    # stage 1: every sample that needs cp > 1 opens a microbatch, heaviest first
    heavy = sorted((i for i in range(n) if cps[i] > 1), key=lambda i: (-w[i], i))
    buckets = []
    for i in heavy:
        bk = Bucket(cps[i])
        bk.add(i, lengths[i], w[i])
        buckets.append(bk)
    # stage 2: top up with the lightest remaining samples (memory-first)
    light = sorted((i for i in range(n) if cps[i] == 1), key=lambda i: (w[i], i))
    for bk in buckets:
        while light:
            i = light[0]
            if (bk.load + w[i]) * gpus * m <= bk.cp * total and \
                    bk.tokens + rank_tokens(lengths[i], bk.cp) <= mem:
                bk.add(i, lengths[i], w[i])
                light.pop(0)
            else:
                break
    # stage 3: the rest, heaviest first, to the least-loaded cp = 1 microbatch
    ones = gpus * m - sum(bk.cp for bk in buckets)
    if ones < 0:
        return None
    small = [Bucket(1) for _ in range(ones)]
    for i in stage3_order(light, w):
        best = None
        for j, bk in enumerate(small):
            if bk.tokens + lengths[i] <= mem and (best is None or bk.load < small[best].load):
                best = j
        if best is None:
            return None
        small[best].add(i, lengths[i], w[i])
    if not place(buckets, small, gpus, m, max_cp):
        return None
    return buckets + small


def place(split, ones, gpus, m, max_cp):
    """Put every microbatch on the slot grid (gpus ranks x m slots).  Rank
    load counts each microbatch as load * max_cp / cp (per-rank share in
    units of 1/max_cp)."""
    free = [[True] * gpus for _ in range(m)]
    load = [0] * gpus
    order = sorted(range(len(split)), key=lambda j: (-split[j].cp, -split[j].load, split[j].samples[0]))
    for j in order:
        bk = split[j]
        c = bk.cp
        best = None
        for k in range(m):
            for g in range(gpus // c):
                ranks = range(g * c, (g + 1) * c)
                if all(free[k][r] for r in ranks):
                    key = (max(load[r] for r in ranks), k, g)
                    if best is None or key < best[0]:
                        best = (key, k, g)
        if best is None:
            return False
        _, k, g = best
        bk.slot, bk.gpu = k, g * c
        for r in range(g * c, (g + 1) * c):
            free[k][r] = False
            load[r] += bk.load * (max_cp // c)
    for j in sorted(range(len(ones)), key=lambda j: (-ones[j].load, j)):
        bk = ones[j]
        best = None
        for r in range(gpus):
            k = next((k for k in range(m) if free[k][r]), None)
            if k is not None and (best is None or load[r] < load[best[0]]):
                best = (r, k)
        r, k = best
        bk.slot, bk.gpu = k, r
        free[k][r] = False
        load[r] += bk.load * max_cp
    return True


def simulate(buckets, gpus, m, max_cp, V, p):
    """Step time in units of 1/max_cp of the workload unit: every rank's
    time is V * (sum of its slot loads) + (p - 1) * (largest slot load)
    (Eq. 1's W (m V + p - 1) for equal loads); the step waits for the
    slowest rank (section A2, simulator)."""
    cell = [[0] * m for _ in range(gpus)]
    for bk in buckets:
        for r in range(bk.gpu, bk.gpu + bk.cp):
            cell[r][bk.slot] = bk.load * (max_cp // bk.cp)
    return max(V * sum(cell[r]) + (p - 1) * max(cell[r]) for r in range(gpus))


def budget_curve(lengths, gpus, max_cp, a, b, m_min, m_max):
    """Fig. 7's per-microbatch workload budget over m, in IEEE double: the
    quota total/(gpus m), floored by the largest sample's share at max_cp."""
    w = [workload(S, a, b) for S in lengths]
    total, wmax = sum(w), max(w)
    floor_ = float(wmax) / float(max_cp)
    return [max(float(total) / float(gpus * m), floor_) for m in range(m_min, m_max + 1)]


def knee(ms, ys):
    """Point of a decreasing curve farthest below the chord joining its ends,
    after scaling both axes to [0, 1] (Kneedle): the least x + y.  IEEE
    double, ties to the first point."""
    if len(ms) == 1 or ys[0] == ys[-1]:
        return ms[0]
    best, best_v = ms[0], None
    for mi, yi in zip(ms, ys):
        x = float(mi - ms[0]) / float(ms[-1] - ms[0])
        y = (yi - ys[-1]) / (ys[0] - ys[-1])
        v = x + y
        if best_v is None or v < best_v:
            best, best_v = mi, v
    return best


def plan(lengths, gpus, max_cp, pp, vpp, mem, a, b, m_min, m_max, radius):
    """Whole planner (section A7: grid search over the common microbatch
    count near the knee).  Returns a dict, or None if no m is feasible:
      m, time (step time x max_cp, exact int), buckets (list of Bucket),
      times {m: time or None} for every m searched, knee."""
    ms = list(range(m_min, m_max + 1))
    kn = knee(ms, budget_curve(lengths, gpus, max_cp, a, b, m_min, m_max))
    search = ms if radius < 0 else [m for m in ms if abs(m - kn) <= radius]
    best, times = None, {}
    for m in search:
        bks = plan_for_m(lengths, gpus, max_cp, mem, a, b, m)
        t = None if bks is None else simulate(bks, gpus, m, max_cp, vpp, pp)
        times[m] = t
        if t is not None and (best is None or t < best["time"]):
            best = {"m": m, "time": t, "buckets": bks}
    if best is None:
        return None
    best["times"] = times
    best["knee"] = kn
    return best
