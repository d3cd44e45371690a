"""Pins of the Dynamic-CP planner oracle (oracle/dynamic_cp.py).

"Speeding up Variable-Length Training with Dynamic Context Parallelism and
NVIDIA Megatron Core", section A2 (Eq. 1-3, workload model, the three-stage
heuristic, the simulator) and section A7 (grid search near the knee of the
budget curve, Fig. 7).  Each pin reaches the oracle through something other
than its own formula: a linear solve of Eq. 1 and Eq. 3, closed forms of the
cp choice and of the knee, Graham's bound for the greedy stage, Eq. 1's
equal-load form, and brute force over tiny batches."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import dynamic_cp as dc


# ---- Eq. 1-3 --------------------------------------------------------------
@pytest.mark.parametrize("seed", range(6))
def test_quotas_solve_the_linear_system(seed):
    """Eq. 1 (W_1 (m_1 V + p - 1) = W_i (m_i V + p - 1)) and Eq. 3
    (sum W_i m_i = total) as an n x n linear system, solved by LAPACK."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    m = [int(x) for x in rng.integers(1, 17, n)]
    V, p = int(rng.integers(1, 5)), int(rng.integers(1, 9))
    total = int(rng.integers(1, 10**9))
    A = np.zeros((n, n))
    rhs = np.zeros(n)
    for i in range(1, n):
        A[i - 1, 0] = m[0] * V + p - 1
        A[i - 1, i] = -(m[i] * V + p - 1)
    A[n - 1, :] = m
    rhs[n - 1] = total
    want = np.linalg.solve(A, rhs)
    got = np.array([float(w) for w in dc.quotas(m, V, p, total)])
    np.testing.assert_allclose(got, want, rtol=1e-12)


def test_quotas_equal_microbatches_split_evenly():
    """Same m on every rank: every quota is total / (n m), exactly."""
    for n, m, V, p, total in [(4, 3, 2, 4, 1000), (1, 1, 1, 1, 7), (8, 16, 3, 5, 123456789)]:
        assert dc.quotas([m] * n, V, p, total) == [Fraction(total, n * m)] * n


def test_quotas_without_pipeline_give_equal_rank_work():
    """p = 1, V = 1: no bubble, so every rank's work W_i m_i is total / n."""
    m = [1, 2, 5, 7]
    W = dc.quotas(m, 1, 1, 700)
    assert [w * mi for w, mi in zip(W, m)] == [Fraction(175)] * 4


# ---- stage 1: cp size ---------------------------------------------------------
def _pow2_ceil(x):
    return 1 if x <= 1 else 2 ** math.ceil(math.log2(x))


@pytest.mark.parametrize("S,others,gpus,m,max_cp", [
    (4096, [256] * 40, 8, 2, 8), (4096, [4096], 2, 1, 4), (4096, [4096] * 3, 8, 1, 4), (10000, [100], 4, 4, 16),
    (8, [8, 8, 8, 8, 8, 8, 8], 8, 1, 8), (2048, [1024] * 6, 4, 2, 4)])
def test_cp_size_closed_form_workload(S, others, gpus, m, max_cp):
    """b = 0, no memory limit: c = 2^ceil(log2(w gpus m / total)), clipped to
    [1, max_cp].  The second and third cases sit exactly on the quota
    (w gpus m = total, and = 2 total)."""
    lengths = [S] + others
    w = [x * x for x in lengths]
    total = sum(w)
    want = min(max_cp, _pow2_ceil(Fraction(w[0] * gpus * m, total)))
    assert dc.pick_cp(S, w[0], total, gpus, m, max_cp, 10**12) == want


@pytest.mark.parametrize("S,mem,max_cp", [(1000, 1000, 8), (1001, 1000, 8), (4000, 1000, 8), (4001, 1000, 8),
                                          (4000, 999, 8), (63, 2, 32), (64, 2, 32), (65, 2, 32)])
def test_cp_size_closed_form_memory(S, mem, max_cp):
    """Quota never binds (one sample per slot budget is huge): c is the
    smallest power of two with 2 ceil(S / 2c) <= mem, i.e.
    c >= S / (2 floor(mem / 2)), or 1 when S <= mem."""
    total = 10**18
    if S <= mem:
        want = 1
    else:
        want = _pow2_ceil(Fraction(S, 2 * (mem // 2)))
    got = dc.pick_cp(S, S, total, 1, 1, max_cp, mem)
    assert got == (want if want <= max_cp else None)


# ---- knee ---------------------------------------------------------------------
@pytest.mark.parametrize("M", [4, 9, 16, 25, 40, 64, 100])
def test_knee_of_hyperbola(M):
    """y = 1/m on m = 1..M: on the normalised curve x + y is least at the
    real point m* = (M - 1) / sqrt(M) (set the derivative to zero), so the
    discrete knee is floor(m*) or ceil(m*)."""
    ms = list(range(1, M + 1))
    k = dc.knee(ms, [1.0 / m for m in ms])
    mstar = (M - 1) / math.sqrt(M)
    assert math.floor(mstar) <= k <= math.ceil(mstar)


@pytest.mark.parametrize("corner,lo,hi", [(5, 1, 20), (3, 2, 9), (12, 4, 16)])
def test_knee_of_two_segments(corner, lo, hi):
    """A curve that falls linearly to a floor and stays there: the knee is
    the corner."""
    ms = list(range(lo, hi + 1))
    ys = [float(max(corner - m, 0)) * 3.0 + 1.0 for m in ms]
    assert dc.knee(ms, ys) == corner


def test_budget_curve_floor():
    """One sample: the budget is its share at max_cp for every m (gpus >=
    max_cp), so the curve is flat and the knee is the first m."""
    ys = dc.budget_curve([5000], 8, 4, 1, 0, 2, 8)
    assert ys == [5000 * 5000 / 4] * 7
    assert dc.knee(list(range(2, 9)), ys) == 2


# ---- stage 3: Graham's bound for greedy heaviest-first ------------------------
def _opt_makespan(jobs, k):
    best = None
    for a in itertools.product(range(k), repeat=len(jobs)):
        loads = [0] * k
        for j, b in zip(jobs, a):
            loads[b] += j
        best = max(loads) if best is None else min(best, max(loads))
    return best


def _slot_loads(lengths, m, pp=2):
    """One rank, no split (max_cp = 1), w(S) = S: the plan is m microbatches."""
    bks = dc.plan_for_m(lengths, 1, 1, 10**9, 0, 1, m)
    return sorted((b.load for b in bks), reverse=True), bks


def test_graham_tight_instance():
    """Heaviest-first greedy on jobs 3,3,2,2,2 over 2 machines gives 7
    against the optimum 6: exactly Graham's worst case 4/3 - 1/(3m)
    (R. L. Graham, 1969)."""
    loads, _ = _slot_loads([3, 3, 2, 2, 2], 2)
    assert max(loads) == 7 and _opt_makespan([3, 3, 2, 2, 2], 2) == 6


@pytest.mark.parametrize("jobs,k", [([1, 1, 2], 2), ([5, 4, 3, 3, 3], 2), ([2, 2, 2, 3, 3, 3, 4], 3)])
def test_graham_bound_cases(jobs, k):
    loads, _ = _slot_loads(jobs, k)
    assert Fraction(max(loads)) <= (Fraction(4, 3) - Fraction(1, 3 * k)) * _opt_makespan(jobs, k)


@pytest.mark.parametrize("seed", range(12))
def test_graham_bound_random(seed):
    rng = np.random.default_rng(seed)
    n, k = int(rng.integers(2, 8)), int(rng.integers(2, 4))
    jobs = [int(x) for x in rng.integers(1, 30, n)]
    loads, bks = _slot_loads(jobs, k)
    opt = _opt_makespan(jobs, k)
    assert Fraction(max(loads)) <= (Fraction(4, 3) - Fraction(1, 3 * k)) * opt
    assert sorted(i for b in bks for i in b.samples) == list(range(n))


# ---- simulator: Eq. 1's equal-load form --------------------------------------
@pytest.mark.parametrize("gpus,m,V,p", [(4, 3, 2, 4), (8, 1, 1, 1), (2, 5, 3, 2), (1, 4, 1, 8)])
def test_equal_loads_match_eq1(gpus, m, V, p):
    """gpus*m equal samples, one per slot: step time = W (m V + p - 1) with
    W the per-slot share (Eq. 1's left-hand side)."""
    S = 512
    lengths = [S] * (gpus * m)
    bks = dc.plan_for_m(lengths, gpus, 1, 10**9, 1, 0, m)
    assert all(len(b.samples) == 1 for b in bks)
    assert dc.simulate(bks, gpus, m, 1, V, p) == S * S * (m * V + p - 1)


def test_single_huge_sample_takes_max_cp():
    """One sample far over the quota: cp = max_cp, and the step time is its
    share times (V + p - 1) when m = 1 and gpus = max_cp."""
    bks = dc.plan_for_m([8192], 4, 4, 10**9, 1, 0, 1)
    assert [b.cp for b in bks] == [4]
    assert dc.simulate(bks, 4, 1, 4, 2, 3) == 8192 * 8192 * (2 + 3 - 1)   # share * max_cp / cp = w


# ---- whole plans: invariants and brute force ----------------------------------
def _check_plan(lengths, bks, gpus, m, max_cp, mem, a, b):
    seen = sorted(i for bk in bks for i in bk.samples)
    assert seen == list(range(len(lengths)))
    cells = {}
    w = [dc.workload(S, a, b) for S in lengths]
    total = sum(w)
    for j, bk in enumerate(bks):
        assert bk.cp in [2 ** e for e in range(10)] and bk.cp <= max_cp
        assert bk.gpu % bk.cp == 0 and 0 <= bk.slot < m
        assert bk.tokens == sum(dc.rank_tokens(lengths[i], bk.cp) for i in bk.samples) <= mem
        assert bk.load == sum(w[i] for i in bk.samples)
        for r in range(bk.gpu, bk.gpu + bk.cp):
            assert (r, bk.slot) not in cells
            cells[(r, bk.slot)] = j
        if bk.cp > 1:
            # no over-splitting: its opening sample would not fit at cp/2
            S0, w0, h = lengths[bk.samples[0]], w[bk.samples[0]], bk.cp // 2
            assert dc.rank_tokens(S0, h) > mem or w0 * gpus * m > h * total
    assert len(cells) == gpus * m


@pytest.mark.parametrize("seed", range(10))
def test_plan_invariants(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(5, 60))
    lengths = [int(x) for x in np.minimum(rng.lognormal(6.0, 1.3, n).astype(int) + 1, 30000)]
    gpus, max_cp = [(8, 4), (4, 4), (16, 8), (2, 1), (8, 2)][seed % 5]
    a, b = (1, int(rng.integers(0, 3000)))
    mem = int(max(lengths) // max_cp + 4000)
    res = dc.plan(lengths, gpus, max_cp, 2, 2, mem, a, b, 1, 6, -1)
    assert res is not None
    _check_plan(lengths, res["buckets"], gpus, res["m"], max_cp, mem, a, b)
    assert res["time"] == min(t for t in res["times"].values() if t is not None)


def _time_of(cells_of, lengths, gpus, m, V, p):
    """Step time of an assignment sample -> cell (rank * m + slot), by the
    simulator's rule, written out independently of the oracle."""
    cell = [[0] * m for _ in range(gpus)]
    for S, c in zip(lengths, cells_of):
        cell[c // m][c % m] += S
    return max(V * sum(cell[r]) + (p - 1) * max(cell[r]) for r in range(gpus))


@pytest.mark.parametrize("seed", range(8))
def test_brute_force_tiny_batches(seed):
    """Tiny batches, w(S) = S, one cp size: the brute-force optimum over all
    (gpus*m)^n assignments is a lower bound of the plan's step time, and the
    oracle's simulator agrees with an independent evaluation of its plan."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(2, 7))
    lengths = [int(x) for x in rng.integers(1, 40, n)]
    gpus, m, V, p = 2, int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(1, 4))
    opt = min(_time_of(a, lengths, gpus, m, V, p) for a in itertools.product(range(gpus * m), repeat=n))
    bks = dc.plan_for_m(lengths, gpus, 1, 10**9, 0, 1, m)
    t = dc.simulate(bks, gpus, m, 1, V, p)
    where = [0] * n
    for bk in bks:
        for i in bk.samples:
            where[i] = bk.gpu * m + bk.slot
    assert t == _time_of(where, lengths, gpus, m, V, p)
    assert t >= opt


def test_infeasible_when_sample_exceeds_memory_at_max_cp():
    assert dc.plan([100000, 10], 4, 4, 1, 1, 1000, 1, 0, 1, 4, -1) is None


# ---- planted mistakes ------------------------------------------------------------
def test_planted_eq1_sign_is_caught(monkeypatch):
    def bad(m, V, p, total):
        inv = [Fraction(mi, mi * V - p + 1) for mi in m]
        K = Fraction(total) / sum(inv)
        return [K / (mi * V - p + 1) for mi in m]
    monkeypatch.setattr(dc, "quotas", bad)
    with pytest.raises(AssertionError):
        for seed in range(6):
            test_quotas_solve_the_linear_system(seed)


def test_planted_ascending_greedy_is_caught(monkeypatch):
    """Stage 3 taking the lightest sample first breaks Graham's bound on
    jobs 1,1,2 over 2 slots (3 against the optimum 2)."""
    monkeypatch.setattr(dc, "stage3_order", lambda items, w: sorted(items, key=lambda i: (w[i], i)))
    with pytest.raises(AssertionError):
        test_graham_bound_cases([1, 1, 2], 2)


def test_planted_knee_argmax_is_caught(monkeypatch):
    def farthest_above(ms, ys):
        vals = [float(mi - ms[0]) / float(ms[-1] - ms[0]) + (yi - ys[-1]) / (ys[0] - ys[-1])
                for mi, yi in zip(ms, ys)]
        return ms[int(np.argmax(vals))]
    monkeypatch.setattr(dc, "knee", farthest_above)
    with pytest.raises(AssertionError):
        test_knee_of_hyperbola(16)


def test_planted_cp_off_by_one_is_caught(monkeypatch):
    """A strict quota test (< instead of <=) moves samples that sit exactly
    on the quota to the next cp size."""
    orig = dc.pick_cp

    def strict(S, w, total, gpus, m, max_cp, mem):
        c = 1
        while True:
            if dc.rank_tokens(S, c) <= mem and (w * gpus * m < c * total or c == max_cp):
                return c
            if c == max_cp:
                return None
            c *= 2
    monkeypatch.setattr(dc, "pick_cp", strict)
    with pytest.raises(AssertionError):
        test_cp_size_closed_form_workload(4096, [4096], 2, 1, 4)
    with pytest.raises(AssertionError):
        test_cp_size_closed_form_workload(4096, [4096] * 3, 8, 1, 4)
    assert orig is not None
