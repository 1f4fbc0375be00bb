"""Latency-constrained layer-wise N:M search.

The configuration side of "Realizable N:M Sparse Transformer Inference via
Search-Kernel Co-Design" (Sec. 3): choose one N:M pattern per layer so that
the model's predicted latency (the calibrated look-up table of ``lut.py``)
stays within a budget while the model keeps as much quality as possible; the
pages search the fragmented feasible region with a feasibility-aware
evolutionary solver.

Quality here is a proxy (the pages' objective needs trained weights and an
evaluation dataset): the fraction of each layer's weight energy sum(w^2)
that its N:M choice keeps (top-N by magnitude in every group of M), summed
over layers with optional per-layer weights.  Problem: pick c_l per layer l
to maximise sum_l score[l][c_l] subject to sum_l lat[l][c_l] <= budget -- a
multiple-choice knapsack.

Solvers:
- ``solve_exact``: dynamic programming over latency quantised to ``res`` us
  (the optimum up to that resolution; the reference for the others);
- ``solve_greedy``: start from the best-scoring choice of every layer and
  repeatedly take the downgrade with the least score lost per microsecond
  saved until the budget holds, then spend the slack on upgrades;
- ``solve_evolutionary``: the pages' three-stage heuristic with constraint
  relaxation (seeding and exploration under a relaxed budget, then
  convergence with the budget tightened to the target and a local search);
  an individual over the current budget is repaired by the greedy downgrade
  rule, so the search moves between the disconnected feasible pieces rather
  than discarding what lies between them.
"""
from __future__ import annotations

import random
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np


def retained_energy(W: np.ndarray, N: int, M: int) -> float:
    """Fraction of sum(w^2) that top-N-by-magnitude selection in every group
    of M consecutive elements along a row keeps (1.0 for N == M)."""
    w = np.asarray(W, dtype=np.float64)
    R, K = w.shape
    if K % M:
        raise ValueError("K must be a multiple of M")
    e = (w * w).reshape(R, K // M, M)
    total = e.sum()
    if total == 0 or N >= M:
        return 1.0
    kept = np.sort(e, axis=2)[:, :, M - N:].sum()
    return float(kept / total)


@dataclass
class Problem:
    """score[l][c] (higher is better) and lat[l][c] (microseconds) of choice c
    for layer l; ``budget`` in microseconds."""
    score: np.ndarray
    lat: np.ndarray
    budget: float

    def __post_init__(self):
        self.score = np.asarray(self.score, dtype=np.float64)
        self.lat = np.asarray(self.lat, dtype=np.float64)
        if self.score.shape != self.lat.shape or self.score.ndim != 2:
            raise ValueError("score and lat must both be [layers][choices]")

    @property
    def layers(self) -> int:
        return self.score.shape[0]

    def value(self, a: Sequence[int]) -> float:
        return float(self.score[np.arange(self.layers), a].sum())

    def latency(self, a: Sequence[int]) -> float:
        return float(self.lat[np.arange(self.layers), a].sum())

    def feasible(self, a: Sequence[int], budget: Optional[float] = None) -> bool:
        return self.latency(a) <= (self.budget if budget is None else budget) + 1e-9


@dataclass
class Solution:
    choice: List[int]
    value: float
    latency: float
    feasible: bool


def _solution(p: Problem, a) -> Solution:
    a = [int(x) for x in a]
    return Solution(a, p.value(a), p.latency(a), p.feasible(a))


def solve_exact(p: Problem, res: float = 0.1) -> Solution:
    """Best assignment with latencies rounded up to multiples of ``res``
    (so the returned assignment is feasible for the true latencies)."""
    L, C = p.score.shape
    q = np.ceil(p.lat / res - 1e-9).astype(np.int64)
    cap = int(np.floor(p.budget / res + 1e-9))
    NEG = -np.inf
    best = np.full(cap + 1, NEG)
    best[0] = 0.0
    arg = np.zeros((L, cap + 1), dtype=np.int8)
    for l in range(L):
        nb = np.full(cap + 1, NEG)
        for c in range(C):
            w = q[l, c]
            if w > cap:
                continue
            cand = np.full(cap + 1, NEG)
            cand[w:] = best[:cap + 1 - w] + p.score[l, c]
            better = cand > nb
            nb[better] = cand[better]
            arg[l, better] = c
        best = nb
    if not np.isfinite(best).any():
        # nothing fits: the fastest choice everywhere (infeasible)
        return _solution(p, np.argmin(p.lat, axis=1))
    used = int(np.argmax(best))
    a = [0] * L
    for l in range(L - 1, -1, -1):
        c = int(arg[l, used])
        a[l] = c
        used -= int(q[l, c])
    return _solution(p, a)


def _repair(p: Problem, a: List[int], budget: float) -> List[int]:
    """Downgrade (to a faster choice) the layer losing the least score per
    microsecond saved, until the assignment fits ``budget``."""
    a = list(a)
    idx = np.arange(p.layers)
    while p.latency(a) > budget + 1e-9:
        cur_s, cur_t = p.score[idx, a], p.lat[idx, a]
        ds = cur_s[:, None] - p.score            # score lost by switching
        dt = cur_t[:, None] - p.lat              # latency saved by switching
        ratio = np.where(dt > 1e-12, ds / np.maximum(dt, 1e-12), np.inf)
        l, c = np.unravel_index(np.argmin(ratio), ratio.shape)
        if not np.isfinite(ratio[l, c]):
            break                                 # nothing faster is left
        a[l] = int(c)
    return a


def _fill(p: Problem, a: List[int], budget: float) -> List[int]:
    """Spend remaining slack: take the upgrade with the most score gained per
    microsecond that still fits, until none fits."""
    a = list(a)
    idx = np.arange(p.layers)
    while True:
        slack = budget - p.latency(a)
        cur_s, cur_t = p.score[idx, a], p.lat[idx, a]
        gain = p.score - cur_s[:, None]
        cost = p.lat - cur_t[:, None]
        ok = (gain > 1e-12) & (cost <= slack + 1e-9)
        if not ok.any():
            return a
        ratio = np.where(ok, gain / np.maximum(cost, 1e-12), -np.inf)
        l, c = np.unravel_index(np.argmax(ratio), ratio.shape)
        a[l] = int(c)


def solve_greedy(p: Problem) -> Solution:
    a = list(np.argmax(p.score, axis=1))
    a = _repair(p, a, p.budget)
    return _solution(p, _fill(p, a, p.budget))


def _local_search(p: Problem, a: List[int], budget: float, passes: int = 3) -> List[int]:
    """Moves on a feasible assignment: set one layer, then two layers, to
    other choices, repair the rest to the budget, spend the slack; keep a
    move when the score rises.  A few passes over all such moves."""
    best = list(a)
    C = p.score.shape[1]

    def attempt(b):
        nonlocal best
        b = _fill(p, _repair(p, b, budget), budget)
        if p.latency(b) <= budget + 1e-9 and p.value(b) > p.value(best) + 1e-12:
            best = b
            return True
        return False

    for _ in range(passes):
        improved = False
        for l in range(p.layers):
            for c in range(C):
                if c != best[l]:
                    b = list(best)
                    b[l] = c
                    improved |= attempt(b)
        for l in range(p.layers):
            for m in range(l + 1, p.layers):
                for c in range(C):
                    for d in range(C):
                        if c != best[l] and d != best[m]:
                            b = list(best)
                            b[l], b[m] = c, d
                            improved |= attempt(b)
        if not improved:
            break
    return best


def solve_evolutionary(p: Problem, pop: int = 64, generations: int = 200, relax: float = 0.25,
                       mutation: float = 0.05, seed: int = 0) -> Solution:
    """Three-stage heuristic search with constraint relaxation (the pages'
    search, Sec. 3: relaxation keeps the search from converging early inside
    one piece of a fragmented feasible region):

    1. seeding under a relaxed budget (1 + relax) x target: the greedy
       assignment and random assignments, each repaired to the relaxed budget
       and its slack spent;
    2. exploration, a third of the generations, at the relaxed budget:
       crossover and mutation, every child repaired to it, so individuals
       between the target-feasible pieces survive;
    3. convergence, the rest of the generations, with the budget tightened
       linearly to the target (then held there), elitist, and a local search
       of single-layer moves on the best target-feasible individual.
    """
    rng = random.Random(seed)
    L, C = p.score.shape
    fitness = p.value
    relaxed = p.budget * (1.0 + relax)
    mutation = max(mutation, 1.0 / L)          # at least one changed layer per child on average
    g1 = max(1, generations // 3)
    g2 = max(1, generations - g1)

    def evolve(popl, bud):
        elite = popl[: max(2, pop // 8)]
        nxt = [list(a) for a in elite]
        while len(nxt) < pop:
            x, y = rng.sample(popl[: max(2, pop // 2)], 2)     # parents from the better half
            child = [x[i] if rng.random() < 0.5 else y[i] for i in range(L)]
            for i in range(L):
                if rng.random() < mutation:
                    child[i] = rng.randrange(C)
            nxt.append(_fill(p, _repair(p, child, bud), bud))
        return nxt

    # stage 1: seeds under the relaxed budget
    popl = [_fill(p, _repair(p, list(np.argmax(p.score, axis=1)), relaxed), relaxed)]
    popl += [_fill(p, _repair(p, [rng.randrange(C) for _ in range(L)], relaxed), relaxed) for _ in range(pop - 1)]
    # stage 2: exploration at the relaxed budget
    for _ in range(g1):
        popl.sort(key=fitness, reverse=True)
        popl = evolve(popl, relaxed)
    # stage 3: tighten to the target, converge, refine
    best = None
    for g in range(g2 + 1):
        bud = p.budget + (relaxed - p.budget) * max(0.0, 1.0 - g / max(1, 0.75 * g2))
        popl = [_repair(p, a, bud) for a in popl]
        popl.sort(key=fitness, reverse=True)
        for a in popl:
            if p.feasible(a) and (best is None or fitness(a) > fitness(best)):
                best = list(a)
                break
        if g == g2:
            break
        popl = evolve(popl, bud)
    if best is None:
        best = _repair(p, popl[0], p.budget)
    best = _fill(p, best, p.budget)
    if p.feasible(best):
        best = _local_search(p, best, p.budget)
    return _solution(p, best)


def brute_force(p: Problem) -> Solution:
    """Exhaustive optimum (tiny problems only; for tests)."""
    import itertools
    L, C = p.score.shape
    best = None
    for a in itertools.product(range(C), repeat=L):
        if p.feasible(a) and (best is None or p.value(a) > p.value(best)):
            best = a
    if best is None:
        best = tuple(np.argmin(p.lat, axis=1))
    return _solution(p, best)
