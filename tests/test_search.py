"""Layer-wise N:M search under a latency budget: the proxy objective, the
exact solver against brute force, the heuristics against the exact one."""
import numpy as np
import pytest

from semi_structured_sparse_nm_amd.search import (Problem, brute_force, retained_energy, solve_evolutionary,
                                                  solve_exact, solve_greedy)


def test_retained_energy_hand_cases():
    W = np.array([[1.0, -2.0, 3.0, -4.0, 0.0, 0.0, 0.0, 5.0]])
    # 2:4 keeps {3, -4} and {0 (any), 5}: (9 + 16 + 25) / (1 + 4 + 9 + 16 + 25)
    assert retained_energy(W, 2, 4) == pytest.approx(50 / 55)
    assert retained_energy(W, 1, 4) == pytest.approx(41 / 55)
    assert retained_energy(W, 4, 8) == pytest.approx((25 + 16 + 9 + 4) / 55)
    assert retained_energy(W, 4, 4) == 1.0 and retained_energy(W, 8, 8) == 1.0
    assert retained_energy(np.zeros((2, 8)), 1, 4) == 1.0
    with pytest.raises(ValueError):
        retained_energy(np.ones((1, 6)), 1, 4)


def test_retained_energy_orders_the_patterns():
    W = np.random.default_rng(0).standard_normal((64, 256))
    e = {nm: retained_energy(W, *nm) for nm in ((1, 4), (2, 8), (2, 4), (4, 8), (8, 8))}
    assert e[(1, 4)] < e[(2, 8)] < e[(2, 4)] < e[(4, 8)] < e[(8, 8)] == 1.0


def _random_problem(rng, L, C, integer=True, slack=0.6):
    score = rng.random((L, C))
    lat = rng.integers(1, 20, (L, C)).astype(float) if integer else rng.random((L, C)) * 20
    lo, hi = lat.min(axis=1).sum(), lat.max(axis=1).sum()
    return Problem(score, lat, lo + slack * (hi - lo))


@pytest.mark.parametrize("seed", range(12))
def test_exact_equals_brute_force(seed):
    rng = np.random.default_rng(seed)
    p = _random_problem(rng, L=6, C=3, slack=rng.random())
    ex, bf = solve_exact(p, res=1.0), brute_force(p)
    assert ex.feasible and bf.feasible
    assert ex.value == pytest.approx(bf.value)


def test_exact_respects_the_budget_with_fractional_latencies():
    rng = np.random.default_rng(3)
    for _ in range(5):
        p = _random_problem(rng, L=10, C=4, integer=False)
        s = solve_exact(p, res=0.05)
        assert s.feasible and s.latency <= p.budget + 1e-9


@pytest.mark.parametrize("seed", range(6))
def test_heuristics_feasible_and_close_to_optimal(seed):
    rng = np.random.default_rng(100 + seed)
    p = _random_problem(rng, L=24, C=4, slack=0.3 + 0.5 * rng.random())
    ex = solve_exact(p, res=1.0)
    gr = solve_greedy(p)
    ev = solve_evolutionary(p, pop=48, generations=120, seed=seed)
    for s in (gr, ev):
        assert s.feasible
        assert s.value <= ex.value + 1e-9
    assert ev.value >= 0.99 * ex.value
    assert gr.value >= 0.9 * ex.value


def test_unreachable_budget_returns_the_fastest_assignment():
    p = Problem([[1.0, 2.0], [1.0, 2.0]], [[5.0, 9.0], [5.0, 9.0]], budget=4.0)
    for s in (solve_exact(p, res=1.0), solve_greedy(p), solve_evolutionary(p, pop=8, generations=5)):
        assert not s.feasible and s.choice == [0, 0]


def test_generous_budget_takes_every_best_choice():
    rng = np.random.default_rng(7)
    p = _random_problem(rng, L=8, C=4, slack=1.0)
    best = list(np.argmax(p.score, axis=1))
    for s in (solve_exact(p, res=1.0), solve_greedy(p), solve_evolutionary(p, pop=16, generations=20)):
        assert s.choice == best


@pytest.mark.parametrize("seed", range(5))
def test_three_stage_search_finds_the_optimum_of_small_problems(seed):
    """The staged search (relaxed seeding and exploration, tightening,
    local search) reaches the exhaustive optimum on small problems and its
    answer always fits the target budget."""
    rng = np.random.default_rng(300 + seed)
    p = _random_problem(rng, L=7, C=4, slack=0.2 + 0.6 * rng.random())
    bf = brute_force(p)
    ev = solve_evolutionary(p, pop=24, generations=30, seed=seed)
    assert ev.feasible
    assert ev.value == pytest.approx(bf.value, abs=1e-9)
