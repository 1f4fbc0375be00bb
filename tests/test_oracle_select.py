"""Pins of the oracle's kept-set selection and compression (CPU only).

The selection is checked against an independent characterisation: among all
C(M, N) subsets of a group, the kept set maximises the exact sum of |w|, and
among maximisers it is the lexicographically smallest position tuple.  That is
the same set as "top N by |w|, ties to the lower position" (the lowest-position
choice among boundary ties is the lexicographic minimum), but it is computed
by enumeration with exact rational arithmetic, so a wrong sort key, direction
or tie rule in the oracle fails here.
"""
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest

import nm_inputs
import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _mag_exact(a, dt):
    """Exact rational |w| of every element."""
    f = oracle.to_f64(a, dt)
    return [[Fraction(abs(float(v))) for v in row] for row in f]


def brute_keep(row_mags, N, M):
    """Kept positions per group by subset enumeration (max sum, lexicographic min)."""
    out = []
    for g in range(len(row_mags) // M):
        grp = row_mags[g * M:(g + 1) * M]
        best, best_set = None, None
        for sub in itertools.combinations(range(M), N):   # lexicographic order
            s = sum(grp[i] for i in sub)
            if best is None or s > best:
                best, best_set = s, sub
        out.append(best_set)
    return out


def _check_against_brute(W, N, M, dt):
    vals, idx = oracle.compress(W, N, M, dt)
    mags = _mag_exact(W, dt)
    for r in range(W.shape[0]):
        want = brute_keep(mags[r], N, M)
        for g, sub in enumerate(want):
            assert tuple(int(i) for i in idx[r, g]) == sub, (r, g, W[r, g * M:(g + 1) * M])
            for j, i in enumerate(sub):
                assert vals[r, g, j] == W[r, g * M + i]


@pytest.mark.parametrize("N", [1, 2, 3, 4])
def test_exhaustive_m4_small_ints(N):
    # every group in {-2..2}^4: 625 groups with heavy magnitude ties
    W = np.array(list(itertools.product(range(-2, 3), repeat=4)), dtype=np.int8)
    _check_against_brute(W, N, 4, "i8")


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7, 8])
def test_exhaustive_m8_ternary(N):
    # every group in {-1,0,1}^8: 6561 groups
    W = np.array(list(itertools.product((-1, 0, 1), repeat=8)), dtype=np.int8)
    _check_against_brute(W, N, 8, "i8")


@pytest.mark.parametrize("M", [4, 8])
def test_random_int8_with_extremes(M):
    r = nm_inputs.rng(1, "select", M)
    W = r.integers(-128, 128, size=(64, 8 * M)).astype(np.int8)
    W[0, :M] = -128
    W[1, :M] = [127, -128] * (M // 2)
    for N in range(1, M + 1):
        _check_against_brute(W, N, M, "i8")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("M", [4, 8])
def test_random_fp(dt, M):
    W = nm_inputs.normal((48, 4 * M), 0.02, dt, 2, "select-fp", M)
    if dt == "f16":
        W[0, :4] = np.array([0.0, -0.0, 0.0, -0.0], np.float16)  # signed zeros tie
        W[1, :4] = np.array([1e-7, -1e-7, 6e-8, 65504.0], np.float16)  # subnormals, max
    for N in range(1, M + 1):
        _check_against_brute(W, N, M, dt)


def _parse_vals(tokens, dt):
    """Row values of a golden line: decimals, 'inf' / '-inf', or 0x.... raw
    16-bit patterns (fp16 / bf16)."""
    if dt == "i8":
        return np.array([int(t) for t in tokens], dtype=np.int8)
    bits = np.empty(len(tokens), np.uint16)
    for i, t in enumerate(tokens):
        if t.lower().startswith("0x"):
            bits[i] = int(t, 16)
        elif dt == "f16":
            bits[i] = np.array([float(t)], np.float16).view(np.uint16)[0]
        else:
            bits[i] = oracle.f64_to_bf16_bits(np.array([float(t)]))[0]
    return bits.view(np.float16) if dt == "f16" else bits


def test_golden_hand_examples(golden_dir):
    n = 0
    for line in open(os.path.join(golden_dir, "select_ties.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        head, row, want = [p.strip() for p in line.split("|")]
        dt, N, M = head.split()
        N, M = int(N), int(M)
        W = _parse_vals(row.split(), dt)[None, :]
        _, idx = oracle.compress(W, N, M, dt)
        want_sets = [tuple(int(t) for t in g.split()) for g in want.split(";")]
        got = [tuple(int(i) for i in idx[0, g]) for g in range(idx.shape[1])]
        assert got == want_sets, line
        n += 1
    assert n >= 10


@pytest.mark.parametrize("N,M", [(1, 4), (2, 4), (3, 4), (4, 4), (2, 8), (4, 8), (8, 8)])
def test_roundtrip_and_counts(N, M):
    W = nm_inputs.uniform_int8((40, 16 * M), 3, "roundtrip", N, M)
    vals, idx = oracle.compress(W, N, M, "i8")
    Wm = oracle.decompress(vals, idx, 40, 16 * M, N, M, "i8")
    # exactly N kept slots per group, ascending distinct positions
    assert np.all(np.diff(idx.astype(int), axis=2) > 0) if N > 1 else True
    assert idx.max() < M
    # decompress(compress(W)) == mask (.) W with the brute-force mask
    mags = _mag_exact(W, "i8")
    mask = np.zeros_like(W, dtype=bool)
    for r in range(W.shape[0]):
        for g, sub in enumerate(brute_keep(mags[r], N, M)):
            for i in sub:
                mask[r, g * M + i] = True
    assert np.array_equal(Wm, np.where(mask, W, 0).astype(np.int8))
    # nonzeros per group <= N (kept zeros are still kept slots)
    nnz = (Wm.reshape(40, -1, M) != 0).sum(axis=2)
    assert nnz.max() <= N
    assert mask.reshape(40, -1, M).sum(axis=2).min() == N


def test_rejects_bad_arguments():
    W = np.zeros((2, 8), np.int8)
    with pytest.raises(ValueError):
        oracle.compress(W, 0, 4, "i8")
    with pytest.raises(ValueError):
        oracle.compress(W, 5, 4, "i8")
    with pytest.raises(ValueError):
        oracle.compress(np.zeros((2, 6), np.int8), 2, 4, "i8")
