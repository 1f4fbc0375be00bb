"""Pins of the oracle's product and epilogue (CPU only).

 - O1 (decompress + naive loop) == O2 (direct compressed loop), bitwise.
 - N == M reduces to a dense product: equal to numpy's int64 / fp64 matmul.
 - Tiny random cases against a pure-Python sum over the brute-force mask.
 - Identity and one-hot activations return mask (.) W column by column.
 - Closed-form row checksums and linearity at larger sizes.
 - The requantising epilogue against hand-computed cases.
"""
import itertools
import os

import numpy as np
import pytest

import nm_inputs
import oracle
from tests.test_oracle_select import _mag_exact, brute_keep


def _wx(dt, R, K, T, seed, tag):
    if dt == "i8":
        return (nm_inputs.uniform_int8((R, K), seed, tag, "W"),
                nm_inputs.uniform_int8((K, T), seed, tag, "X"))
    return (nm_inputs.normal((R, K), 0.02, dt, seed, tag, "W"),
            nm_inputs.normal((K, T), 1.0, dt, seed, tag, "X"))


@pytest.mark.parametrize("dt", ["i8", "f16", "bf16"])
@pytest.mark.parametrize("N,M", [(1, 4), (2, 4), (4, 8), (2, 8), (8, 8)])
def test_o1_equals_o2_bitwise(dt, N, M):
    R, K, T = 23, 6 * M, 19
    W, X = _wx(dt, R, K, T, 5, f"o1o2-{N}-{M}")
    vals, idx = oracle.compress(W, N, M, dt)
    Wm = oracle.decompress(vals, idx, R, K, N, M, dt)
    a1 = oracle.spmm_dense(Wm, X, dt)
    a2 = oracle.spmm_direct(vals, idx, X, R, K, N, M, dt)
    assert np.array_equal(a1, a2)
    # a row subset returns the same rows
    rows = np.array([22, 0, 7], np.int64)
    a3 = oracle.spmm_direct(vals, idx, X, R, K, N, M, dt, rows=rows)
    assert np.array_equal(a3, a2[rows])


@pytest.mark.parametrize("M", [4, 8])
def test_dense_special_case_int(M):
    # N == M keeps everything: the product is numpy's exact int64 matmul
    R, K, T = 37, 12 * M, 29
    W, X = _wx("i8", R, K, T, 6, f"dense-{M}")
    vals, idx = oracle.compress(W, M, M, "i8")
    acc = oracle.spmm_direct(vals, idx, X, R, K, M, M, "i8")
    assert np.array_equal(acc, W.astype(np.int64) @ X.astype(np.int64))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_dense_special_case_fp(dt):
    R, K, T = 31, 64, 17
    W, X = _wx(dt, R, K, T, 7, "dense-fp")
    vals, idx = oracle.compress(W, 4, 4, dt)
    acc = oracle.spmm_direct(vals, idx, X, R, K, 4, 4, dt)
    ref = oracle.to_f64(W, dt) @ oracle.to_f64(X, dt)
    scale = np.abs(oracle.to_f64(W, dt)) @ np.abs(oracle.to_f64(X, dt))
    assert np.all(np.abs(acc - ref) <= 1e-13 * scale + 1e-300)


def test_tiny_bruteforce_python():
    r = nm_inputs.rng(8, "tiny")
    for case in range(60):
        M = [4, 8][case % 2]
        N = int(r.integers(1, M + 1))
        R = int(r.integers(1, 9))
        K = M * int(r.integers(1, 3))
        T = int(r.integers(1, 9))
        W = r.integers(-128, 128, size=(R, K)).astype(np.int8)
        X = r.integers(-128, 128, size=(K, T)).astype(np.int8)
        acc = oracle.reference(W, X, N, M, "i8", "i32")
        mags = _mag_exact(W, "i8")
        for i in range(R):
            keep = brute_keep(mags[i], N, M)
            ks = [g * M + j for g, sub in enumerate(keep) for j in sub]
            for t in range(T):
                want = sum(int(W[i, k]) * int(X[k, t]) for k in ks)
                assert acc[i, t] == want, (case, i, t)


@pytest.mark.parametrize("dt", ["i8", "f16", "bf16"])
@pytest.mark.parametrize("N,M", [(2, 4), (1, 4), (4, 8), (8, 8)])
def test_identity_activation_returns_masked_weights(dt, N, M):
    R, K = 20, 4 * M
    W, _ = _wx(dt, R, K, 1, 9, "ident")
    one = {"i8": np.int8(1), "f16": np.float16(1.0), "bf16": np.uint16(0x3F80)}[dt]
    X = np.zeros((K, K), dtype=W.dtype)
    np.fill_diagonal(X, one)
    vals, idx = oracle.compress(W, N, M, dt)
    Wm = oracle.decompress(vals, idx, R, K, N, M, dt)
    acc = oracle.spmm_direct(vals, idx, X, R, K, N, M, dt)
    assert np.array_equal(acc, oracle.to_f64(Wm, dt).astype(acc.dtype))


@pytest.mark.parametrize("N,M", [(2, 4), (3, 8)])
def test_one_hot_activation(N, M):
    R, K, T = 16, 2 * M, 5
    W, _ = _wx("i8", R, K, T, 10, "onehot")
    vals, idx = oracle.compress(W, N, M, "i8")
    Wm = oracle.decompress(vals, idx, R, K, N, M, "i8")
    for k0 in range(M):            # every position of one full group
        for t0 in (0, T - 1):
            X = np.zeros((K, T), np.int8)
            X[M + k0, t0] = 1
            acc = oracle.spmm_direct(vals, idx, X, R, K, N, M, "i8")
            want = np.zeros((R, T), np.int64)
            want[:, t0] = Wm[:, M + k0]
            assert np.array_equal(acc, want)


@pytest.mark.parametrize("N,M", [(2, 4), (4, 8)])
def test_checksum_and_linearity(N, M):
    R, K, T = 96, 192, 211
    W, X1 = _wx("i8", R, K, T, 11, "cks")
    X2 = nm_inputs.uniform_int8((K, T), 11, "cks", "X2", lo=-60, hi=60)
    X1 = np.clip(X1, -60, 60).astype(np.int8)
    vals, idx = oracle.compress(W, N, M, "i8")
    Wm = oracle.decompress(vals, idx, R, K, N, M, "i8").astype(np.int64)
    a1 = oracle.spmm_direct(vals, idx, X1, R, K, N, M, "i8")
    # sum_t Y[r,t] = sum_k Wm[r,k] * (sum_t X[k,t])
    assert np.array_equal(a1.sum(axis=1), Wm @ X1.astype(np.int64).sum(axis=1))
    a2 = oracle.spmm_direct(vals, idx, X2, R, K, N, M, "i8")
    a12 = oracle.spmm_direct(vals, idx, (X1.astype(np.int16) + X2).astype(np.int8),
                             R, K, N, M, "i8")
    assert np.array_equal(a12, a1 + a2)


def test_requant_golden(golden_dir):
    acc, bias, scale, want = [], [], [], []
    for line in open(os.path.join(golden_dir, "requant_i8.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        a, b, s, y = line.split()
        acc.append(int(a))
        bias.append(int(b))
        scale.append(float.fromhex(s))
        want.append(int(y))
    n = len(acc)
    assert n >= 15
    # one row per case so that each gets its own bias and scale
    y = oracle.requant_i8(np.array(acc, np.int64)[:, None], np.array(bias, np.int32),
                          np.array(scale, np.float32))
    assert y[:, 0].tolist() == want


def test_requant_saturates_and_rounds_like_numpy_definition():
    # compare with a vectorised restatement in numpy float32 (RNE everywhere)
    r = nm_inputs.rng(12, "requant")
    acc = r.integers(-2**26, 2**26, size=(64, 50))
    bias = r.integers(-2**20, 2**20, size=64).astype(np.int32)
    scale = (r.random(64) * 1e-5).astype(np.float32)
    y = oracle.requant_i8(acc, bias, scale)
    f = (acc + bias[:, None]).astype(np.float32)
    p = (f * scale[:, None]).astype(np.float32)
    want = np.clip(np.rint(p), -128, 127).astype(np.int8)
    assert np.array_equal(y, want)


def test_reference_fp_rounding():
    R, K, T = 8, 16, 9
    W, X = _wx("f16", R, K, T, 13, "refround")
    y64 = oracle.reference(W, X, 2, 4, "f16", "f64")
    assert np.array_equal(oracle.reference(W, X, 2, 4, "f16", "f16"), y64.astype(np.float16))
    b = oracle.reference(W, X, 2, 4, "f16", "bf16")
    back = oracle.to_f64(b, "bf16")
    # one rounding to 8 significant bits: error <= half an ulp
    m, e = np.frexp(y64)
    assert np.all(np.abs(back - y64) <= np.ldexp(1.0, e - 9) + 0.0)


def test_exhaustive_int_sums_small():
    # all 2:4 patterns of a single group against every one-hot column
    for w in itertools.product((-3, 0, 2, 5), repeat=4):
        W = np.array([w], np.int8)
        X = np.eye(4, dtype=np.int8)
        acc = oracle.reference(W, X, 2, 4, "i8", "i32")
        mags = _mag_exact(W, "i8")
        keep = brute_keep(mags[0], 2, 4)[0]
        want = [w[k] if k in keep else 0 for k in range(4)]
        assert acc[0].tolist() == want


def test_reference_fp_bias_and_row_subset_by_hand():
    """oracle.reference with an fp32 bias, a `rows` subset and each output
    rounding, against values worked out by hand.

    W (2:4): row 0 = [1, -3, 2, 0.5] keeps positions 1, 2 (|-3|, |2|);
    row 1 = [0, 4, -1, 1] keeps positions 1, 2 (|4|, then |-1| == |1| goes to
    the lower position).  X = [[1, 2], [3, 4], [5, 6], [7, 8]]:
    row 0 -> [-3*3 + 2*5, -3*4 + 2*6] = [1, 0];
    row 1 -> [4*3 - 5, 4*4 - 6] = [7, 10].
    bias = [0.5, -0.25] -> [[1.5, 0.5], [6.75, 9.75]]; rows = [1] selects the
    second row and must take bias[1], not bias[0]."""
    for dt in ("f16", "bf16"):
        Wf = np.array([[1, -3, 2, 0.5], [0, 4, -1, 1]], np.float64)
        Xf = np.array([[1, 2], [3, 4], [5, 6], [7, 8]], np.float64)
        if dt == "f16":
            W, X = Wf.astype(np.float16), Xf.astype(np.float16)
        else:
            W, X = oracle.f64_to_bf16_bits(Wf), oracle.f64_to_bf16_bits(Xf)
        bias = np.array([0.5, -0.25], np.float32)
        full = oracle.reference(W, X, 2, 4, dt, "f64", bias=bias)
        assert full.tolist() == [[1.5, 0.5], [6.75, 9.75]]
        sub = oracle.reference(W, X, 2, 4, dt, "f64", bias=bias, rows=[1])
        assert sub.tolist() == [[6.75, 9.75]]
        assert oracle.reference(W, X, 2, 4, dt, "f32", bias=bias, rows=[1]).tolist() == [[6.75, 9.75]]
        nob = oracle.reference(W, X, 2, 4, dt, "f64", rows=[0, 1])
        assert nob.tolist() == [[1.0, 0.0], [7.0, 10.0]]
    # bf16 output rounding: 6.75 and 9.75 are exact in bf16 (8 significant
    # bits); 1/3-ish values are not -- 257 -> 256 (ties to even), 259 -> 260
    W = oracle.f64_to_bf16_bits(np.array([[1, 0, 0, 0]], np.float64))
    X = oracle.f64_to_bf16_bits(np.array([[256], [0], [0], [0]], np.float64))
    y = oracle.reference(W, X, 1, 4, "bf16", "bf16", bias=np.array([1.0], np.float32))
    assert oracle.to_f64(y, "bf16").tolist() == [[256.0]]
    y = oracle.reference(W, X, 1, 4, "bf16", "bf16", bias=np.array([3.0], np.float32))
    assert oracle.to_f64(y, "bf16").tolist() == [[260.0]]


def test_reference_int8_row_subset_by_hand():
    """int8 reference on a `rows` subset indexes bias and scale by the
    original row numbers.  Row 2 of W = [10, -20, 1, 0] keeps positions 0, 1;
    X column = [3, 1, 7, 7] -> acc = 30 - 20 = 10; + bias[2] = 5 -> 15;
    * scale[2] = 0.5 -> 7.5 -> 8 (round half to even); int32 out: 15.
    Row 0 = [1, 1, 1, 1] keeps positions 0, 1 -> acc 4, + bias[0] 100 -> 104;
    row 1 with scale 1 and bias 200: 2*3 + 2*1 + 200 = 208 -> saturates to
    127."""
    W = np.array([[1, 1, 1, 1], [2, 2, 2, 2], [10, -20, 1, 0]], np.int8)
    X = np.array([[3], [1], [7], [7]], np.int8)
    bias = np.array([100, 200, 5], np.int32)
    scale = np.array([1.0, 1.0, 0.5], np.float32)
    assert oracle.reference(W, X, 2, 4, "i8", "i32", bias=bias, rows=[2]).tolist() == [[15]]
    assert oracle.reference(W, X, 2, 4, "i8", "i8", bias=bias, scale=scale, rows=[2]).tolist() == [[8]]
    assert oracle.reference(W, X, 2, 4, "i8", "i8", bias=bias, scale=scale, rows=[0, 2]).tolist() == [[104], [8]]
    assert oracle.reference(W, X, 2, 4, "i8", "i8", bias=bias, scale=scale, rows=[1]).tolist() == [[127]]
