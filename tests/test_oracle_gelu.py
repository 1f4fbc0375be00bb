"""Pins of the oracle's fused-activation epilogue (GELU, x * Phi(x)).

The pages name no activation; the fused FC1 epilogue takes the exact
Gaussian-error linear unit of the ViT / Swin MLP.  Pinned to the standard
normal distribution function at tabulated points, to the identity
gelu(x) - gelu(-x) = x (Phi(x) + Phi(-x) = 1), to its curvature at 0
(gelu(h) + gelu(-h) = h (2 Phi(h) - 1) ~ 2 phi(0) h^2, which a wrong erf
argument scale breaks), its limits, and hand-computed int8 cases."""
import math

import numpy as np
import pytest

import oracle

# standard normal distribution function Phi(x) at tabulated points
# (any table of the normal integral, e.g. Abramowitz & Stegun Table 26.1)
PHI = [(0.5, 0.691462461274013), (1.0, 0.841344746068543), (1.5, 0.933192798731142),
       (2.0, 0.977249868051821), (3.0, 0.998650101968370)]


def test_gelu_at_tabulated_points():
    for x, phi in PHI:
        assert oracle.gelu(np.array([x]))[0] == pytest.approx(x * phi, rel=1e-13, abs=0)
        assert oracle.gelu(np.array([-x]))[0] == pytest.approx(-x * (1.0 - phi), rel=1e-11, abs=0)
    assert oracle.gelu(np.array([0.0]))[0] == 0.0


def test_gelu_odd_part_is_identity():
    x = np.random.default_rng(0).standard_normal(10000) * 3
    d = oracle.gelu(x) - oracle.gelu(-x)
    assert np.allclose(d, x, rtol=1e-14, atol=1e-15)


def test_gelu_curvature_at_zero():
    h = np.array([1e-3, 1e-4])
    even = (oracle.gelu(h) + oracle.gelu(-h)) / h ** 2
    assert np.allclose(even, 2.0 / math.sqrt(2.0 * math.pi), rtol=1e-5)


def test_gelu_limits():
    x = np.array([9.0, 20.0, 1e3])
    assert np.array_equal(oracle.gelu(x), x)
    assert np.all(np.abs(oracle.gelu(-x)) < 1e-17)


def test_requant_gelu_i8_hand_cases():
    # scale 1/4096 turns acc 4096 k into p = k exactly
    acc = np.array([[4096, -4096, 0, 40960, -40960, 2048, 3 * 4096]], dtype=np.int64)
    scale = np.array([1.0 / 4096], dtype=np.float32)
    y, near = oracle.requant_gelu_i8(acc, None, scale, out_scale=100.0)
    # 100 * (1 * 0.84134..) = 84.13 -> 84; 100 * (-1 * 0.15866..) = -15.87 -> -16;
    # 0 -> 0; p = 10 -> 1000 -> 127; p = -10 -> ~ -7.7e-21 -> 0;
    # p = 0.5 -> 100 * 0.5 * 0.69146.. = 34.57 -> 35; p = 3 -> 299.6 -> 127
    assert y.tolist() == [[84, -16, 0, 127, 0, 35, 127]]
    assert not near.any()
    # bias joins the integer sum before the conversion: 2048 + 2048 = 4096 -> p = 1
    y, _ = oracle.requant_gelu_i8(np.array([[2048]]), np.array([2048], np.int32), scale, 100.0)
    assert y.tolist() == [[84]]
    # an output scale that puts v within 1e-12 of 84.5 marks the decision open
    os_ = np.float32(84.5 / 0.841344746068543)
    y, near = oracle.requant_gelu_i8(np.array([[4096]]), None, scale, float(os_))
    v = 0.841344746068543 * float(os_)
    assert abs(v - 84.5) < 1e-5 and near.all() and y[0, 0] in (84, 85)


def test_reference_gelu_paths():
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((8, 16)) * 0.5).astype(np.float16)
    X = rng.standard_normal((16, 5)).astype(np.float16)
    plain = oracle.reference(W, X, 2, 4, "f16", "f64")
    act = oracle.reference(W, X, 2, 4, "f16", "f64", act="gelu")
    assert np.allclose(act, plain * 0.5 * (1 + np.vectorize(math.erf)(plain / math.sqrt(2))), rtol=1e-14)
    Wq = rng.integers(-127, 128, (8, 16)).astype(np.int8)
    Xq = rng.integers(-127, 128, (16, 5)).astype(np.int8)
    s = np.full(8, 1e-4, np.float32)
    y, near = oracle.reference(Wq, Xq, 2, 4, "i8", "i8", scale=s, act="gelu", out_scale=20.0)
    acc = oracle.reference(Wq, Xq, 2, 4, "i8", "i32").astype(np.int64)
    p = (acc.astype(np.float32) * s[:, None]).astype(np.float64)
    v = p * 0.5 * (1 + np.vectorize(math.erf)(p / math.sqrt(2))) * 20.0
    want = np.clip(np.rint(v), -128, 127)
    assert np.array_equal(y[~near], want[~near])
    with pytest.raises(ValueError):
        oracle.reference(W, X, 2, 4, "f16", "f64", act="relu")
