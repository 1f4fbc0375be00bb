"""The latency look-up table: lookup, interpolation, prediction, calibration,
persistence (CPU), and a measured table predicting a measured stack (GPU)."""
import math

import pytest

from semi_structured_sparse_nm_amd.lut import LatencyLUT, LayerShape


def L(T=1024, R=768, K=768, N=2, M=4, dt="i8", out="i8"):
    return LayerShape(R, K, T, N, M, dt, out)


def test_exact_and_interpolated_lookup():
    lut = LatencyLUT()
    lut.add(L(T=1000), 10.0)
    lut.add(L(T=3000), 30.0)
    lut.add(L(T=5000), 40.0)
    assert lut.lookup(L(T=1000)) == 10.0
    assert lut.lookup(L(T=2000)) == pytest.approx(20.0)
    assert lut.lookup(L(T=4000)) == pytest.approx(35.0)
    # extrapolation from the two nearest entries
    assert lut.lookup(L(T=7000)) == pytest.approx(50.0)
    assert lut.lookup(L(T=500)) == pytest.approx(5.0)
    # a single entry scales in proportion to T
    lut.add(L(T=100, N=1), 4.0)
    assert lut.lookup(L(T=300, N=1)) == pytest.approx(12.0)


def test_lookup_is_keyed_by_the_whole_shape():
    lut = LatencyLUT()
    lut.add(L(N=2, M=4), 10.0)
    for other in (L(N=1, M=4), L(N=2, M=8), L(R=769), L(K=1024), L(dt="f16", out="f16"), L(out="i32")):
        assert other not in lut
        with pytest.raises(KeyError):
            lut.lookup(other)
    assert L(N=2, M=4) in lut


def test_add_replaces_an_entry_and_rejects_bad_values():
    lut = LatencyLUT()
    lut.add(L(T=10), 1.0)
    lut.add(L(T=10), 2.0)
    assert len(lut) == 1 and lut.lookup(L(T=10)) == 2.0
    for bad in (0.0, -1.0, math.inf, math.nan):
        with pytest.raises(ValueError):
            lut.add(L(T=11), bad)


def test_predict_and_calibrate():
    lut = LatencyLUT()
    a, b = L(N=1), L(N=2)
    lut.add(a, 10.0)
    lut.add(b, 20.0)
    stack = [a, b, b, a, b]
    assert lut.predict(stack) == pytest.approx(80.0)
    gap = lut.calibrate(stack, 90.0)
    assert gap == pytest.approx(2.0)
    assert lut.predict(stack) == pytest.approx(90.0)
    assert lut.predict([a]) == pytest.approx(12.0)
    with pytest.raises(ValueError):
        lut.calibrate([], 1.0)


def test_json_round_trip():
    lut = LatencyLUT(gap_us=1.5, device="dev")
    lut.add(L(T=16, dt="f16", out="f16", N=4, M=8), 9.5)
    lut.add(L(T=2048, dt="f16", out="f16", N=4, M=8), 110.0)
    lut.add(L(T=12608), 31.0)
    back = LatencyLUT.from_json(lut.to_json())
    assert back.gap_us == 1.5 and back.device == "dev" and len(back) == 3
    assert back.keys() == lut.keys()
    for layer in (L(T=16, dt="f16", out="f16", N=4, M=8), L(T=1000, dt="f16", out="f16", N=4, M=8), L(T=12608)):
        assert back.lookup(layer) == lut.lookup(layer)


@pytest.mark.gpu
def test_measured_table_predicts_a_measured_stack():
    """Calibrate the per-launch gap on one mixed stack and predict another
    (other order and mix) within 10%.  These stacks are short (6 and 8
    launches of small layers) and timed a few times, so launch jitter weighs
    more than in the 48-layer ViT-B stacks `bench.py --lut` predicts (0.6-2.1%
    there)."""
    from semi_structured_sparse_nm_amd.lut import measure_layers, time_stack
    shapes = [L(T=4096, R=2048, K=1024, N=n, M=m) for n, m in ((1, 4), (2, 4), (4, 8), (8, 8))]
    lut = measure_layers(shapes, reps=10)
    assert len(lut) == 4 and all(lut.lookup(s) > 0 for s in shapes)
    calib = [shapes[i] for i in (0, 1, 2, 3, 1, 2)]
    lut.calibrate(calib, time_stack(calib, reps=5))
    other = [shapes[i] for i in (3, 3, 0, 2, 1, 0, 1, 3)]
    measured = time_stack(other, reps=5, seed=5)
    pred = lut.predict(other)
    print(f"predicted {pred:.1f} us, measured {measured:.1f} us", flush=True)
    assert abs(pred - measured) / measured < 0.10, (pred, measured)
