"""GPU parity of the three-layer format product (nm_hybrid_spmm) against the
oracle: Y = W X of the whole sparse weight W (every nonzero, in any layer),
fp64, + bias, GELU, rounded to the output dtype.  Format and kernel: page
"Accelerating GPU Inference of Large Language Models with Moderately
Unstructured Sparse Weight Matrices", Methodology 1 and 2."""
import numpy as np
import pytest
import torch

import nm_inputs
import oracle
import semi_structured_sparse_nm_amd as nm
from _parity import TORCH_DT, compare, dev, host

pytestmark = pytest.mark.gpu


def _ref(W, X, dt, bias=None, act="none", rows=None):
    Wd = W if rows is None else W[rows]
    acc = oracle.spmm_dense(Wd, X, dt)
    if bias is not None:
        b = np.asarray(bias, np.float32).astype(np.float64)
        acc = acc + (b if rows is None else b[rows])[:, None]
    if act == "gelu":
        acc = oracle.gelu(acc)
    return acc


def _run(W, X, dt, out, bias=None, act="none", ldx_pad=0, ldy_pad=0):
    R, K = W.shape
    T = X.shape[1]
    h = nm.pack_hybrid(dev(W, dt).cpu(), device="cuda")
    Xf = torch.zeros((K, T + ldx_pad), dtype=TORCH_DT[dt], device="cuda")
    Xf[:, :T] = dev(X, dt)
    Yf = torch.full((R, T + ldy_pad), 7.0, dtype=TORCH_DT[out], device="cuda")
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).cuda()
    nm.spmm_hybrid(h, Xf[:, :T], bias=b, out_dtype=TORCH_DT[out], out=Yf[:, :T], act=act)
    torch.cuda.synchronize()
    Y = host(Yf, out)
    if ldy_pad:   # the padding columns are not written
        assert np.all(Y[:, T:].astype(np.float64) == 7.0) if out != "bf16" else True
    return Y[:, :T], h


CASES = [
    # R, K, T, density
    (16, 64, 1, 0.5),
    (37, 520, 3, 0.5),
    (64, 4096, 16, 0.5),
    (48, 8256, 16, 0.5),     # three chunks, ragged last segment
    (100, 2048, 40, 0.5),    # three token tiles
    (40, 1024, 16, 0.3),
    (40, 1024, 16, 0.8),     # more surplus than slots: residual
    (300, 512, 8, 0.5),      # several row blocks per workgroup
]


@pytest.mark.parametrize("dt,out", [("f16", "f16"), ("f16", "f32"), ("bf16", "f32"), ("bf16", "bf16")])
@pytest.mark.parametrize("R,K,T,dens", CASES)
def test_hybrid_parity(dt, out, R, K, T, dens):
    W = nm_inputs.unstructured(R, K, dens, dt, 0, "hy", R, K)
    X = nm_inputs.normal((K, T), 1.0, dt, 0, "hyX", K, T)
    print(f"case R={R} K={K} T={T} dens={dens} {dt}->{out}", flush=True)
    Y, h = _run(W, X, dt, out)
    compare(Y, _ref(W, X, dt), out, f"hybrid {R}x{K}x{T} {dens}")


@pytest.mark.parametrize("act", ["none", "gelu"])
def test_hybrid_bias_act_strides(act):
    R, K, T = 70, 1536, 5
    W = nm_inputs.unstructured(R, K, 0.5, "f16", 1, "hyb")
    X = nm_inputs.normal((K, T), 1.0, "f16", 1, "hybX")
    bias = nm_inputs.normal((R,), 0.5, "f32", 1, "hybB")
    Y, _ = _run(W, X, "f16", "f32", bias=bias, act=act, ldx_pad=5, ldy_pad=3)
    compare(Y, _ref(W, X, "f16", bias, act), "f32", f"hybrid bias {act}")


def test_hybrid_structured_and_two_of_four():
    """4:8 weights: held by the first two layers (no residual beyond what the
    code cap leaves); 2:4 weights: Sparse-TC layer only."""
    R, K, T = 96, 768, 16
    W48 = nm_inputs.structured(R, K, 4, 8, "f16", 0, "hy48")
    X = nm_inputs.normal((K, T), 1.0, "f16", 0, "hy48X")
    Y, h = _run(W48, X, "f16", "f32")
    compare(Y, _ref(W48, X, "f16"), "f32", "hybrid 4:8")
    W24 = nm_inputs.structured(R, K, 2, 4, "f16", 0, "hy24")
    Y, h = _run(W24, X, "f16", "f32")
    assert h.n_fill == 0 and h.n_res == 0
    compare(Y, _ref(W24, X, "f16"), "f32", "hybrid 2:4")


def test_hybrid_deterministic():
    R, K, T = 256, 4096, 16
    W = nm_inputs.unstructured(R, K, 0.5, "bf16", 2, "hyd")
    X = nm_inputs.normal((K, T), 1.0, "bf16", 2, "hydX")
    h = nm.pack_hybrid(dev(W, "bf16").cpu(), device="cuda")
    Xd = dev(X, "bf16")
    y1 = nm.spmm_hybrid(h, Xd, out_dtype=torch.float32)
    y2 = nm.spmm_hybrid(h, Xd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("L", nm_inputs.hybrid_workloads(), ids=lambda L: L.name)
def test_hybrid_full_size(L):
    """Every workload at its full size; the whole output against the oracle."""
    inp = nm_inputs.hybrid_inputs(L)
    W, X = inp["W"], inp["X"]
    print(f"case {L.name}", flush=True)
    Y, h = _run(W, X, L.dt, L.out)
    nnz = int(((W.view(np.uint16) & 0x7FFF) != 0).sum())
    print(f"  slot-filled {h.n_fill / nnz:.4f} residual {h.n_res / nnz:.4f} of {nnz} nonzeros", flush=True)
    compare(Y, _ref(W, X, L.dt), L.out, L.name)


def test_hybrid_rejects():
    W = nm_inputs.unstructured(32, 256, 0.5, "f16", 0, "hyr")
    h = nm.pack_hybrid(dev(W, "f16").cpu(), device="cuda")
    X = dev(nm_inputs.normal((256, 4), 1.0, "f16", 0, "hyrX"), "f16")
    with pytest.raises(nm.NmError):
        nm.spmm_hybrid(h, X, out_dtype=torch.int32)
    d = h.desc()
    d.codes_bytes -= 8
    Y = torch.empty((32, 4), dtype=torch.float16, device="cuda")
    st = nm.lib().nm_hybrid_spmm(__import__("ctypes").byref(d), X.data_ptr(), 4, 4, Y.data_ptr(), 4, nm.NM_F16,
                                 None, 0, None)
    assert st == nm.NM_EINVAL
