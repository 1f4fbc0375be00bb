"""Shared helpers of the GPU parity tests: host inputs -> device, one call of
the library, comparison with the oracle at the documented tolerance."""
from __future__ import annotations

import numpy as np
import torch

import nm_inputs
import oracle
import semi_structured_sparse_nm_amd as nm

TORCH_DT = {"i8": torch.int8, "f16": torch.float16, "bf16": torch.bfloat16, "i32": torch.int32,
            "f32": torch.float32}

# fp16 / bf16 inputs, fp32 output or fp16 output: max |gpu - ref| / max |ref| <= 2e-3,
# ref = the fp64 product (fp32 accumulation of exact products keeps the error
# far below this; an fp16 output adds at most half an fp16 ulp, 2^-11 relative).
FP_TOL = 2e-3
# bf16 output: rounding to 8 significant bits alone can cost 2^-8 of max |ref|;
# elementwise the result must also be within one bf16 ulp of the rounded ref
# plus the fp32 accumulation error of the value before rounding (bounded here
# by 2^-16 max |ref|, far above the ~1e-6 relative error of fp32 sums of at
# most 5504 products, far below a bf16 ulp of max |ref|).
BF16_OUT_TOL = 2.0 ** -8 + 1e-4
BF16_ACC_SLACK = 2.0 ** -16


def dev(a: np.ndarray, dt: str, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dt == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(device)


def host(t: torch.Tensor, dt: str) -> np.ndarray:
    t = t.cpu()
    if dt == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def run(W, X, N, M, dt, out, bias=None, scale=None, ldx_pad=0, ldy_pad=0, sentinel=None, act="none",
        out_scale=1.0):
    """One nm_pack + nm_spmm (nm_spmm_act) call; returns (Y host array [R, T], packed)."""
    R, K = W.shape
    T = X.shape[1]
    Wd = dev(W, dt)
    Xfull = torch.zeros((K, T + ldx_pad), dtype=TORCH_DT[dt], device="cuda")
    Xfull[:, :T] = dev(X, dt)
    Xv = Xfull[:, :T]
    p = nm.pack(Wd, N, M)
    Yfull = torch.empty((R, T + ldy_pad), dtype=TORCH_DT[out], device="cuda")
    if sentinel is not None:
        Yfull.fill_(sentinel)
    Yv = Yfull[:, :T]
    b = None
    if bias is not None:
        b = torch.from_numpy(np.asarray(bias)).to("cuda")
    s = None if scale is None else torch.from_numpy(np.asarray(scale, np.float32)).to("cuda")
    nm.spmm(p, Xv, bias=b, scale=s, out_dtype=TORCH_DT[out], out=Yv, act=act, out_scale=out_scale)
    torch.cuda.synchronize()
    return host(Yfull, out), p


def packed_host(p):
    v = p.values.cpu().numpy()
    m = None if p.meta is None else p.meta.cpu().numpy()
    return v, m


def compare(Y, ref, out, what=""):
    """Element-by-element comparison at the tolerance of the output dtype."""
    if out in ("i32", "i8"):
        bad = np.argwhere(Y != ref)
        assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}: " \
                              f"gpu {Y[tuple(bad[0])]} ref {ref[tuple(bad[0])]}"
        return 0.0
    ref64 = ref
    y64 = oracle.to_f64(Y, out) if out == "bf16" else np.asarray(Y).astype(np.float64)
    den = max(np.abs(ref64).max(), 1e-30)
    err = np.abs(y64 - ref64).max() / den
    tol = BF16_OUT_TOL if out == "bf16" else FP_TOL
    assert np.isfinite(y64).all(), f"{what}: non-finite output"
    if err > tol:
        d = np.abs(y64 - ref64) / den
        bad = np.argwhere(d > tol)
        rows, cols = np.unique(bad[:, 0]), np.unique(bad[:, 1])
        i = tuple(np.unravel_index(np.argmax(d), d.shape))
        raise AssertionError(
            f"{what}: max-abs-normalised error {err:.3e} > {tol:.3e} at {i} (gpu {y64[i]} ref "
            f"{ref64[i]}); {len(bad)} bad elements in rows {rows[:12].tolist()}.. ({len(rows)}) "
            f"cols {cols[:12].tolist()}.. ({len(cols)})")
    if out == "bf16":
        rr = oracle.to_f64(oracle.round_to(ref64, "bf16"), "bf16")
        m, e = np.frexp(np.where(rr == 0, 1e-38, rr))
        ulp = np.ldexp(1.0, e - 8)
        lim = ulp * (1 + 1e-12) + BF16_ACC_SLACK * den
        assert np.all(np.abs(y64 - rr) <= lim), \
            f"{what}: more than 1 bf16 ulp + fp32 accumulation slack off"

    return float(err)


def reference(W, X, N, M, dt, out, bias=None, scale=None, rows=None, act="none", out_scale=1.0):
    """Oracle result in the comparison domain: exact ints, or fp64 for fp
    outputs; int8 with an activation: (codes, open-decision mask)."""
    if dt == "i8":
        return oracle.reference(W, X, N, M, dt, out, bias=bias, scale=scale, rows=rows, act=act,
                                out_scale=out_scale)
    return oracle.reference(W, X, N, M, dt, "f64", bias=bias, rows=rows, act=act)


def compare_i8_open(Y, ref, near, what=""):
    """int8 codes whose exact value lies within the oracle's tolerance of a
    half-integer may take either neighbouring code (a binary32 evaluation of
    the activation decides them); every other code must match exactly."""
    Y = np.asarray(Y).astype(np.int64)
    ref = np.asarray(ref).astype(np.int64)
    bad = np.argwhere((Y != ref) & ~near)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches on closed decisions, first at {bad[:5].tolist()}: " \
                          f"gpu {Y[tuple(bad[0])]} ref {ref[tuple(bad[0])]}"
    assert np.all(np.abs(Y - ref)[near] <= 1), f"{what}: an open decision is off by more than one code"
    return int((Y != ref).sum())


def layer_case(L: nm_inputs.Layer, seed: int = 0):
    inp = nm_inputs.make_inputs(L, seed)
    return inp["W"], inp["X"], inp["bias"], inp["scale"]
