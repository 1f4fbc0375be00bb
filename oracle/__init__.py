"""CPU oracle for the N:M sparse weight x dense activation product.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use it; the product path never imports it.  It shares no code with
the HIP library.  The arithmetic lives in ``nm_oracle.c`` (plain C, built with
gcc); this module only marshals numpy arrays and rounds fp64 results to the
output dtype.

Paper followed: "Realizable N:M Sparse Transformer Inference via Search-Kernel
Co-Design" (arXiv 2607.12505) -- Sec. 2.1 (N of every M weights kept),
Sec. 4.2 (only the kept values of each window are computed on; execution
changes, the product does not).  Selection by largest |w| with ties to the
lower position, and the int8 requantising epilogue, are readings where the
pages are silent.

Every function here is pinned by the CPU tests (brute-force subset selection,
O1 == O2, dense special case N == M against numpy, identity / one-hot inputs,
closed-form checksums, hand-computed epilogue cases).

dtype names: 'i8' (numpy int8), 'f16' (numpy float16), 'bf16' (numpy uint16
holding raw bfloat16 bits).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nm_oracle.c")
_LIB = os.path.join(_HERE, "_nm_oracle.so")
_DT = {"i8": 0, "f16": 1, "bf16": 2}
_NP = {"i8": np.int8, "f16": np.float16, "bf16": np.uint16}

_lib = None


def build(force: bool = False) -> str:
    """Compile nm_oracle.c with gcc (-O2, no fp contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-std=c11", "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_compress.argtypes = [P, I64, I64, I, I, I, P, P]
        L.orc_decompress.argtypes = [P, P, I64, I64, I, I, I, P]
        L.orc_spmm_dense.argtypes = [P, P, I64, I64, I64, I, P, P]
        L.orc_spmm_direct.argtypes = [P, P, P, I64, I64, I64, I, I, I, P, I64, P, P, I]
        L.orc_requant_i8.argtypes = [P, I64, I64, P, P, P]
        L.orc_gelu.argtypes = [P, I64, P]
        L.orc_requant_gelu_i8.argtypes = [P, I64, I64, P, P, ctypes.c_float, ctypes.c_double, P, P]
        L.orc_read_packed.argtypes = [P, P, I64, I64, I, I, I, P, P]
        L.orc_check_padding.argtypes = [P, P, I64, I64, I, I, I]
        L.orc_check_padding.restype = ctypes.c_int64
        L.orc_max_threads.argtypes = []
        L.orc_hy_encode.argtypes = [P, I64, I64, I64, I, P, P, P, P, P, I64, P]
        L.orc_hy_read.argtypes = [P, P, P, P, P, I64, I64, I, P]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as(a, dt):
    a = np.ascontiguousarray(a)
    if a.dtype != _NP[dt]:
        raise TypeError(f"expected {_NP[dt]} for dtype {dt}, got {a.dtype}")
    return a


def _ok(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def compress(W, N: int, M: int, dt: str):
    """Top-N-by-|w| per group of M along K -> (vals[R][K/M][N], idx[R][K/M][N])."""
    W = _as(W, dt)
    R, K = W.shape
    vals = np.empty((R, K // M, N), dtype=_NP[dt])
    idx = np.empty((R, K // M, N), dtype=np.uint8)
    _ok(_load().orc_compress(_ptr(W), R, K, N, M, _DT[dt], _ptr(vals), _ptr(idx)), "compress")
    return vals, idx


def decompress(vals, idx, R: int, K: int, N: int, M: int, dt: str):
    """Zero-filled dense mask (.) W, same dtype as the values."""
    vals = _as(vals, dt)
    idx = np.ascontiguousarray(idx, dtype=np.uint8)
    Wm = np.empty((R, K), dtype=_NP[dt])
    _ok(_load().orc_decompress(_ptr(vals), _ptr(idx), R, K, N, M, _DT[dt], _ptr(Wm)), "decompress")
    return Wm


def spmm_dense(Wm, X, dt: str):
    """O1: naive triple loop over the decompressed matrix. int64 or float64."""
    Wm, X = _as(Wm, dt), _as(X, dt)
    R, K = Wm.shape
    K2, T = X.shape
    assert K == K2
    if dt == "i8":
        acc = np.empty((R, T), dtype=np.int64)
        _ok(_load().orc_spmm_dense(_ptr(Wm), _ptr(X), R, K, T, 0, _ptr(acc), None), "spmm_dense")
    else:
        acc = np.empty((R, T), dtype=np.float64)
        _ok(_load().orc_spmm_dense(_ptr(Wm), _ptr(X), R, K, T, _DT[dt], None, _ptr(acc)),
            "spmm_dense")
    return acc


def spmm_direct(vals, idx, X, R: int, K: int, N: int, M: int, dt: str, rows=None,
                nthreads: int = 0):
    """O2: loop over the compressed representation (only `rows`, if given)."""
    vals, X = _as(vals, dt), _as(X, dt)
    idx = np.ascontiguousarray(idx, dtype=np.uint8)
    K2, T = X.shape
    assert K == K2
    rws = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nr = R if rws is None else len(rws)
    if dt == "i8":
        acc = np.empty((nr, T), dtype=np.int64)
        ai, af = acc, None
    else:
        acc = np.empty((nr, T), dtype=np.float64)
        ai, af = None, acc
    _ok(_load().orc_spmm_direct(_ptr(vals), _ptr(idx), _ptr(X), R, K, T, N, M, _DT[dt], _ptr(rws),
                                nr, _ptr(ai), _ptr(af), nthreads), "spmm_direct")
    return acc


def requant_i8(acc, bias=None, scale=None):
    """sat_int8(round_half_even(f32(acc + bias[r]) * scale[r]))."""
    acc = np.ascontiguousarray(acc, dtype=np.int64)
    R, T = acc.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.int32)
    s = np.ascontiguousarray(scale, dtype=np.float32)
    y = np.empty((R, T), dtype=np.int8)
    _ok(_load().orc_requant_i8(_ptr(acc), R, T, _ptr(b), _ptr(s), _ptr(y)), "requant_i8")
    return y


def gelu(x):
    """x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)) in float64 (the fused FC1
    activation; the pages name none, this is the reading adopted)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    _ok(_load().orc_gelu(_ptr(x), x.size, _ptr(y)), "gelu")
    return y


# smallest half-integer distance under which an int8 GELU decision is taken
# as open; the C side widens it per element to four times the error bound of
# a binary32 evaluation with an erf accurate to 6e-7 (see orc_requant_gelu_i8)
GELU_I8_TOL = 2e-4


def requant_gelu_i8(acc, bias=None, scale=None, out_scale: float = 1.0, tol: float = GELU_I8_TOL):
    """sat_int8(rne(gelu(f32(acc + bias[r]) * scale[r]) * out_scale)) and the
    mask of decisions within `tol` of a half-integer."""
    acc = np.ascontiguousarray(acc, dtype=np.int64)
    R, T = acc.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.int32)
    s = np.ascontiguousarray(scale, dtype=np.float32)
    y = np.empty((R, T), dtype=np.int8)
    near = np.empty((R, T), dtype=np.uint8)
    _ok(_load().orc_requant_gelu_i8(_ptr(acc), R, T, _ptr(b), _ptr(s), float(out_scale), float(tol),
                                    _ptr(y), _ptr(near)), "requant_gelu_i8")
    return y, near.astype(bool)


def read_packed(values, meta, R: int, K: int, N: int, M: int, dt: str):
    """Decode the GPU library's blocked packed layout into (vals, idx)."""
    values = np.ascontiguousarray(values).view(np.uint8)
    meta = np.zeros(1, np.uint8) if meta is None or N == M else \
        np.ascontiguousarray(meta).view(np.uint8)
    vals = np.empty((R, K // M, N), dtype=_NP[dt])
    idx = np.empty((R, K // M, N), dtype=np.uint8)
    _ok(_load().orc_read_packed(_ptr(values), _ptr(meta), R, K, N, M, _DT[dt], _ptr(vals),
                                _ptr(idx)), "read_packed")
    return vals, idx


def check_padding(values, meta, R: int, K: int, N: int, M: int, dt: str) -> int:
    """Number of padding-rule violations in a packed buffer pair (0 = clean)."""
    values = np.ascontiguousarray(values).view(np.uint8)
    meta = None if meta is None or N == M else np.ascontiguousarray(meta).view(np.uint8)
    n = _load().orc_check_padding(_ptr(values), _ptr(meta), R, K, N, M, _DT[dt])
    if n < 0:
        raise ValueError("oracle check_padding rejected its arguments")
    return int(n)


def hy_geometry(R: int, K: int):
    """(nRB, nKB, nSeg) of the three-layer format."""
    nRB, nKB = (R + 15) // 16, (K + 63) // 64
    return nRB, nKB, (nKB + 7) // 8


def hy_encode(W, dt: str):
    """Three-layer image (Sparse-TC 2:4, slot filling with PDD codes, CSR
    residual) of raw fp16 / bf16 weights: dict of uint8 / int32 / uint32
    arrays 'values', 'meta', 'codes', 'res_ptr', 'res_ent'."""
    if dt not in ("f16", "bf16"):
        raise ValueError(dt)
    Wb = np.ascontiguousarray(W).view(np.uint16)
    R, K = Wb.shape
    nRB, nKB, nSeg = hy_geometry(R, K)
    img = {"values": np.empty(nRB * nKB * 1024, np.uint8),
           "meta": np.empty(nRB * nKB * 128, np.uint8),
           "codes": np.empty(nRB * nSeg * 512, np.uint8),
           "res_ptr": np.empty(nRB * nSeg * 16 + 1, np.int32)}
    n = ctypes.c_int64(0)
    args = lambda ent, cap: (_ptr(Wb), K, R, K, _DT[dt], _ptr(img["values"]), _ptr(img["meta"]),
                             _ptr(img["codes"]), _ptr(img["res_ptr"]), _ptr(ent), cap,
                             ctypes.byref(n))
    rc = _load().orc_hy_encode(*args(None, 0))
    if rc < 0:
        raise ValueError("oracle hy_encode rejected its arguments")
    ent = np.empty(max(n.value, 1), np.uint32)
    _ok(_load().orc_hy_encode(*args(ent, n.value)), "hy_encode")
    img["res_ent"] = ent[:n.value]
    return img


def hy_read(img, R: int, K: int, dt: str):
    """Dense raw bits (uint16, R x K) rebuilt from a three-layer image."""
    W = np.empty((R, K), np.uint16)
    ent = img["res_ent"] if len(img["res_ent"]) else np.zeros(1, np.uint32)
    rc = _load().orc_hy_read(_ptr(np.ascontiguousarray(img["values"]).view(np.uint8)),
                             _ptr(np.ascontiguousarray(img["meta"]).view(np.uint8)),
                             _ptr(np.ascontiguousarray(img["codes"]).view(np.uint8)),
                             _ptr(np.ascontiguousarray(img["res_ptr"], dtype=np.int32)),
                             _ptr(np.ascontiguousarray(ent, dtype=np.uint32)), R, K, _DT[dt],
                             _ptr(W))
    if rc == -2:
        raise ValueError("inconsistent three-layer image")
    _ok(rc, "hy_read")
    return W


def max_threads() -> int:
    return int(_load().orc_max_threads())


# ---------------------------------------------------------------- rounding
def to_f64(a, dt: str):
    """Exact float64 view of i8 / f16 / bf16-bits arrays."""
    if dt == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32) \
            .astype(np.float64)
    return np.asarray(a).astype(np.float64)


def f64_to_bf16_bits(x):
    """Round float64 to bfloat16 (round half to even, one rounding), raw bits."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                  # x = m * 2^e, 0.5 <= |m| < 1
    q = np.rint(m * 256.0)              # 8 significant bits, half to even
    y = np.ldexp(q, e - 8).astype(np.float32)  # exact in binary32
    return (y.view(np.uint32) >> 16).astype(np.uint16)


def round_to(acc_f64, out: str):
    """Round an fp64 result once to the output dtype ('f16', 'bf16', 'f32')."""
    if out == "f16":
        return np.asarray(acc_f64, dtype=np.float64).astype(np.float16)
    if out == "bf16":
        return f64_to_bf16_bits(acc_f64)
    if out == "f32":
        return np.asarray(acc_f64, dtype=np.float64).astype(np.float32)
    raise ValueError(out)


def reference(W, X, N: int, M: int, dt: str, out: str, bias=None, scale=None, rows=None,
              nthreads: int = 0, act: str = "none", out_scale: float = 1.0):
    """Whole chain: select -> direct compressed product -> epilogue.

    i8 inputs: out 'i32' gives acc + bias (int32 range), out 'i8' the
    requantised int8.  fp inputs: fp64 acc (+ bias) rounded once to `out`; with
    out == 'f64' the unrounded value.  `rows` restricts the output to those
    rows (bias/scale are then indexed by the original row numbers).
    act == 'gelu': fp outputs take gelu of the fp64 value before rounding;
    int8 outputs return (codes, open-decision mask) of requant_gelu_i8.
    """
    if act not in ("none", "gelu"):
        raise ValueError(act)
    R, K = W.shape
    vals, idx = compress(W, N, M, dt)
    acc = spmm_direct(vals, idx, X, R, K, N, M, dt, rows=rows, nthreads=nthreads)
    sel = slice(None) if rows is None else np.asarray(rows, dtype=np.int64)
    if dt == "i8":
        b = None if bias is None else np.asarray(bias, dtype=np.int32)[sel]
        if out == "i32":
            y = acc + (0 if b is None else b.astype(np.int64)[:, None])
            assert np.all(np.abs(y) < 2**31), "int32 range exceeded"
            return y.astype(np.int32)
        if out == "i8":
            if act == "gelu":
                return requant_gelu_i8(acc, b, np.asarray(scale, dtype=np.float32)[sel], out_scale)
            return requant_i8(acc, b, np.asarray(scale, dtype=np.float32)[sel])
        raise ValueError(out)
    if bias is not None:
        acc = acc + np.asarray(bias, dtype=np.float32).astype(np.float64)[sel][:, None]
    if act == "gelu":
        acc = gelu(acc)
    return acc if out == "f64" else round_to(acc, out)
