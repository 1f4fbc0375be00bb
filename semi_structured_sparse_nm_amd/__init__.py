"""MI355X (gfx950) N:M semi-structured sparse weight x dense activation product.

Thin Python binding of libnmsparse.so (C ABI in include/nm_sparse.h): it only
marshals torch tensors to device pointers and the current HIP stream; every
step of the computation runs in the library's HIP kernels.  PyTorch provides
device memory and streams.  There is no CPU fallback: without the built
library every call raises.

    p = pack(W, N, M)                      # W: [R, K] int8 / float16 / bfloat16 on the GPU
    Y = spmm(p, X, bias=None, scale=None, out_dtype=None)   # X: [K, T]  ->  Y: [R, T]

Operation: paper "Realizable N:M Sparse Transformer Inference via
Search-Kernel Co-Design" (arXiv 2607.12505) -- Sec. 2.1 N:M constraint,
Sec. 4.2 packed windows and micro-dense execution.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnmsparse.so")

NM_OK, NM_EINVAL, NM_EUNSUPPORTED, NM_EHIP = 0, 1, 2, 3
NM_I8, NM_F16, NM_BF16, NM_I32, NM_F32 = 0, 1, 2, 3, 4
FORMAT_VERSION = 1

_TORCH_TO_NM = {torch.int8: NM_I8, torch.float16: NM_F16, torch.bfloat16: NM_BF16,
                torch.int32: NM_I32, torch.float32: NM_F32}
_NM_TO_TORCH = {v: k for k, v in _TORCH_TO_NM.items()}


class NmPacked(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("K", ctypes.c_int64), ("N", ctypes.c_int32),
                ("M", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("format_version", ctypes.c_uint32), ("values", ctypes.c_void_p),
                ("values_bytes", ctypes.c_size_t), ("meta", ctypes.c_void_p),
                ("meta_bytes", ctypes.c_size_t)]


class NmHybrid(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("K", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("format_version", ctypes.c_uint32),
                ("values", ctypes.c_void_p), ("values_bytes", ctypes.c_size_t),
                ("meta", ctypes.c_void_p), ("meta_bytes", ctypes.c_size_t),
                ("codes", ctypes.c_void_p), ("codes_bytes", ctypes.c_size_t),
                ("res_ptr", ctypes.c_void_p), ("res_ptr_bytes", ctypes.c_size_t),
                ("res_ent", ctypes.c_void_p), ("res_ent_bytes", ctypes.c_size_t),
                ("n_fill", ctypes.c_int64), ("n_res", ctypes.c_int64)]


HYBRID_BUFFERS = ("values", "meta", "codes", "res_ptr", "res_ent")


class NmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libnmsparse.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m semi_structured_sparse_nm_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        PP = ctypes.POINTER(NmPacked)
        L.nm_pack_size.argtypes = [I64, I64, I32, I32, I32, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]
        L.nm_pack.argtypes = [P, I64, PP, P]
        L.nm_spmm_workspace_size.argtypes = [PP, I64, I32, ctypes.POINTER(SZ)]
        L.nm_spmm_tk_workspace_size.argtypes = [PP, I64, I32, ctypes.POINTER(SZ)]
        L.nm_spmm.argtypes = [PP, P, I64, I64, P, I64, I32, P, P, P, SZ, P]
        L.nm_status_str.argtypes = [ctypes.c_int]
        L.nm_status_str.restype = ctypes.c_char_p
        L.nm_spmm_variant.argtypes = [PP, I64, I32]
        L.nm_spmm_variant.restype = ctypes.c_char_p
        L.nm_spmm_ksplit.argtypes = [PP, I64, I32, I32]
        L.nm_spmm_ksplit.restype = I32
        L.nm_spmm_variant_act.argtypes = [PP, I64, I32, I32]
        L.nm_spmm_variant_act.restype = ctypes.c_char_p
        L.nm_spmm_act.argtypes = [PP, P, I64, I64, P, I64, I32, P, P, I32, ctypes.c_float, P, SZ, P]
        L.nm_spmm_act.restype = ctypes.c_int
        L.nm_spmm_tk.argtypes = [PP, P, I64, I64, P, I64, I32, P, P, I32, ctypes.c_float, P, SZ, P]
        L.nm_spmm_tk.restype = ctypes.c_int
        L.nm_spmm_variant_tk.argtypes = [PP, I64, I32, I32]
        L.nm_spmm_variant_tk.restype = ctypes.c_char_p
        L.nm_spmm_noalloc.argtypes = [PP, P, I64, I64, P, I64, I32, P, P, I32, ctypes.c_float, P]
        L.nm_spmm_noalloc.restype = ctypes.c_int
        L.nm_spmm_noalloc_max_bytes.argtypes = []
        L.nm_spmm_noalloc_max_bytes.restype = SZ
        HP = ctypes.POINTER(NmHybrid)
        L.nm_hybrid_pack_size.argtypes = [P, I64, I64, I64, I32, HP]
        L.nm_hybrid_pack.argtypes = [P, I64, HP]
        L.nm_hybrid_spmm.argtypes = [HP, P, I64, I64, P, I64, I32, P, I32, P]
        for f in ("nm_pack_size", "nm_pack", "nm_spmm_workspace_size", "nm_spmm", "nm_hybrid_pack_size",
                  "nm_hybrid_pack", "nm_hybrid_spmm"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def status_str(s: int) -> str:
    return lib().nm_status_str(int(s)).decode()


def _check(st: int, what: str):
    if st != NM_OK:
        raise NmError(st, what)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def pack_size(rows: int, K: int, N: int, M: int, dtype: int):
    vb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().nm_pack_size(rows, K, N, M, dtype, ctypes.byref(vb), ctypes.byref(mb)),
           "nm_pack_size")
    return vb.value, mb.value


@dataclass
class Packed:
    """Packed N:M weights on the GPU (two uint8 device buffers + shape)."""
    rows: int
    K: int
    N: int
    M: int
    dtype: int
    values: torch.Tensor
    meta: torch.Tensor | None
    format_version: int = FORMAT_VERSION

    def desc(self) -> NmPacked:
        d = NmPacked()
        d.rows, d.K, d.N, d.M, d.dtype = self.rows, self.K, self.N, self.M, self.dtype
        d.format_version = self.format_version
        d.values, d.values_bytes = self.values.data_ptr(), self.values.numel()
        if self.meta is not None:
            d.meta, d.meta_bytes = self.meta.data_ptr(), self.meta.numel()
        else:
            d.meta, d.meta_bytes = None, 0
        return d

    @property
    def torch_dtype(self):
        return _NM_TO_TORCH[self.dtype]


def pack(W: torch.Tensor, N: int, M: int) -> Packed:
    """nm_pack: keep the N largest-|w| of every M consecutive K-elements of each row."""
    if W.dim() != 2 or W.stride(1) != 1:
        raise ValueError("W must be a 2-D tensor with unit stride along K")
    dt = _TORCH_TO_NM.get(W.dtype)
    if dt not in (NM_I8, NM_F16, NM_BF16):
        raise TypeError(f"unsupported weight dtype {W.dtype}")
    if W.device.type != "cuda":
        raise ValueError(f"W is on {W.device}, not on a GPU")
    R, K = W.shape
    vb, mb = pack_size(R, K, N, M, dt)
    values = torch.empty(vb, dtype=torch.uint8, device=W.device)
    meta = torch.empty(mb, dtype=torch.uint8, device=W.device) if mb else None
    p = Packed(R, K, N, M, dt, values, meta, 0)
    d = p.desc()
    _check(lib().nm_pack(W.data_ptr(), W.stride(0), ctypes.byref(d), _stream(W.device)), "nm_pack")
    p.format_version = d.format_version
    return p


def _check_operands(p: Packed, X: torch.Tensor, out: torch.Tensor, out_dtype: torch.dtype,
                    bias: torch.Tensor | None, scale: torch.Tensor | None,
                    workspace: torch.Tensor | None) -> None:
    """Type, length and device checks of one product's operands, before any
    launch: the kernels size every buffer range from the requested dtypes and
    R, so a mismatch here would read or write past a tensor's end."""
    wdt = p.torch_dtype
    if X.dtype != wdt:
        raise TypeError(f"activation dtype {X.dtype} does not match the weight dtype {wdt}")
    if out.dtype != out_dtype:
        raise TypeError(f"out has dtype {out.dtype}, the call asks for {out_dtype}")
    if _TORCH_TO_NM.get(out_dtype) is None:
        raise TypeError(f"unsupported output dtype {out_dtype}")
    want_bias = torch.int32 if p.dtype == NM_I8 else torch.float32
    for name, t, dt in (("bias", bias, want_bias), ("scale", scale, torch.float32)):
        if t is None:
            continue
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt} for {wdt} weights, got {t.dtype}")
        if t.dim() != 1 or t.numel() != p.rows or (t.numel() > 1 and t.stride(0) != 1):
            raise ValueError(f"{name} must be a contiguous vector of length R={p.rows}, got {tuple(t.shape)}")
    if out_dtype == torch.int8 and scale is None:
        raise ValueError("int8 output needs a float32 scale of length R")
    dev = p.values.device
    if dev.type != "cuda":
        raise ValueError(f"the packed weight is on {dev}, not on a GPU")
    for name, t in (("X", X), ("out", out), ("bias", bias), ("scale", scale), ("workspace", workspace),
                    ("meta", p.meta)):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the packed weight on {dev}")
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")


def default_out_dtype(wdt: int) -> torch.dtype:
    return {NM_I8: torch.int32, NM_F16: torch.float16, NM_BF16: torch.bfloat16}[wdt]


def workspace_size(p: Packed, T: int, out_dtype: torch.dtype) -> int:
    n = ctypes.c_size_t()
    d = p.desc()
    _check(lib().nm_spmm_workspace_size(ctypes.byref(d), T, _TORCH_TO_NM[out_dtype], ctypes.byref(n)),
           "nm_spmm_workspace_size")
    return n.value


def workspace_size_tk(p: Packed, T: int, out_dtype: torch.dtype) -> int:
    """nm_spmm_tk_workspace_size: the workspace linear() needs."""
    n = ctypes.c_size_t()
    d = p.desc()
    _check(lib().nm_spmm_tk_workspace_size(ctypes.byref(d), T, _TORCH_TO_NM[out_dtype], ctypes.byref(n)),
           "nm_spmm_tk_workspace_size")
    return n.value


ACTS = {"none": 0, "gelu": 1}


def variant(p: Packed, T: int, out_dtype: torch.dtype, act: str = "none") -> str:
    d = p.desc()
    return lib().nm_spmm_variant_act(ctypes.byref(d), T, _TORCH_TO_NM[out_dtype], ACTS[act]).decode()


def variant_tk(p: Packed, T: int, out_dtype: torch.dtype, act: str = "none") -> str:
    d = p.desc()
    return lib().nm_spmm_variant_tk(ctypes.byref(d), T, _TORCH_TO_NM[out_dtype], ACTS[act]).decode()


def ksplit(p: Packed, T: int, out_dtype: torch.dtype, act: str = "none") -> int:
    """K slices (workgroup-level split of K) nm_spmm would use; 1 = none."""
    d = p.desc()
    return int(lib().nm_spmm_ksplit(ctypes.byref(d), T, _TORCH_TO_NM[out_dtype], ACTS[act]))


def spmm(p: Packed, X: torch.Tensor, bias: torch.Tensor | None = None,
         scale: torch.Tensor | None = None, out_dtype: torch.dtype | None = None,
         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
         act: str = "none", out_scale: float = 1.0) -> torch.Tensor:
    """nm_spmm (nm_spmm_act with `act` != "none"): Y[R, T] =
    epilogue((mask . W) @ X) with X [K, T] (tokens contiguous); act "gelu"
    fuses GELU into the epilogue (int8 output: out_scale requantises it)."""
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a 2-D tensor with unit stride along T")
    if X.shape[0] != p.K:
        raise ValueError(f"X has {X.shape[0]} rows, the weight has K={p.K}")
    T = X.shape[1]
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else default_out_dtype(p.dtype)
    if out is None:
        out = torch.empty((p.rows, T), dtype=out_dtype, device=X.device)
    if out.dim() != 2 or out.stride(1) != 1 or tuple(out.shape) != (p.rows, T):
        raise ValueError("out must be [R, T] with unit stride along T")
    _check_operands(p, X, out, out_dtype, bias, scale, workspace)
    need = workspace_size(p, T, out_dtype)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    d = p.desc()
    st = lib().nm_spmm_act(ctypes.byref(d), X.data_ptr(), X.stride(0), T, out.data_ptr(), out.stride(0),
                           _TORCH_TO_NM[out_dtype], None if bias is None else bias.data_ptr(),
                           None if scale is None else scale.data_ptr(), ACTS[act], float(out_scale),
                           None if workspace is None else workspace.data_ptr(),
                           0 if workspace is None else workspace.numel() * workspace.element_size(),
                           _stream(X.device))
    _check(st, "nm_spmm_act" if act != "none" else "nm_spmm")
    return out


def spmm_noalloc(p: Packed, X: torch.Tensor, out: torch.Tensor, bias: torch.Tensor | None = None,
                 scale: torch.Tensor | None = None, act: str = "none", out_scale: float = 1.0) -> torch.Tensor:
    """nm_spmm_noalloc: spmm() into a caller-given `out` with no allocation
    at all (the library's per-device scratch replaces the workspace), for
    code that cannot allocate, such as HIP graph capture."""
    if X.dim() != 2 or X.stride(1) != 1 or X.shape[0] != p.K:
        raise ValueError("X must be [K, T] with unit stride along T")
    T = X.shape[1]
    if out.dim() != 2 or out.stride(1) != 1 or tuple(out.shape) != (p.rows, T):
        raise ValueError("out must be [R, T] with unit stride along T")
    _check_operands(p, X, out, out.dtype, bias, scale, None)
    d = p.desc()
    st = lib().nm_spmm_noalloc(ctypes.byref(d), X.data_ptr(), X.stride(0), T, out.data_ptr(), out.stride(0),
                               _TORCH_TO_NM[out.dtype], None if bias is None else bias.data_ptr(),
                               None if scale is None else scale.data_ptr(), ACTS[act], float(out_scale),
                               _stream(X.device))
    _check(st, "nm_spmm_noalloc")
    return out


def noalloc_max_bytes() -> int:
    return int(lib().nm_spmm_noalloc_max_bytes())


def linear(p: Packed, Xt: torch.Tensor, bias: torch.Tensor | None = None,
           scale: torch.Tensor | None = None, out_dtype: torch.dtype | None = None,
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
           act: str = "none", out_scale: float = 1.0) -> torch.Tensor:
    """nm_spmm_tk, the PyTorch-linear layout: Yt[T, R] = epilogue(Xt @ (mask . W)^T)
    with Xt [T, K] (K contiguous), as torch.nn.functional.linear takes it."""
    if Xt.dim() != 2 or Xt.stride(1) != 1:
        raise ValueError("Xt must be a 2-D tensor with unit stride along K")
    if Xt.shape[1] != p.K:
        raise ValueError(f"Xt has {Xt.shape[1]} columns, the weight has K={p.K}")
    T = Xt.shape[0]
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else default_out_dtype(p.dtype)
    if out is None:
        out = torch.empty((T, p.rows), dtype=out_dtype, device=Xt.device)
    if out.dim() != 2 or out.stride(1) != 1 or tuple(out.shape) != (T, p.rows):
        raise ValueError("out must be [T, R] with unit stride along R")
    _check_operands(p, Xt, out, out_dtype, bias, scale, workspace)
    need = workspace_size_tk(p, T, out_dtype)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=Xt.device)
    d = p.desc()
    st = lib().nm_spmm_tk(ctypes.byref(d), Xt.data_ptr(), Xt.stride(0), T, out.data_ptr(), out.stride(0),
                          _TORCH_TO_NM[out_dtype], None if bias is None else bias.data_ptr(),
                          None if scale is None else scale.data_ptr(), ACTS[act], float(out_scale),
                          None if workspace is None else workspace.data_ptr(),
                          0 if workspace is None else workspace.numel() * workspace.element_size(),
                          _stream(Xt.device))
    _check(st, "nm_spmm_tk")
    return out


# ---------------------------------------------------------------- three-layer format
@dataclass
class Hybrid:
    """A weight in the three-layer format (Sparse-TC 2:4, slot filling with
    PDD codes, CSR residual) as five uint8 buffers on one device."""
    rows: int
    K: int
    dtype: int
    values: torch.Tensor
    meta: torch.Tensor
    codes: torch.Tensor
    res_ptr: torch.Tensor
    res_ent: torch.Tensor | None
    n_fill: int
    n_res: int
    format_version: int = FORMAT_VERSION

    def desc(self) -> NmHybrid:
        d = NmHybrid()
        d.rows, d.K, d.dtype, d.format_version = self.rows, self.K, self.dtype, self.format_version
        d.n_fill, d.n_res = self.n_fill, self.n_res
        for name in HYBRID_BUFFERS:
            t = getattr(self, name)
            setattr(d, name, None if t is None else t.data_ptr())
            setattr(d, name + "_bytes", 0 if t is None else t.numel())
        return d

    @property
    def torch_dtype(self):
        return _NM_TO_TORCH[self.dtype]

    def nbytes(self) -> int:
        return sum(0 if getattr(self, n) is None else getattr(self, n).numel() for n in HYBRID_BUFFERS)


def hybrid_pack_host(W: torch.Tensor) -> Hybrid:
    """nm_hybrid_pack on the host: W (float16 / bfloat16, any device) is
    copied to host memory and packed there; the buffers are CPU tensors."""
    if W.dim() != 2:
        raise ValueError("W must be 2-D")
    dt = _TORCH_TO_NM.get(W.dtype)
    if dt not in (NM_F16, NM_BF16):
        raise TypeError(f"the three-layer format takes float16 / bfloat16 weights, not {W.dtype}")
    Wh = W.detach().to("cpu").contiguous()
    R, K = Wh.shape
    d = NmHybrid()
    _check(lib().nm_hybrid_pack_size(Wh.data_ptr(), K, R, K, dt, ctypes.byref(d)), "nm_hybrid_pack_size")
    bufs = {n: torch.empty(getattr(d, n + "_bytes"), dtype=torch.uint8) for n in HYBRID_BUFFERS}
    h = Hybrid(R, K, dt, bufs["values"], bufs["meta"], bufs["codes"], bufs["res_ptr"],
               bufs["res_ent"] if d.n_res else None, d.n_fill, d.n_res, 0)
    dd = h.desc()
    _check(lib().nm_hybrid_pack(Wh.data_ptr(), K, ctypes.byref(dd)), "nm_hybrid_pack")
    h.format_version = dd.format_version
    return h


def pack_hybrid(W: torch.Tensor, device=None) -> Hybrid:
    """Pack W into the three-layer format (host packer, offline) and place the
    buffers on `device` (default: W's device, which must be a GPU)."""
    device = torch.device(device) if device is not None else W.device
    if device.type != "cuda":
        raise ValueError(f"target device {device} is not a GPU")
    h = hybrid_pack_host(W)
    for n in HYBRID_BUFFERS:
        t = getattr(h, n)
        if t is not None:
            setattr(h, n, t.to(device))
    return h


def spmm_hybrid(h: Hybrid, X: torch.Tensor, bias: torch.Tensor | None = None,
                out_dtype: torch.dtype | None = None, out: torch.Tensor | None = None,
                act: str = "none") -> torch.Tensor:
    """nm_hybrid_spmm: Y[R, T] = epilogue(W @ X) for a three-layer weight,
    X [K, T] (tokens contiguous)."""
    if X.dim() != 2 or X.stride(1) != 1 or X.shape[0] != h.K:
        raise ValueError("X must be [K, T] with unit stride along T")
    if X.dtype != h.torch_dtype:
        raise TypeError(f"X is {X.dtype}, the weight is {h.torch_dtype}")
    T = X.shape[1]
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else h.torch_dtype
    if out is None:
        out = torch.empty((h.rows, T), dtype=out_dtype, device=X.device)
    if out.dim() != 2 or out.stride(1) != 1 or tuple(out.shape) != (h.rows, T) or out.dtype != out_dtype:
        raise ValueError("out must be [R, T] of out_dtype with unit stride along T")
    tensors = [X, out] + [getattr(h, n) for n in HYBRID_BUFFERS if getattr(h, n) is not None]
    if bias is not None:
        if bias.dtype != torch.float32 or bias.numel() != h.rows or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous float32 [R] tensor")
        tensors.append(bias)
    for t in tensors:
        if t.device != X.device:
            raise ValueError(f"operand on {t.device}, X on {X.device}")
    d = h.desc()
    st = lib().nm_hybrid_spmm(ctypes.byref(d), X.data_ptr(), X.stride(0), T, out.data_ptr(), out.stride(0),
                              _TORCH_TO_NM[out_dtype], None if bias is None else bias.data_ptr(),
                              ACTS[act], _stream(X.device))
    _check(st, "nm_hybrid_spmm")
    return out
