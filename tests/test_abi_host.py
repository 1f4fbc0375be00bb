"""Host-side checks of the C ABI (no GPU needed).

 - the shared library loads and exports every function include/nm_sparse.h
   declares;
 - nm_pack_size matches the packed layout's size formulas;
 - every documented validation error is returned before anything is launched
   (the arguments are rejected on the host, so no device is touched).
"""
import ctypes
import os
import re

import pytest

import semi_structured_sparse_nm_amd as nm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nm_sparse.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nm_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert {"nm_pack", "nm_spmm", "nm_pack_size", "nm_spmm_workspace_size",
            "nm_status_str"} <= set(names)
    L = nm.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in the header but not exported"


def test_status_strings_cover_every_code():
    for s in (nm.NM_OK, nm.NM_EINVAL, nm.NM_EUNSUPPORTED, nm.NM_EHIP):
        assert nm.status_str(s).startswith("NM_")
    assert nm.status_str(99) == "unknown nm_status"


@pytest.mark.parametrize("dt,eb", [(nm.NM_I8, 1), (nm.NM_F16, 2), (nm.NM_BF16, 2)])
@pytest.mark.parametrize("N,M", [(1, 4), (2, 4), (3, 4), (4, 4), (1, 8), (2, 8), (3, 8), (4, 8), (8, 8)])
@pytest.mark.parametrize("R,K", [(1, 8), (17, 96), (192, 192), (3072, 768), (4096, 11008)])
def test_pack_size_formula(dt, eb, N, M, R, K):
    vb, mb = nm.pack_size(R, K, N, M, dt)
    KB = 128 // eb
    C = KB // M * N
    w = 0 if N == M else {4: 2, 8: 3}[M]
    MR = (C * w + 7) // 8
    MR = (MR + 3) // 4 * 4
    nblk = -(-R // 16) * -(-K // KB)
    assert vb == nblk * 16 * C * eb
    assert mb == nblk * 16 * MR


@pytest.mark.parametrize("args,want", [
    ((0, 8, 2, 4, nm.NM_I8), nm.NM_EINVAL),        # rows < 1
    ((4, 0, 2, 4, nm.NM_I8), nm.NM_EINVAL),        # K < 1
    ((4, 8, 0, 4, nm.NM_I8), nm.NM_EINVAL),        # N < 1
    ((4, 8, 5, 4, nm.NM_I8), nm.NM_EINVAL),        # N > M
    ((4, 10, 2, 4, nm.NM_I8), nm.NM_EINVAL),       # K % M
    ((4, 12, 2, 6, nm.NM_I8), nm.NM_EUNSUPPORTED),  # M not in {4, 8}
    ((4, 16, 2, 16, nm.NM_I8), nm.NM_EUNSUPPORTED),
    ((4, 8, 2, 4, nm.NM_I32), nm.NM_EUNSUPPORTED),  # weight dtype
    ((4, 8, 2, 4, 17), nm.NM_EUNSUPPORTED),
])
def test_pack_size_errors(args, want):
    vb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    assert nm.lib().nm_pack_size(*args, ctypes.byref(vb), ctypes.byref(mb)) == want
    assert nm.lib().nm_pack_size(4, 8, 2, 4, nm.NM_I8, None, ctypes.byref(mb)) == nm.NM_EINVAL


# Fake, well-aligned device addresses: every case below is rejected on the
# host before a launch, so they are never dereferenced.
FAKE = 0x7f0000000000


def _desc(R=32, K=64, N=2, M=4, dt=nm.NM_I8, **kw):
    vb, mb = nm.pack_size(R, K, N, M, dt)
    d = nm.NmPacked()
    d.rows, d.K, d.N, d.M, d.dtype = R, K, N, M, dt
    d.format_version = nm.FORMAT_VERSION
    d.values, d.values_bytes = FAKE, vb
    d.meta, d.meta_bytes = (FAKE + (1 << 24), mb) if mb else (None, 0)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _spmm(d, X=FAKE + (2 << 24), ldx=100, T=100, Y=FAKE + (3 << 24), ldy=100, ydt=nm.NM_I32,
          bias=None, scale=None, ws=None, wsb=0):
    return nm.lib().nm_spmm(ctypes.byref(d), X, ldx, T, Y, ldy, ydt, bias, scale, ws, wsb, None)


def test_spmm_validation_errors():
    L = nm.lib()
    ok = _desc()
    assert L.nm_spmm(None, FAKE, 1, 1, FAKE, 1, nm.NM_I32, None, None, None, 0, None) == nm.NM_EINVAL
    assert _spmm(ok, X=None) == nm.NM_EINVAL
    assert _spmm(ok, Y=None) == nm.NM_EINVAL
    assert _spmm(ok, T=0) == nm.NM_EINVAL
    assert _spmm(ok, ldx=99) == nm.NM_EINVAL
    assert _spmm(ok, ldy=99) == nm.NM_EINVAL
    assert _spmm(ok, ydt=nm.NM_I8) == nm.NM_EINVAL            # scale required for int8 output
    assert _spmm(ok, ydt=nm.NM_F16) == nm.NM_EUNSUPPORTED    # int8 weights -> fp16 not provided
    assert _spmm(ok, ydt=99) == nm.NM_EUNSUPPORTED
    assert _spmm(_desc(values_bytes=ok.values_bytes + 1)) == nm.NM_EINVAL
    assert _spmm(_desc(meta_bytes=0)) == nm.NM_EINVAL
    assert _spmm(_desc(meta=None)) == nm.NM_EINVAL
    assert _spmm(_desc(values=None)) == nm.NM_EINVAL
    assert _spmm(_desc(format_version=0)) == nm.NM_EINVAL
    bad = _desc()
    bad.N = 5
    assert _spmm(bad) == nm.NM_EINVAL
    bad = _desc()
    bad.M = 6
    assert _spmm(bad) == nm.NM_EUNSUPPORTED
    assert _spmm(_desc(values=FAKE + 8)) == nm.NM_EUNSUPPORTED  # packed buffers need 16 B alignment
    f16 = _desc(dt=nm.NM_F16)
    assert _spmm(f16, ydt=nm.NM_F16, X=FAKE + 1) == nm.NM_EUNSUPPORTED  # X not 2-byte aligned
    assert _spmm(f16, ydt=nm.NM_F32, Y=FAKE + 2) == nm.NM_EUNSUPPORTED  # Y not 4-byte aligned
    assert _spmm(f16, ydt=nm.NM_BF16) == nm.NM_EUNSUPPORTED


def test_pack_validation_errors():
    L = nm.lib()
    d = _desc(format_version=0)
    assert L.nm_pack(None, 64, ctypes.byref(d), None) == nm.NM_EINVAL
    assert L.nm_pack(FAKE, 64, None, None) == nm.NM_EINVAL
    assert L.nm_pack(FAKE, 63, ctypes.byref(d), None) == nm.NM_EINVAL          # ldw < K
    bad = _desc(values_bytes=d.values_bytes - 1, format_version=0)
    assert L.nm_pack(FAKE, 64, ctypes.byref(bad), None) == nm.NM_EINVAL
    f16 = _desc(dt=nm.NM_F16, format_version=0)
    assert L.nm_pack(FAKE + 1, 64, ctypes.byref(f16), None) == nm.NM_EUNSUPPORTED
    assert d.format_version == 0   # untouched on error


def test_workspace_and_variant_queries():
    L = nm.lib()
    d = _desc()
    n = ctypes.c_size_t(123)
    assert L.nm_spmm_workspace_size(ctypes.byref(d), 100, nm.NM_I32, ctypes.byref(n)) == nm.NM_OK
    assert L.nm_spmm_workspace_size(ctypes.byref(d), 0, nm.NM_I32, ctypes.byref(n)) == nm.NM_EINVAL
    assert L.nm_spmm_workspace_size(ctypes.byref(d), 100, nm.NM_I32, None) == nm.NM_EINVAL
    assert L.nm_spmm_variant(ctypes.byref(d), 100, nm.NM_I32).decode() != "invalid"
    assert L.nm_spmm_variant(ctypes.byref(d), 0, nm.NM_I32).decode() == "invalid"
    assert L.nm_spmm_variant(None, 100, nm.NM_I32).decode() == "invalid"


def _ksplit(d, T, ydt, act=0):
    return nm.lib().nm_spmm_ksplit(ctypes.byref(d), T, ydt, act)


def _ws(d, T, ydt):
    n = ctypes.c_size_t()
    assert nm.lib().nm_spmm_workspace_size(ctypes.byref(d), T, ydt, ctypes.byref(n)) == nm.NM_OK
    return n.value


def test_ksplit_choice_and_workspace(monkeypatch):
    """K split across workgroups: chosen for deep-K shapes with few output
    tiles, never for shapes that fill the GPU; the workspace query reports
    the slices' partial sums; NM_SPMM_VARIANT=":<S>" forces a divisor of the column
    blocks or turns the split off."""
    # Swin-T stage-4 MLP out-projection, fp16 2:4: 39 tiles, 48 column blocks
    deep = _desc(R=768, K=3072, dt=nm.NM_F16)
    S = _ksplit(deep, 1568, nm.NM_F16)
    assert S > 1 and 48 % S == 0 and 48 // S >= 4
    assert _ws(deep, 1568, nm.NM_F16) == S * 768 * 1568 * 4
    # same for the dense-expand kernel (1:4)
    deep14 = _desc(R=768, K=3072, N=1, M=4, dt=nm.NM_F16)
    assert _ksplit(deep14, 1568, nm.NM_F16) > 1
    # ViT-B FC1 int8 2:4 at batch 64 fills the GPU: no split, no workspace
    wide = _desc(R=3072, K=768)
    assert _ksplit(wide, 12608, nm.NM_I8) == 1 and _ws(wide, 12608, nm.NM_I8) == 0
    # decode shapes split K inside a workgroup instead
    assert _ksplit(deep, 16, nm.NM_F16) == 1
    assert _ksplit(deep, 0, nm.NM_F16) == 0
    monkeypatch.setenv("NM_SPMM_VARIANT", ":3")
    assert _ksplit(deep, 1568, nm.NM_F16) == 3
    assert _ws(deep, 1568, nm.NM_F16) == 3 * 768 * 1568 * 4
    monkeypatch.setenv("NM_SPMM_VARIANT", ":5")     # does not divide 48 blocks
    assert _ksplit(deep, 1568, nm.NM_F16) == 1
    monkeypatch.setenv("NM_SPMM_VARIANT", ":1")
    assert _ksplit(deep, 1568, nm.NM_F16) == 1 and _ws(deep, 1568, nm.NM_F16) == 0


def test_split_call_validates_its_workspace(monkeypatch):
    monkeypatch.setenv("NM_SPMM_VARIANT", ":4")
    d = _desc(R=768, K=3072, dt=nm.NM_F16)
    need = _ws(d, 1568, nm.NM_F16)
    assert need == 4 * 768 * 1568 * 4
    kw = dict(T=1568, ldx=1568, ldy=1568, ydt=nm.NM_F16)
    assert _spmm(d, **kw) == nm.NM_EINVAL                                      # none given
    assert _spmm(d, ws=FAKE + (4 << 24), wsb=need - 1, **kw) == nm.NM_EINVAL   # too small
    assert _spmm(d, ws=FAKE + (4 << 24) + 8, wsb=need, **kw) == nm.NM_EUNSUPPORTED  # misaligned


def _spmm_act(d, act, out_scale=1.0, X=FAKE + (2 << 24), ldx=100, T=100, Y=FAKE + (3 << 24), ldy=100,
              ydt=nm.NM_I8, scale=FAKE + (5 << 24)):
    return nm.lib().nm_spmm_act(ctypes.byref(d), X, ldx, T, Y, ldy, ydt, None, scale, act, out_scale,
                                None, 0, None)


def test_activation_validation_and_variant_choice():
    """nm_spmm_act rejects unknown activations, an activation on raw int32
    accumulators and a non-finite output scale before any launch; the
    activation leaves the kernel choice as it is (every default kernel
    carries it)."""
    d = _desc()
    assert _spmm_act(d, 2) == nm.NM_EUNSUPPORTED
    assert _spmm_act(d, -1) == nm.NM_EUNSUPPORTED
    assert _spmm_act(d, 1, ydt=nm.NM_I32) == nm.NM_EUNSUPPORTED
    assert _spmm_act(d, 1, out_scale=float("inf")) == nm.NM_EINVAL
    assert _spmm_act(d, 1, out_scale=float("nan")) == nm.NM_EINVAL
    assert _spmm_act(d, 1, ydt=nm.NM_I8, scale=None) == nm.NM_EINVAL
    L = nm.lib()
    va = lambda d, T, y, a: L.nm_spmm_variant_act(ctypes.byref(d), T, y, a).decode()
    fc1 = _desc(R=3072, K=768)
    assert va(fc1, 12608, nm.NM_I8, 0) == "smfmac_i8_2of4_stationary"
    assert va(fc1, 12608, nm.NM_I8, 1) == "smfmac_i8_2of4_stationary"
    assert va(_desc(R=768, K=768), 12608, nm.NM_I8, 1) == "smfmac_i8_2of4_persistent_w8"
    deep = _desc(R=3072, K=3072, N=1, M=4)
    assert va(deep, 12608, nm.NM_I8, 1) == "repack24_smfmac_i8_2of4_persistent"
    assert va(_desc(R=3072, K=3072, N=4, M=8), 12608, nm.NM_I8, 1) == "expand_mfma_persistent"
    assert va(fc1, 12608, nm.NM_I32, 1) == "invalid"
    assert va(fc1, 12608, nm.NM_I8, 7) == "invalid"
    assert L.nm_spmm_variant(ctypes.byref(fc1), 12608, nm.NM_I8).decode() == va(fc1, 12608, nm.NM_I8, 0)
    f16 = _desc(R=3072, K=768, dt=nm.NM_F16)
    assert va(f16, 1568, nm.NM_F16, 1) == "smfmac_h_2of4_persistent"
    assert va(f16, 16, nm.NM_F16, 1) == "smfmac_h_2of4_decode"


def test_tk_layout_validation():
    """nm_spmm_tk checks its strides against K and R (not T) before any
    launch and shares nm_spmm_act's other checks."""
    L = nm.lib()
    d = _desc(R=32, K=64)

    def tk(ldx=64, T=100, ldy=32, ydt=nm.NM_I32, act=0, X=FAKE + (2 << 24), Y=FAKE + (3 << 24)):
        return L.nm_spmm_tk(ctypes.byref(d), X, ldx, T, Y, ldy, ydt, None, None, act, 1.0, None, 0, None)

    assert tk(ldx=63) == nm.NM_EINVAL
    assert tk(ldy=31) == nm.NM_EINVAL
    assert tk(T=0) == nm.NM_EINVAL
    assert tk(X=None) == nm.NM_EINVAL
    assert tk(act=1) == nm.NM_EUNSUPPORTED          # activation on raw int32
    assert tk(ydt=nm.NM_I8) == nm.NM_EINVAL         # scale required
    assert L.nm_spmm_variant_tk(ctypes.byref(d), 100, nm.NM_I32, 0).decode() == "smfmac_i8_2of4_tk"
    # rows not a multiple of 16, other N:M and fp weights take the generic kernel
    for other in (_desc(R=33, K=64), _desc(R=32, K=64, N=1, M=4), _desc(R=32, K=64, dt=nm.NM_F16)):
        y = nm.NM_F16 if other.dtype == nm.NM_F16 else nm.NM_I32
        assert L.nm_spmm_variant_tk(ctypes.byref(other), 100, y, 0).decode() == "generic_dense_expand"


def test_int8_workgroup_size_choice():
    """int8 2:4 (256 CUs assumed without a GPU), the ViT-B shapes at batch
    64: the weight-stationary kernel for K in (640, 768] with at least 3.5
    token steps per CU; else 8-wave persistent workgroups unless the 4-wave
    kernel's 256 x 128 tiles number at least four per CU."""
    L = nm.lib()
    v = lambda R, K, T: L.nm_spmm_variant(ctypes.byref(_desc(R=R, K=K)), T, nm.NM_I8).decode()
    assert v(3072, 768, 12608) == "smfmac_i8_2of4_stationary"        # FC1: 4.6 steps per CU
    assert v(2304, 768, 12608) == "smfmac_i8_2of4_stationary"        # QKV: 3.8
    assert v(768, 3072, 12608) == "smfmac_i8_2of4_persistent_w8"     # FC2: K past 768
    assert v(768, 768, 12608) == "smfmac_i8_2of4_persistent_w8"      # proj: 1.5 steps, 297 tiles
    assert v(3072, 768, 4096) == "smfmac_i8_2of4_persistent_w8"      # 1.5 steps: 384 tiles
    assert v(3072, 640, 12608) == "smfmac_i8_2of4_persistent"        # K 640: five column blocks
    assert v(16896, 768, 12608) == "smfmac_i8_2of4_persistent"       # 33 row tiles > 32 per XCD


@pytest.mark.parametrize("N,M", [(1, 4), (1, 8), (2, 8)])
def test_repack24_choice_and_workspace(monkeypatch, N, M):
    """1:4, 1:8 and 2:8 int8 products large enough (R K T >= 2^31) run
    re-packed to 2:4 on the sparse-MFMA tile kernels and ask for the 2:4
    copy's workspace; small products, fp16 weights (unless forced), N:M
    outside 2:4 and a forced N:M kernel do not."""
    monkeypatch.delenv("NM_SPMM_VARIANT", raising=False)
    L = nm.lib()

    def q(d, T, ydt):
        n = ctypes.c_size_t()
        assert L.nm_spmm_workspace_size(ctypes.byref(d), T, ydt, ctypes.byref(n)) == nm.NM_OK
        return L.nm_spmm_variant(ctypes.byref(d), T, ydt).decode(), n.value, \
            L.nm_spmm_ksplit(ctypes.byref(d), T, ydt, 0)

    def copy_bytes(R, K, dt):
        vb, mb = nm.pack_size(R, K, 2, 4, dt)
        return (vb + 255) // 256 * 256 + mb

    fc1 = _desc(R=3072, K=768, N=N, M=M)
    assert q(fc1, 12608, nm.NM_I8) == ("repack24_smfmac_i8_2of4_stationary", copy_bytes(3072, 768, nm.NM_I8), 1)
    fc2 = _desc(R=768, K=3072, N=N, M=M)
    assert q(fc2, 12608, nm.NM_I8) == ("repack24_smfmac_i8_2of4_persistent_w8", copy_bytes(768, 3072, nm.NM_I8), 1)
    h = _desc(R=3072, K=768, N=N, M=M, dt=nm.NM_F16)
    assert q(h, 3136, nm.NM_F16)[:2] == ("expand_mfma_persistent", 0)         # fp16: not by default
    assert q(fc1, 256, nm.NM_I8)[:2] == ("expand_mfma_persistent", 0)        # R K T < 2^31
    assert q(fc1, 16, nm.NM_I8)[:2] == ("expand_mfma_decode", 0)
    tk = lambda d, T: L.nm_spmm_variant_tk(ctypes.byref(d), T, nm.NM_I8, 0).decode()
    assert tk(fc1, 12608) == "repack24_smfmac_i8_2of4_stationary_tk"
    assert tk(fc1, 256) == "transpose_expand_mfma_persistent"               # below the re-pack size
    monkeypatch.setenv("NM_SPMM_VARIANT", "expand_mfma_persistent")
    assert q(fc1, 12608, nm.NM_I8)[:2] == ("expand_mfma_persistent", 0)
    monkeypatch.setenv("NM_SPMM_VARIANT", "repack24_smfmac_i8_2of4_persistent")
    assert q(fc1, 256, nm.NM_I8)[:2] == ("repack24_smfmac_i8_2of4_persistent", copy_bytes(3072, 768, nm.NM_I8))
    monkeypatch.setenv("NM_SPMM_VARIANT", "repack24_smfmac_h_2of4_persistent")
    assert q(h, 3136, nm.NM_F16) == ("repack24_smfmac_h_2of4_persistent", copy_bytes(3072, 768, nm.NM_F16), 1)


def _split_bytes(R, K):
    """Workspace of the two-layer split: two 2:4 copies (values, then meta at
    the next 256-byte boundary), each rounded up to 256 bytes."""
    vb, mb = nm.pack_size(R, K, 2, 4, nm.NM_I8)
    return 2 * (((vb + 255) // 256 * 256 + mb + 255) // 256 * 256)


@pytest.mark.parametrize("N,M", [(4, 4), (8, 8)])
def test_dense24_choice(monkeypatch, N, M):
    """Dense int8 weights (N = M), K in (640, 768], large enough: the
    two-layer kernel with the layers taken in registers, no workspace;
    otherwise not."""
    monkeypatch.delenv("NM_SPMM_VARIANT", raising=False)
    L = nm.lib()
    v = lambda d, T, y=nm.NM_I8: L.nm_spmm_variant(ctypes.byref(d), T, y).decode()
    for R in (3072, 2304, 768):
        d = _desc(R=R, K=768, N=N, M=M)
        assert v(d, 12608) == v(d, 12608, nm.NM_I32) == "dense24_smfmac_i8_stationary"
        assert _ws(d, 12608, nm.NM_I8) == 0
    assert v(_desc(R=768, K=3072, N=N, M=M), 12608) != "dense24_smfmac_i8_stationary"
    assert v(_desc(R=3072, K=768, N=N, M=M), 256) != "dense24_smfmac_i8_stationary"
    tk = L.nm_spmm_variant_tk(ctypes.byref(_desc(R=3072, K=768, N=N, M=M)), 12608, nm.NM_I8, 0).decode()
    assert tk == "dense24_smfmac_i8_stationary_tk"
    monkeypatch.setenv("NM_SPMM_VARIANT", "dense24_smfmac_i8_stationary")
    assert v(_desc(R=40, K=768, N=N, M=M), 64) == "dense24_smfmac_i8_stationary"
    assert v(_desc(R=40, K=768, N=4, M=8), 64) != "dense24_smfmac_i8_stationary"   # not dense


@pytest.mark.parametrize("N,M", [(3, 4), (3, 8), (4, 8), (7, 8)])
def test_split24_choice_and_workspace(monkeypatch, N, M):
    """int8 N:M with more than two kept members per group of four, K in
    (640, 768], large enough (R K T >= 2^31): split into two 2:4 layers and
    the weight-stationary kernel over both, with the two copies' workspace;
    deeper K, small products, fp16 weights, decode shapes, more than 256
    row tiles and the [T][K] layout do not; forcing works on any N:M (1:4
    included)."""
    monkeypatch.delenv("NM_SPMM_VARIANT", raising=False)
    L = nm.lib()
    v = lambda d, T, y=nm.NM_I8: L.nm_spmm_variant(ctypes.byref(d), T, y).decode()
    split = "split24_smfmac_i8_stationary"
    for R in (3072, 2304, 768):                          # ViT-B FC1, QKV, proj
        d = _desc(R=R, K=768, N=N, M=M)
        assert v(d, 12608) == split
        assert v(d, 12608, nm.NM_I32) == split
        assert _ws(d, 12608, nm.NM_I8) == _split_bytes(R, 768)
        assert L.nm_spmm_ksplit(ctypes.byref(d), 12608, nm.NM_I8, 0) == 1
    assert v(_desc(R=3072, K=704, N=N, M=M), 12608) == split          # six column blocks, the last partial
    assert v(_desc(R=768, K=3072, N=N, M=M), 12608) != split   # FC2: K past 768
    assert v(_desc(R=3072, K=640, N=N, M=M), 12608) != split   # five column blocks
    assert v(_desc(R=3072, K=768, N=N, M=M), 256) != split     # R K T < 2^31
    assert v(_desc(R=3072, K=768, N=N, M=M), 16) != split
    assert v(_desc(R=3072, K=768, N=N, M=M, dt=nm.NM_F16), 12608, nm.NM_F16) != split
    assert v(_desc(R=65792, K=768, N=N, M=M), 4096) != split   # 257 row tiles
    tk = L.nm_spmm_variant_tk(ctypes.byref(_desc(R=3072, K=768, N=N, M=M)), 12608, nm.NM_I8, 0).decode()
    assert tk == split + "_tk"
    monkeypatch.setenv("NM_SPMM_VARIANT", split)
    small = _desc(R=40, K=768, N=1, M=4)
    assert v(small, 64) == split
    assert _ws(small, 64, nm.NM_I8) == _split_bytes(40, 768)
    assert v(_desc(R=40, K=1024, N=N, M=M), 64) != split                # K past 768: not eligible


def test_tk_transpose_choice_and_workspace(monkeypatch):
    """Large [T][K] calls without a kernel of their own in that layout run
    through the [K][T] kernels between two transposes, and ask for X', Y'
    (and split partials) in the workspace; small ones stay on the generic
    kernel."""
    monkeypatch.delenv("NM_SPMM_VARIANT", raising=False)
    L = nm.lib()
    tk = lambda d, T, y: L.nm_spmm_variant_tk(ctypes.byref(d), T, y, 0).decode()

    def ws(d, T, y):
        n = ctypes.c_size_t()
        assert L.nm_spmm_tk_workspace_size(ctypes.byref(d), T, y, ctypes.byref(n)) == nm.NM_OK
        return n.value

    r256 = lambda n: (n + 255) // 256 * 256
    d48 = _desc(R=3072, K=768, N=4, M=8)
    # int8 4:8 at K 768: the two-layer kernel of the layout (its split copy)
    assert tk(d48, 12608, nm.NM_I8) == "split24_smfmac_i8_stationary_tk"
    assert ws(d48, 12608, nm.NM_I8) == _split_bytes(3072, 768)
    d48k = _desc(R=768, K=3072, N=4, M=8)                   # K past 768: through the [K][T] kernel
    assert tk(d48k, 12608, nm.NM_I8) == "transpose_expand_mfma_persistent"
    assert ws(d48k, 12608, nm.NM_I8) == r256(3072 * 12608) + r256(768 * 12608)
    h = _desc(R=3072, K=768, dt=nm.NM_F16)
    assert tk(h, 3137, nm.NM_F16) == "transpose_smfmac_h_2of4_persistent"
    assert ws(h, 3137, nm.NM_F16) == r256(768 * 3152 * 2) + r256(3072 * 3152 * 2)
    assert tk(_desc(R=192, K=192, N=4, M=8), 197, nm.NM_I32) == "generic_dense_expand"
    assert tk(_desc(R=3072, K=768), 12608, nm.NM_I8) == "smfmac_i8_2of4_stationary_tk"
    assert tk(_desc(R=768, K=768), 12608, nm.NM_I8) == "smfmac_i8_2of4_tk"      # proj: 1.5 steps per CU
    assert tk(_desc(R=768, K=3072), 12608, nm.NM_I8) == "smfmac_i8_2of4_tk"     # FC2: K past 768
    assert ws(_desc(R=3072, K=768), 12608, nm.NM_I8) == 0
    # the [K][T] query: no transposes, the two-layer split of the 4:8 weight
    assert _ws(d48, 12608, nm.NM_I8) == _split_bytes(3072, 768)
    monkeypatch.setenv("NM_SPMM_VARIANT", "generic_dense_expand")
    assert tk(d48, 12608, nm.NM_I8) == "generic_dense_expand"


def test_tk_workspace_size_validation():
    """nm_spmm_tk_workspace_size checks its arguments like the [K][T] query."""
    L = nm.lib()
    d = _desc(R=3072, K=768, N=4, M=8)
    n = ctypes.c_size_t()
    assert L.nm_spmm_tk_workspace_size(ctypes.byref(d), 12608, nm.NM_I8, None) == nm.NM_EINVAL
    assert L.nm_spmm_tk_workspace_size(ctypes.byref(d), 0, nm.NM_I8, ctypes.byref(n)) == nm.NM_EINVAL
    assert L.nm_spmm_tk_workspace_size(ctypes.byref(d), 16, nm.NM_F16, ctypes.byref(n)) == nm.NM_EUNSUPPORTED
    assert L.nm_spmm_tk_workspace_size(None, 16, nm.NM_I8, ctypes.byref(n)) == nm.NM_EINVAL
    assert L.nm_spmm_tk_workspace_size(ctypes.byref(_desc(R=64, K=64, N=4, M=8)), 16, nm.NM_I8,
                                       ctypes.byref(n)) == nm.NM_OK and n.value == 0


def test_binding_rejects_mismatched_operands_before_any_call(monkeypatch):
    """spmm() / linear() check dtypes, lengths and devices before touching the
    library: a mismatch raises TypeError / ValueError and nothing is launched
    (the library handle is poisoned here, so any call would fail loudly)."""
    import torch
    import semi_structured_sparse_nm_amd as nm

    def no_call():
        raise AssertionError("the library was called")

    monkeypatch.setattr(nm, "lib", no_call)
    R, K, T = 16, 64, 8
    vb, mb = 16 * 64 // 2 * 2, 16 * 16 // 1
    p16 = nm.Packed(R, K, 2, 4, nm.NM_F16, torch.empty(vb, dtype=torch.uint8),
                    torch.empty(mb, dtype=torch.uint8), nm.FORMAT_VERSION)
    p8 = nm.Packed(R, K, 2, 4, nm.NM_I8, torch.empty(vb // 2, dtype=torch.uint8),
                   torch.empty(mb, dtype=torch.uint8), nm.FORMAT_VERSION)
    X16 = torch.zeros((K, T), dtype=torch.float16)
    X8 = torch.zeros((K, T), dtype=torch.int8)
    with pytest.raises(TypeError):
        nm.spmm(p16, X8)                                             # activation dtype
    with pytest.raises(TypeError):
        nm.spmm(p16, torch.zeros((K, T), dtype=torch.float32))
    with pytest.raises(TypeError):
        nm.spmm(p8, X8, out=torch.empty((R, T), dtype=torch.int8), out_dtype=torch.int32,
                scale=torch.ones(R))                                 # out tensor vs out dtype
    with pytest.raises(TypeError):
        nm.spmm(p16, X16, bias=torch.zeros(R, dtype=torch.float16))  # fp bias must be float32
    with pytest.raises(TypeError):
        nm.spmm(p8, X8, bias=torch.zeros(R, dtype=torch.float32))    # int8 bias must be int32
    with pytest.raises(ValueError):
        nm.spmm(p16, X16, bias=torch.zeros(R - 1, dtype=torch.float32))
    with pytest.raises(TypeError):
        nm.spmm(p8, X8, out_dtype=torch.int8, scale=torch.ones(R, dtype=torch.float64))
    with pytest.raises(ValueError):
        nm.spmm(p8, X8, out_dtype=torch.int8, scale=torch.ones(R + 3))
    with pytest.raises(ValueError):
        nm.spmm(p8, X8, out_dtype=torch.int8)                        # int8 output needs a scale
    with pytest.raises(ValueError):
        nm.spmm(p16, X16)                                            # weights not on a GPU
    with pytest.raises(TypeError):
        nm.linear(p16, torch.zeros((T, K), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        nm.linear(p16, torch.zeros((T, K), dtype=torch.float16), bias=torch.zeros(2 * R))
    with pytest.raises(ValueError):
        nm.pack(torch.zeros((R, K), dtype=torch.float16), 2, 4)      # W not on a GPU
