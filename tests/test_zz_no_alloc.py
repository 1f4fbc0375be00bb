"""nm_spmm_noalloc (the entry point that allocates nothing) against nm_spmm_act
with a caller-given workspace, through the C ABI, on the calls that use a
workspace: a K split across workgroups (Swin-T stage-4 MLP out-projection,
fp16 2:4), a 2:4 re-pack of an int8 1:4 weight (ViT-B FC1) and the two-layer
split of an int8 4:8 weight (ViT-B FC1).  Two calls in
a row, the second smaller; the results must be identical bit for bit (same
kernels, same split) and match the oracle.  A split whose partial sums exceed
the scratch is rejected before any launch."""
import ctypes
import os

import numpy as np
import pytest
import torch

import nm_inputs
import semi_structured_sparse_nm_amd as nm
from tests._parity import TORCH_DT, compare, dev, host, reference

pytestmark = pytest.mark.gpu


def _ws_call(p, X, T, out_t, b, s):
    """nm_spmm_act with its own workspace (the existing entry point)."""
    Y = torch.empty((p.rows, T), dtype=out_t, device="cuda")
    return nm.spmm(p, X, bias=b, scale=s, out_dtype=out_t, out=Y)


def _noalloc_call(p, X, T, out_t, b, s):
    Y = torch.empty((p.rows, T), dtype=out_t, device="cuda")
    d = p.desc()
    st = nm.lib().nm_spmm_noalloc(ctypes.byref(d), X.data_ptr(), X.stride(0), T, Y.data_ptr(), Y.stride(0),
                                  nm._TORCH_TO_NM[out_t], None if b is None else b.data_ptr(),
                                  None if s is None else s.data_ptr(), 0, 1.0,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == nm.NM_OK, nm.status_str(st)
    return Y


CASES = [
    # (what, R, K, T first, T second, N, M, dt, out, variant prefix)
    ("ksplit_swin_s4_fc2", 768, 3072, 1568, 784, 2, 4, "f16", "f16", "smfmac_h_2of4_persistent"),
    ("repack_vitb_fc1_1of4", 3072, 768, 12608, 6304, 1, 4, "i8", "i8", "repack24_"),
    ("split_vitb_fc1_4of8", 3072, 768, 12608, 6304, 4, 8, "i8", "i8", "split24_"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_entry(case):
    what, R, K, T1, T2, N, M, dt, out, vpre = case
    out_t = TORCH_DT[out]
    W = (nm_inputs.quant_layer(R, K, T1, N, M, 0, what).W if dt == "i8"
         else nm_inputs.normal((R, K), 0.02, dt, 0, what, "W"))
    p = nm.pack(dev(W, dt), N, M)
    for T in (T1, T2):
        if dt == "i8":
            q = nm_inputs.quant_layer(R, K, T, N, M, 0, what, T)
            Xh, bh, sh = q.X, q.bias, q.scale
        else:
            Xh = nm_inputs.normal((K, T), 1.0, dt, 0, what, "X", T)
            bh, sh = nm_inputs.normal((R,), 0.05, "f32", 0, what, "b"), None
        assert nm.variant(p, T, out_t).startswith(vpre)
        need = nm.workspace_size(p, T, out_t)
        assert 0 < need <= nm.noalloc_max_bytes()
        X = dev(Xh, dt)
        b = torch.from_numpy(np.asarray(bh)).cuda()
        s = None if sh is None else torch.from_numpy(np.asarray(sh, np.float32)).cuda()
        Yw = _ws_call(p, X, T, out_t, b, s)
        Yn = _noalloc_call(p, X, T, out_t, b, s)
        torch.cuda.synchronize()
        yw, yn = host(Yw, out), host(Yn, out)
        assert np.array_equal(np.asarray(yw).view(np.uint8), np.asarray(yn).view(np.uint8)), f"{what} T={T}"
        rows = np.arange(0, R, 5)
        ref = reference(W, Xh, N, M, dt, out, bias=bh, scale=sh, rows=rows)
        compare(np.asarray(yn)[rows], ref, out, f"{what} T={T}")


def test_noalloc_rejects_a_split_beyond_the_scratch():
    """A forced 16-way K split of a 768 x 8192 fp16 weight at T = 1568 needs
    16 * 768 * 1568 * 4 B = 77 MB of partial sums: NM_EINVAL, and the output
    is left as it was (nothing launched)."""
    R, K, T = 768, 8192, 1568
    W = nm_inputs.normal((R, K), 0.02, "f16", 1, "noalloc-big", "W")
    p = nm.pack(dev(W, "f16"), 2, 4)
    X = dev(nm_inputs.normal((K, T), 1.0, "f16", 1, "noalloc-big", "X"), "f16")
    old = os.environ.get("NM_SPMM_VARIANT")
    os.environ["NM_SPMM_VARIANT"] = "smfmac_h_2of4_persistent:16"
    try:
        assert nm.ksplit(p, T, torch.float16) == 16
        assert nm.workspace_size(p, T, torch.float16) > nm.noalloc_max_bytes()
        Y = torch.full((R, T), 3.0, dtype=torch.float16, device="cuda")
        d = p.desc()
        st = nm.lib().nm_spmm_noalloc(ctypes.byref(d), X.data_ptr(), T, T, Y.data_ptr(), T, nm.NM_F16, None, None,
                                      0, 1.0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        assert st == nm.NM_EINVAL
        assert bool((Y == 3.0).all())
    finally:
        if old is None:
            os.environ.pop("NM_SPMM_VARIANT", None)
        else:
            os.environ["NM_SPMM_VARIANT"] = old
