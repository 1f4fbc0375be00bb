"""The library's three-layer packer (host code, nm_hybrid_pack) against the
oracle's independent encoder: byte-identical images (CPU only; the library is
loaded but no GPU is touched).  Format: page "Accelerating GPU Inference of
Large Language Models with Moderately Unstructured Sparse Weight Matrices",
Methodology 1."""
import ctypes

import numpy as np
import pytest
import torch

import nm_inputs
import oracle
import semi_structured_sparse_nm_amd as nm


def _lib_image(W, dt):
    t = torch.from_numpy(np.ascontiguousarray(W).view(np.uint16).view(np.int16))
    t = t.view(torch.float16 if dt == "f16" else torch.bfloat16)
    h = nm.hybrid_pack_host(t)
    img = {n: (getattr(h, n).numpy() if getattr(h, n) is not None else np.zeros(0, np.uint8))
           for n in nm.HYBRID_BUFFERS}
    return h, img


def _same(h, img, ref):
    assert np.array_equal(img["values"], ref["values"])
    assert np.array_equal(img["meta"], ref["meta"])
    assert np.array_equal(img["codes"], ref["codes"])
    assert np.array_equal(img["res_ptr"].view(np.int32), ref["res_ptr"])
    assert np.array_equal(img["res_ent"].view(np.uint32), ref["res_ent"])
    assert h.n_res == len(ref["res_ent"])


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("R,K,dens", [(16, 64, 0.5), (37, 520, 0.5), (64, 1024, 0.3), (20, 700, 0.75),
                                      (1, 4, 1.0), (33, 4096, 0.5), (17, 8200, 0.5)])
def test_packer_matches_oracle(dt, R, K, dens):
    W = nm_inputs.unstructured(R, K, dens, dt, 0, "hypack", R, K)
    h, img = _lib_image(W, dt)
    ref = oracle.hy_encode(W, dt)
    _same(h, img, ref)
    # slot-filled count: nonzero codes
    nib = np.stack([ref["codes"] & 15, ref["codes"] >> 4], -1)
    assert h.n_fill == int((nib != 0).sum())


def test_packer_matches_oracle_structured_and_specials():
    W = nm_inputs.structured(48, 1536, 4, 8, "f16", 0, "hypack48").view(np.uint16).copy()
    rng = np.random.default_rng(3)
    pos = rng.choice(W.size, 200, replace=False)
    specials = np.array([0x7C00, 0xFC00, 0x7E00, 0x7C01, 0x8000, 0x0001, 0x3C00, 0xBC00], np.uint16)
    W.flat[pos] = specials[np.arange(200) % len(specials)]
    h, img = _lib_image(W, "f16")
    _same(h, img, oracle.hy_encode(W.view(np.float16), "f16"))


def test_packer_rejects_bad_shapes():
    d = nm.NmHybrid()
    W = np.zeros((4, 10), np.float16)
    st = nm.lib().nm_hybrid_pack_size(W.ctypes.data, 10, 4, 10, nm.NM_F16, ctypes.byref(d))
    assert st == nm.NM_EINVAL                                    # K % 4 != 0
    W = np.zeros((4, 8), np.int8)
    st = nm.lib().nm_hybrid_pack_size(W.ctypes.data, 8, 4, 8, nm.NM_I8, ctypes.byref(d))
    assert st == nm.NM_EUNSUPPORTED
    W = np.zeros((4, 8), np.float16)
    st = nm.lib().nm_hybrid_pack_size(W.ctypes.data, 4, 4, 8, nm.NM_F16, ctypes.byref(d))
    assert st == nm.NM_EINVAL                                    # ldw < K
