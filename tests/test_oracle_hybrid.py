"""Pins of the oracle's three-layer format encoder and reader (CPU only).

The format: a Sparse-TC 2:4 layer with 2-bit positions, a Slot-Filling layer
whose elements sit in the 2:4 layer's empty slots with 4-bit relative
distances (PDD) and dummy points for long gaps, and a CSR residual layer
(page "Accelerating GPU Inference of Large Language Models with Moderately
Unstructured Sparse Weight Matrices", Methodology 1).  What pins it:
  - hand-worked byte images (golden/hybrid_images.txt): a PDD chain, a run of
    dummy points, slots exhausted into the residual, the sixteen-code cap;
  - round trip: the reader rebuilds every nonzero of W exactly, each one
    once, for random, ragged and non-finite inputs;
  - special case: for weights that already satisfy 2:4 the format is the
    2:4 packing (positions and values of the pinned 2:4 selection), with no
    slot-filled element and no residual;
  - counts: Sparse-TC + slot-filled + residual = nonzeros, no distance code
    above 15, at most sixteen codes per fill unit.
"""
import os

import numpy as np
import pytest

import oracle


def _f(v, dt):
    if dt == "f16":
        return int(np.array([v], np.float16).view(np.uint16)[0])
    return int(np.array([v], np.float32).view(np.uint32)[0] >> 16)   # exact for these values


def _cases(golden_dir):
    cur = None
    for raw in open(os.path.join(golden_dir, "hybrid_images.txt")):
        line = raw.split("#")[0].strip()
        if not line:
            continue
        t = line.split()
        if t[0] == "case":
            cur = dict(name=t[1], R=int(t[2]), K=int(t[3]), dt=t[4], w=[], slot=[], codes={}, res=[])
        elif t[0] == "w":
            cur["w"].append((int(t[1]), int(t[2]), float(t[3])))
        elif t[0] == "slot":
            cur["slot"].append(tuple(int(x) for x in t[1:5]) + (float(t[5]),))
        elif t[0] == "codes":
            cur["codes"][(int(t[1]), int(t[2]), int(t[3]))] = bytes.fromhex(t[4])
        elif t[0] == "res":
            cur["res"].append((int(t[1]), int(t[2]), float(t[3])))
        elif t[0] == "end":
            yield cur
            cur = None


def _slot(img, K, r, kb, c):
    nKB = (K + 63) // 64
    blk = (r // 16) * nKB + kb
    rr = r % 16
    v = int(img["values"][blk * 1024 + rr * 64 + 2 * c]) | (int(img["values"][blk * 1024 + rr * 64 + 2 * c + 1]) << 8)
    word = int.from_bytes(bytes(img["meta"][blk * 128 + rr * 8: blk * 128 + rr * 8 + 8]), "little")
    return (word >> (2 * c)) & 3, v


def test_golden_hybrid_images(golden_dir):
    n = 0
    for c in _cases(golden_dir):
        R, K, dt = c["R"], c["K"], c["dt"]
        W = np.zeros((R, K), np.uint16)
        for r, col, v in c["w"]:
            W[r, col] = _f(v, dt)
        img = oracle.hy_encode(W.view(np.float16) if dt == "f16" else W, dt)
        nRB, nKB, nSeg = oracle.hy_geometry(R, K)
        if c["slot"]:
            want = {(r, kb, s): (p, _f(v, dt)) for r, kb, s, p, v in c["slot"]}
            for r in range(R):
                for kb in range(nKB):
                    for s in range(32):
                        exp = want.get((r, kb, s), (1 if s % 2 == 0 else 0, 0))
                        assert _slot(img, K, r, kb, s) == exp, (c["name"], r, kb, s)
        for rb in range(nRB):
            for s in range(nSeg):
                for q in range(4):
                    for rr in range(16):
                        off = ((rb * nSeg + s) * 64 + 16 * q + rr) * 8
                        got = bytes(img["codes"][off:off + 8])
                        assert got == c["codes"].get((rb * 16 + rr, s, q), bytes(8)), (c["name"], rb, s, q, rr)
        # residual: exactly the listed entries, CSR over (row block, segment, row)
        got = []
        rp = img["res_ptr"]
        for rb in range(nRB):
            for s in range(nSeg):
                for rr in range(16):
                    z = (rb * nSeg + s) * 16 + rr
                    cols = []
                    for e in range(rp[z], rp[z + 1]):
                        ent = int(img["res_ent"][e])
                        cols.append(512 * s + (ent >> 16))
                        got.append((rb * 16 + rr, 512 * s + (ent >> 16), ent & 0xFFFF))
                    assert cols == sorted(cols)
        assert sorted(got) == sorted((r, col, _f(v, dt)) for r, col, v in c["res"]), c["name"]
        # and the image reads back to W
        assert np.array_equal(oracle.hy_read(img, R, K, dt), W), c["name"]
        n += 1
    assert n == 4


def _sparse(rng, R, K, dens, dt):
    W = (rng.standard_normal((R, K)) * 0.02).astype(np.float32)
    W = np.where(rng.random((R, K)) < dens, W, 0.0)
    if dt == "f16":
        return W.astype(np.float16)
    return (W.view(np.uint32) >> 16).astype(np.uint16)


def _canon(Wbits):
    Wbits = np.asarray(Wbits).view(np.uint16)
    return np.where((Wbits & 0x7FFF) == 0, 0, Wbits).astype(np.uint16)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("R,K,dens", [(16, 64, 0.5), (37, 520, 0.5), (64, 1024, 0.3), (20, 700, 0.7),
                                      (3, 4, 1.0), (48, 4096, 0.5)])
def test_round_trip(dt, R, K, dens):
    rng = np.random.default_rng(R * 1000 + K)
    W = _sparse(rng, R, K, dens, dt)
    img = oracle.hy_encode(W, dt)
    assert np.array_equal(oracle.hy_read(img, R, K, dt), _canon(W))


def test_round_trip_nonfinite_and_signed_zero():
    rng = np.random.default_rng(5)
    W = _sparse(rng, 32, 512, 0.6, "f16").view(np.uint16).copy()
    pos = rng.choice(W.size, 60, replace=False)
    specials = np.array([0x7C00, 0xFC00, 0x7E00, 0x7C01, 0x8000, 0xFE01], np.uint16)
    W.flat[pos] = specials[np.arange(60) % len(specials)]
    img = oracle.hy_encode(W.view(np.float16), "f16")
    assert np.array_equal(oracle.hy_read(img, 32, 512, "f16"), _canon(W))


def test_two_of_four_weights_are_the_2to4_packing():
    """Weights with at most two nonzeros per group: no slot filling, no
    residual, and every group with two nonzeros holds exactly what the pinned
    2:4 selection keeps."""
    rng = np.random.default_rng(7)
    R, K = 40, 640
    W = (rng.standard_normal((R, K)) * 0.02).astype(np.float16)
    vals, idx = oracle.compress(W, 2, 4, "f16")          # top-2 of every group
    W2 = oracle.decompress(vals, idx, R, K, 2, 4, "f16")
    img = oracle.hy_encode(W2, "f16")
    assert len(img["res_ent"]) == 0 and not img["codes"].any()
    pv, pi = oracle.read_packed(img["values"], img["meta"], R, K, 2, 4, "f16")
    assert np.array_equal(pi, idx) and np.array_equal(pv.view(np.uint16), vals.view(np.uint16))


def _fu_stats(img, R, K):
    nRB, nKB, nSeg = oracle.hy_geometry(R, K)
    codes = img["codes"].reshape(-1, 8)
    nib = np.stack([codes & 15, codes >> 4], -1).reshape(-1, 16)
    return nib


def test_counts_add_up():
    rng = np.random.default_rng(11)
    R, K = 64, 2048
    W = _sparse(rng, R, K, 0.5, "f16")
    img = oracle.hy_encode(W, "f16")
    nnz = int(((W.view(np.uint16) & 0x7FFF) != 0).sum())
    nib = _fu_stats(img, R, K)
    filled = int((nib != 0).sum())
    # Sparse-TC holds min(nz, 2) per group
    g = ((W.view(np.uint16) & 0x7FFF) != 0).reshape(R, K // 4, 4).sum(-1)
    tc = int(np.minimum(g, 2).sum())
    assert tc + filled + len(img["res_ent"]) == nnz
    assert int(img["res_ptr"][-1]) == len(img["res_ent"])
    # ~50% unstructured: most surplus is slot-filled, a few percent residual
    assert 0.10 < filled / nnz < 0.20 and len(img["res_ent"]) / nnz < 0.06
