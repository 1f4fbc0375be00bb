"""Pins of the oracle's reader for the GPU library's packed layout (CPU only).

The fixtures in golden/packed_format.txt are byte images built by hand from
the layout's description; the reader must decode them to the kept sets the
top-|w| rule gives, and must find no padding violation in them.
"""
import os

import numpy as np
import pytest

import oracle


def _cases(golden_dir):
    cur = None
    for raw in open(os.path.join(golden_dir, "packed_format.txt")):
        line = raw.split("#")[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "case":
            cur = dict(dt=tok[1], **{k: int(v) for k, v in (t.split("=") for t in tok[2:])})
            cur["values"], cur["meta"] = {}, {}
        elif tok[0] in ("values_len", "meta_len"):
            cur[tok[0]] = int(tok[1])
            cur[tok[0].split("_")[0] + "_fill"] = int(tok[3], 16)
        elif tok[0] in ("values", "meta"):
            cur[tok[0]][int(tok[1].rstrip(":"))] = bytes(int(b, 16) for b in tok[2:])
        elif tok[0] == "end":
            yield cur
            cur = None
        else:
            cur[tok[0]] = line[len(tok[0]):].strip()


def _image(n, fill, pieces):
    a = np.full(n, fill, np.uint8)
    for off, bs in pieces.items():
        a[off:off + len(bs)] = np.frombuffer(bs, np.uint8)
    return a


def test_golden_packed_images(golden_dir):
    n = 0
    for c in _cases(golden_dir):
        R, K, N, M, dt = c["R"], c["K"], c["N"], c["M"], c["dt"]
        values = _image(c["values_len"], c["values_fill"], c["values"])
        meta = _image(c["meta_len"], c["meta_fill"], c["meta"]) if c["meta_len"] else None
        vals, idx = oracle.read_packed(values, meta, R, K, N, M, dt)
        if "W" in c:
            W = np.array([int(t) for t in c["W"].split()], np.int8)[None, :]
        elif "Wbits" in c:
            W = np.array([int(t, 16) for t in c["Wbits"].split()], np.uint16)[None, :]
            W = W.view(np.float16) if dt == "f16" else W
        else:
            W = np.array([[int(t) for t in r.split()] for r in c["W_rows"].split("|")], np.int8)
        # the hand image must hold exactly what the selection rule keeps
        cv, ci = oracle.compress(W, N, M, dt)
        assert np.array_equal(ci, idx)
        assert np.array_equal(cv.view(np.uint8), vals.view(np.uint8))
        if "expect_idx" in c:
            assert idx[0].ravel().tolist() == [int(t) for t in c["expect_idx"].split()]
        if "expect_vals" in c:
            assert vals[0].ravel().astype(int).tolist() == [int(t) for t in c["expect_vals"].split()]
        if "expect_valbits" in c:
            assert vals[0].ravel().view(np.uint16).tolist() == \
                [int(t, 16) for t in c["expect_valbits"].split()]
        assert oracle.check_padding(values, meta, R, K, N, M, dt) == 0
        n += 1
    assert n == 4


def test_padding_checker_flags_planted_mistakes(golden_dir):
    # plant mistakes in a hand image (on the CPU) and check they are counted
    c = next(iter(_cases(golden_dir)))
    values = _image(c["values_len"], c["values_fill"], c["values"])
    meta = _image(c["meta_len"], c["meta_fill"], c["meta"])
    bad_v = values.copy()
    bad_v[64 * 3 + 5] = 1            # row 3 is outside R=1: must be zero
    assert oracle.check_padding(bad_v, meta, 1, 8, 2, 4, "i8") == 1
    bad_m = meta.copy()
    bad_m[16 * 2] = 0x00             # row 2 slots (0,1,0,1) -> (0,0,0,0): two wrong
    assert oracle.check_padding(values, bad_m, 1, 8, 2, 4, "i8") == 2


def test_reader_roundtrip_through_a_second_layout_writer():
    # An independent writer of the layout in numpy (bit by bit) must round-trip
    # through the C reader for every supported N:M and dtype.
    rng = np.random.default_rng(14)
    for dt, b in (("i8", 1), ("f16", 2)):
        for N, M in ((1, 4), (2, 4), (3, 4), (4, 4), (1, 8), (2, 8), (4, 8), (8, 8)):
            R, K = 21, (128 // b) + 3 * M if M == 4 else (128 // b) + 2 * M
            W = (rng.integers(-100, 100, (R, K)).astype(np.int8) if dt == "i8"
                 else rng.standard_normal((R, K)).astype(np.float16))
            vals, idx = oracle.compress(W, N, M, dt)
            KB = 128 // b
            C = KB // M * N
            w = {4: 2, 8: 3}[M]
            MR = -(-(C * w) // 8)
            MR = -(-MR // 4) * 4
            nRB, nKB = -(-R // 16), -(-K // KB)
            V = np.zeros(nRB * nKB * 16 * C * b, np.uint8)
            bits = np.zeros(nRB * nKB * 16 * MR * 8, np.uint8)
            G, GB = K // M, KB // M
            vb = vals.view(np.uint8).reshape(R, G, N, b)
            for rb in range(nRB):
                for kb in range(nKB):
                    blk = rb * nKB + kb
                    for rr in range(16):
                        for c in range(C):
                            r, g, j = rb * 16 + rr, kb * GB + c // N, c % N
                            real = r < R and g < G
                            off = (blk * 16 * C + rr * C + c) * b
                            if real:
                                V[off:off + b] = vb[r, g, j]
                            pos = idx[r, g, j] if real else j
                            base = (blk * 16 * MR + rr * MR) * 8 + c * w
                            for bit in range(w):
                                bits[base + bit] = (pos >> bit) & 1
            meta = np.packbits(bits.reshape(-1, 8), axis=1, bitorder="little").ravel()
            v2, i2 = oracle.read_packed(V, meta if N < M else None, R, K, N, M, dt)
            assert np.array_equal(i2, idx), (dt, N, M)
            assert np.array_equal(v2.view(np.uint8), vals.view(np.uint8)), (dt, N, M)
            assert oracle.check_padding(V, meta if N < M else None, R, K, N, M, dt) == 0
