"""GPU parity of nm_pack and nm_spmm against the CPU oracle (needs an MI355X).

 - nm_pack: the packed bytes, decoded by the oracle's independent reader,
   equal the oracle's compression bit for bit, and padding is clean.
 - nm_spmm at sizes the oracle finishes in seconds (several tiles plus ragged
   tails): every dtype pair, every N:M, element by element.
 - Edge shapes: T in {1, 15, 16, 17}, K = M, R = 1 / 17, row strides beyond T,
   output padding untouched.
 - Identity activations return the masked weights; repeated runs are
   bitwise identical.
 - Every workload shape at full size (the launch configuration the benchmark
   times), compared on sampled rows the oracle computes one by one.
"""
import numpy as np
import pytest

import nm_inputs
import oracle
from tests._parity import compare, layer_case, packed_host, reference, run

pytestmark = pytest.mark.gpu

PAIRS = [("i8", "i32"), ("i8", "i8"), ("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"),
         ("bf16", "f32")]
NMS = [(1, 4), (2, 4), (3, 4), (4, 4), (1, 8), (2, 8), (4, 8), (8, 8)]


def _inputs(dt, out, R, K, T, N, M, seed, tag):
    if dt == "i8" and out == "i32":
        return (nm_inputs.uniform_int8((R, K), seed, tag, "W"),
                nm_inputs.uniform_int8((K, T), seed, tag, "X"),
                nm_inputs.uniform_int8((R,), seed, tag, "b").astype(np.int32) * 1000, None)
    if dt == "i8":
        q = nm_inputs.quant_layer(R, K, T, N, M, seed, tag)
        return q.W, q.X, q.bias, q.scale
    W = nm_inputs.normal((R, K), 0.02, dt, seed, tag, "W")
    X = nm_inputs.normal((K, T), 1.0, dt, seed, tag, "X")
    b = nm_inputs.normal((R,), 0.05, "f32", seed, tag, "b")
    return W, X, b, None


@pytest.mark.parametrize("dt", ["i8", "f16", "bf16"])
@pytest.mark.parametrize("N,M", NMS)
def test_pack_matches_oracle(dt, N, M):
    for R, K in ((1, M), (17, 96 if M == 4 else 96), (40, 264 if M == 4 else 264), (33, 512)):
        if dt == "i8":
            # small integers: many magnitude ties
            W = nm_inputs.uniform_int8((R, K), 1, "pack", dt, N, M, R, lo=-3, hi=3)
            W[0, :M] = -128
        else:
            W = nm_inputs.normal((R, K), 0.02, dt, 1, "pack", N, M, R)
            if dt == "f16":
                W[0, :4] = np.array([0.0, -0.0, -0.0, 0.0], np.float16)
        _, p = run(W, np.zeros((K, 1), W.dtype), N, M, dt, {"i8": "i32", "f16": "f16",
                                                          "bf16": "bf16"}[dt])
        v, m = packed_host(p)
        vals, idx = oracle.read_packed(v, m, R, K, N, M, dt)
        cv, ci = oracle.compress(W, N, M, dt)
        assert np.array_equal(ci, idx), (R, K)
        assert np.array_equal(cv.view(np.uint8), vals.view(np.uint8)), (R, K)
        assert oracle.check_padding(v, m, R, K, N, M, dt) == 0, (R, K)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("N,M", [(1, 4), (2, 4), (3, 8), (4, 8)])
def test_pack_nonfinite_matches_oracle(dt, N, M):
    """Weights holding +-Inf and NaNs of several payloads and signs: the packed
    selection equals the oracle's (NaN above Inf above finite, NaNs by
    payload, sign ignored, ties to the lower position)."""
    R, K = 24, 64
    W = nm_inputs.normal((R, K), 0.02, dt, 9, "pack-nonfinite", N, M)
    bits = W.view(np.uint16)
    if dt == "f16":
        specials = np.array([0x7C00, 0xFC00, 0x7E00, 0xFE00, 0x7C01, 0x7FFF, 0xFE01, 0x7BFF], np.uint16)
    else:
        specials = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0x7FFF, 0xFFC1, 0x7F7F], np.uint16)
    rng = np.random.default_rng(11)
    pos = rng.random((R, K)) < 0.3
    bits[pos] = specials[rng.integers(0, len(specials), int(pos.sum()))]
    _, p = run(W, np.zeros((K, 1), W.dtype), N, M, dt, dt)
    v, m = packed_host(p)
    vals, idx = oracle.read_packed(v, m, R, K, N, M, dt)
    cv, ci = oracle.compress(W, N, M, dt)
    assert np.array_equal(ci, idx)
    assert np.array_equal(cv.view(np.uint8), vals.view(np.uint8))


def test_pack_row_stride():
    import torch
    import semi_structured_sparse_nm_amd as nm
    from tests._parity import dev
    R, K = 20, 200
    W = nm_inputs.uniform_int8((R, K + 24), 2, "ldw")
    full = dev(W, "i8")
    p = nm.pack(full[:, :K], 2, 4)
    torch.cuda.synchronize()
    v, m = packed_host(p)
    vals, idx = oracle.read_packed(v, m, R, K, 2, 4, "i8")
    cv, ci = oracle.compress(np.ascontiguousarray(W[:, :K]), 2, 4, "i8")
    assert np.array_equal(ci, idx) and np.array_equal(cv, vals)


@pytest.mark.parametrize("dt,out", PAIRS)
@pytest.mark.parametrize("N,M", NMS)
def test_spmm_small(dt, out, N, M):
    R, K, T = 96, 192, 197
    W, X, b, s = _inputs(dt, out, R, K, T, N, M, 3, f"small-{dt}-{out}-{N}-{M}")
    Y, _ = run(W, X, N, M, dt, out, bias=b, scale=s)
    compare(Y, reference(W, X, N, M, dt, out, bias=b, scale=s), out, f"{dt}->{out} {N}:{M}")


@pytest.mark.parametrize("dt,out", PAIRS)
@pytest.mark.parametrize("R,K,T", [(1, 8, 1), (17, 8, 15), (16, 96, 16), (17, 96, 17),
                                   (33, 200, 64), (5, 1032, 3)])
def test_spmm_edges(dt, out, R, K, T):
    N, M = (2, 4) if K % 8 else (3, 8)
    W, X, b, s = _inputs(dt, out, R, K, T, N, M, 4, f"edge-{dt}-{out}-{R}-{K}-{T}")
    Y, _ = run(W, X, N, M, dt, out, bias=b, scale=s, ldx_pad=5, ldy_pad=3, sentinel=7)
    compare(Y[:, :T], reference(W, X, N, M, dt, out, bias=b, scale=s), out, "edge")
    pad = Y[:, T:]
    want = 7 if out != "bf16" else oracle.round_to(np.array([7.0]), "bf16")[0]
    assert np.all(pad == want), "writes beyond T"


@pytest.mark.parametrize("dt", ["i8", "f16", "bf16"])
@pytest.mark.parametrize("N,M", [(2, 4), (1, 4), (2, 8), (4, 8)])
def test_identity_activation(dt, N, M):
    R, K = 48, 256
    out = {"i8": "i32", "f16": "f32", "bf16": "f32"}[dt]
    if dt == "i8":
        W = nm_inputs.uniform_int8((R, K), 5, "ident")
        X = np.eye(K, dtype=np.int8)
    else:
        W = nm_inputs.normal((R, K), 0.02, dt, 5, "ident")
        one = np.float16(1.0) if dt == "f16" else np.uint16(0x3F80)
        X = np.zeros((K, K), W.dtype)
        np.fill_diagonal(X, one)
    Y, _ = run(W, X, N, M, dt, out)
    vals, idx = oracle.compress(W, N, M, dt)
    Wm = oracle.to_f64(oracle.decompress(vals, idx, R, K, N, M, dt), dt)
    assert np.array_equal(np.asarray(Y).astype(np.float64), Wm)   # every output is one product


@pytest.mark.parametrize("dt,out", [("i8", "i8"), ("f16", "f16"), ("bf16", "f32")])
def test_repeat_runs_bitwise_identical(dt, out):
    R, K, T = 256, 768, 1000
    W, X, b, s = _inputs(dt, out, R, K, T, 2, 4, 6, "repeat")
    Y1, _ = run(W, X, 2, 4, dt, out, bias=b, scale=s)
    Y2, _ = run(W, X, 2, 4, dt, out, bias=b, scale=s)
    assert np.array_equal(np.asarray(Y1).view(np.uint8), np.asarray(Y2).view(np.uint8))


def test_config1_exact():
    (L,) = nm_inputs.config1()
    W, X, b, s = layer_case(L)
    Y, _ = run(W, X, L.N, L.M, L.dt, L.out)
    ref = reference(W, X, L.N, L.M, L.dt, L.out)
    compare(Y, ref, L.out, L.name)
    # closed-form row checksums, exact in int64
    vals, idx = oracle.compress(W, L.N, L.M, L.dt)
    Wm = oracle.decompress(vals, idx, L.R, L.K, L.N, L.M, L.dt).astype(np.int64)
    assert np.array_equal(Y.astype(np.int64).sum(axis=1), Wm @ X.astype(np.int64).sum(axis=1))


def _full_layers():
    seen, out = set(), []
    for cfg, layers in nm_inputs.all_configs().items():
        if cfg == "1":
            continue
        for L in layers:
            key = (L.R, L.K, L.T, L.N, L.M, L.dt, L.out)
            if key in seen:        # the mixed stack repeats shapes of the ViT-B layers
                continue
            seen.add(key)
            out.append(L)
    return out


# Multiply-adds (R K T N / M) up to which a full-size case is compared on
# every output; the oracle's direct loop runs at tens of G multiply-adds per
# second on the host's cores.
FULL_COMPARE_MACS = 16e9


def _full_size_rows(L):
    """Output rows a full-size case compares: every row when the oracle's
    cost allows, else a fixed set -- the first and last row of every 64-row
    band (one wave's rows), and every row of each 256- or 512-row tile that is
    some workgroup's second (or later) tile under the persistent kernels'
    tile orders (XCD x owning a contiguous range of tiles, one workgroup per
    4-wave / 8-wave slot of 256 CUs; row tile fastest, or grouped)."""
    if L.R * L.K * L.T * L.N / L.M <= FULL_COMPARE_MACS:
        return np.arange(L.R)
    rows = set()
    for b0 in range(0, L.R, 64):
        rows.update((b0, min(b0 + 63, L.R - 1)))
    ntok = (L.T + 127) // 128
    for BM, nwg in ((256, 64), (512, 32)):
        mt = (L.R + BM - 1) // BM
        ntot = mt * ntok
        per_xcd = (ntot + 7) // 8
        # the fp16 / bf16 tile kernel orders tiles in groups of gm row tiles
        # (gm = all of them for weights that fit in L2): both orders' rows
        for gm in {mt, _group_rows(L, mt, ntok, 64, True), _group_rows(L, mt, ntok, 32, False)}:
            for x in range(8):
                for L2 in range(x * per_xcd + nwg, min((x + 1) * per_xcd, ntot)):
                    grp, inn = divmod(L2, gm * ntok)
                    r0 = (grp * gm + inn % min(gm, mt - grp * gm)) * BM
                    rows.update(range(r0, min(r0 + BM, L.R)))
    return np.array(sorted(rows))


def _group_rows(L, mt, ntok, nconc, sparse24):
    """gm of the tile kernels' grouped tile order (the host's choice
    restated: fewest operand bytes per 128-column step for the workgroups one
    XCD runs at once, all row tiles when the weight fits in L2), for the
    fp16 / bf16 2:4 kernel (64 workgroups per XCD) or the dense-expand one (32)."""
    eb = 1 if L.dt == "i8" else 2
    w_total = L.R * L.K * L.N // L.M * eb * 1.125
    if w_total <= 4 * 1024 * 1024 or mt <= 1:
        return mt
    if sparse24:
        wk, xk = 256.0 * (64 * 2 + 16), 128.0 * 128 * 2
    else:
        bits = 0 if L.N == L.M else (2 if L.M == 4 else 3)
        wk, xk = 256.0 * 128 * L.N / L.M * (eb + bits / 8.0), 128.0 * 128 * eb
    best, best_cost = mt, None
    for gm in range(1, mt + 1):
        rows = min(gm, nconc)
        toks = min((nconc + rows - 1) // rows, ntok)
        cost = rows * wk + toks * xk
        if best_cost is None or cost < best_cost:
            best, best_cost = gm, cost
    return best


def _full_size_case(L, out=None):
    out = out or L.out
    W, X, b, s = layer_case(L)
    Y, _ = run(W, X, L.N, L.M, L.dt, out, bias=b, scale=s)
    rows = _full_size_rows(L)
    whole = len(rows) == L.R
    ref = reference(W, X, L.N, L.M, L.dt, out, bias=b, scale=s, rows=None if whole else rows)
    compare(np.asarray(Y) if whole else np.asarray(Y)[rows], ref, out, f"{L.name} -> {out}")


@pytest.mark.parametrize("L", _full_layers(), ids=lambda L: L.name)
def test_full_size(L):
    """Every workload shape at full size with the kernel nm_spmm picks for it
    (the launch the benchmark times), on every output or on the rows of
    _full_size_rows."""
    _full_size_case(L)


@pytest.mark.parametrize("L", [L for L in nm_inputs.config5() if L.dt == "bf16"], ids=lambda L: L.name)
def test_full_size_bf16_in_f32_out(L):
    """LLaMA-7B shapes with bf16 operands and fp32 output at the 2e-3
    max-abs-normalised bar (one bf16 ulp of the output alone would exceed
    it, so the bar is checked where the output is fp32)."""
    _full_size_case(L, out="f32")


TK_FULL = ["c2_vitb_fc1_1of4", "c2_vitb_fc2_2of8", "c2_vitb_fc1_4of8", "c3_swin_C96_fc1_2of4",
           "c5_llama_up_2of4_T16_f16"]


@pytest.mark.parametrize("name", TK_FULL)
def test_tk_full_size_sampled_rows(name):
    """nm_spmm_tk (X [T][K], Y [T][R]) at full workload sizes with the
    default choice (re-packed 2:4 [T][K] kernel, or transpose, [K][T] kernel,
    transpose), sampled weight rows against the oracle, and nothing written
    past R."""
    import torch
    import semi_structured_sparse_nm_amd as nm
    from tests._parity import TORCH_DT, dev, host
    L = {l.name: l for ls in nm_inputs.all_configs().values() for l in ls}[name]
    W, X, b, s = layer_case(L)
    p = nm.pack(dev(W, L.dt), L.N, L.M)
    assert nm.variant_tk(p, L.T, TORCH_DT[L.out]).startswith(("repack24_", "transpose_", "smfmac_i8_2of4_tk",
                                                              "split24_", "dense24_"))
    Xt = dev(np.ascontiguousarray(X.T), L.dt)
    Yfull = torch.full((L.T, L.R + 16), 5, dtype=TORCH_DT[L.out], device="cuda")
    kw = {}
    if b is not None:
        kw["bias"] = torch.from_numpy(np.asarray(b)).cuda()
    if s is not None:
        kw["scale"] = torch.from_numpy(np.asarray(s, np.float32)).cuda()
    nm.linear(p, Xt, out_dtype=TORCH_DT[L.out], out=Yfull[:, :L.R], **kw)
    torch.cuda.synchronize()
    Y = host(Yfull, L.out)
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([[0, L.R - 1], rng.integers(0, L.R, 6)]))
    ref = reference(W, X, L.N, L.M, L.dt, L.out, bias=b, scale=s, rows=rows)
    compare(np.ascontiguousarray(Y[:, rows].T), ref, L.out, name)
    want = 5 if L.out != "bf16" else oracle.round_to(np.array([5.0]), "bf16")[0]
    assert np.all(Y[:, L.R:] == want), "writes beyond R"


FAST_I8 = ["smfmac_i8_2of4_persistent", "smfmac_i8_2of4_persistent_w8"]


def _set_forced(name=None, S=None):
    """NM_SPMM_VARIANT=<variant>[:<S>], the library's one debug override:
    set the variant part or the K-slice part, keeping the other."""
    import os
    cur = os.environ.get("NM_SPMM_VARIANT", "")
    v, _, k = cur.partition(":")
    if name is not None:
        v = name
    if S is not None:
        k = str(S)
    os.environ["NM_SPMM_VARIANT"] = v + (":" + k if k else "")


@pytest.fixture
def force_variant():
    import os
    old = os.environ.get("NM_SPMM_VARIANT")
    yield lambda name: _set_forced(name=name)
    if old is None:
        os.environ.pop("NM_SPMM_VARIANT", None)
    else:
        os.environ["NM_SPMM_VARIANT"] = old


@pytest.mark.parametrize("variant", FAST_I8)
@pytest.mark.parametrize("out", ["i8", "i32"])
@pytest.mark.parametrize("R,K,T", [(300, 192, 144), (17, 4, 16), (256, 96, 1008), (520, 768, 400),
                                   (3072, 768, 12608), (259, 1280, 272)])
def test_fast_i8_variants(force_variant, variant, out, R, K, T):
    import torch
    import semi_structured_sparse_nm_amd as nm
    force_variant(variant)
    W, X, b, s = _inputs("i8", out, R, K, T, 2, 4, 8, f"fast-{variant}-{out}-{R}-{K}-{T}")
    p = nm.pack(torch.from_numpy(W).cuda(), 2, 4)
    assert nm.variant(p, T, torch.int8 if out == "i8" else torch.int32) == variant
    Y, _ = run(W, X, 2, 4, "i8", out, bias=b, scale=s, ldx_pad=32, ldy_pad=16 if out == "i8" else 3,
               sentinel=5)
    compare(Y[:, :T], reference(W, X, 2, 4, "i8", out, bias=b, scale=s), out, variant)
    assert np.all(Y[:, T:] == 5), "writes beyond T"


# the weight-stationary int8 2:4 kernel takes K in (640, 768] (six column
# blocks in registers) and R <= 16384 (a workgroup per 512-row tile on each XCD)
STAT_SHAPES = [(300, 768, 144), (17, 700, 16), (520, 768, 400), (1000, 656, 272), (2304, 768, 1040),
               (3072, 768, 12608), (16384, 768, 64), (777, 768, 48), (520, 768, 13408), (300, 768, 38464)]


@pytest.mark.parametrize("out", ["i8", "i32"])
@pytest.mark.parametrize("R,K,T", STAT_SHAPES)
def test_stationary_i8_variant(force_variant, out, R, K, T):
    """Weight-stationary int8 2:4 kernel forced: ragged rows (row blocks past
    R re-read the last one), a partial last column block, one to 197 token
    steps over the XCDs, padded strides; nothing written past T."""
    import torch
    import semi_structured_sparse_nm_amd as nm
    variant = "smfmac_i8_2of4_stationary"
    force_variant(variant)
    W, X, b, s = _inputs("i8", out, R, K, T, 2, 4, 8, f"stat-{out}-{R}-{K}-{T}")
    p = nm.pack(torch.from_numpy(W).cuda(), 2, 4)
    assert nm.variant(p, T, torch.int8 if out == "i8" else torch.int32) == variant
    Y, _ = run(W, X, 2, 4, "i8", out, bias=b, scale=s, ldx_pad=32, ldy_pad=16 if out == "i8" else 3,
               sentinel=5)
    compare(Y[:, :T], reference(W, X, 2, 4, "i8", out, bias=b, scale=s), out, variant)
    assert np.all(Y[:, T:] == 5), "writes beyond T"


@pytest.mark.parametrize("R,K,T", [(300, 768, 144), (520, 768, 400), (1000, 656, 272)])
def test_gelu_i8_stationary(force_variant, R, K, T):
    """GELU between the two scales on the weight-stationary kernel."""
    _gelu_case(force_variant, "smfmac_i8_2of4_stationary", "i8", "i8", 2, 4, R, K, T, 38)


# the small int8 2:4 kernel: any T, rows at any byte alignment
SMALL_SHAPES = [(192, 192, 197), (17, 8, 5), (300, 200, 33), (64, 768, 1), (520, 1000, 61), (16, 4096, 16),
                (33, 132, 300)]


@pytest.mark.parametrize("out", ["i8", "i32"])
@pytest.mark.parametrize("R,K,T", SMALL_SHAPES)
def test_small_i8_variant(force_variant, out, R, K, T):
    """The one-wave-per-tile int8 2:4 kernel forced on odd token counts and
    row pitches that are not multiples of 16 bytes (byte gathers, masked
    token tails, ragged rows and column blocks); nothing written past T."""
    import torch
    import semi_structured_sparse_nm_amd as nm
    variant = "smfmac_i8_2of4_small"
    force_variant(variant)
    W, X, b, s = _inputs("i8", out, R, K, T, 2, 4, 8, f"small-{out}-{R}-{K}-{T}")
    p = nm.pack(torch.from_numpy(W).cuda(), 2, 4)
    assert nm.variant(p, T, torch.int8 if out == "i8" else torch.int32) == variant
    Y, _ = run(W, X, 2, 4, "i8", out, bias=b, scale=s, ldx_pad=3, ldy_pad=5, sentinel=5)
    compare(Y[:, :T], reference(W, X, 2, 4, "i8", out, bias=b, scale=s), out, variant)
    assert np.all(Y[:, T:] == 5), "writes beyond T"


@pytest.mark.parametrize("R,K,T", [(192, 192, 197), (300, 200, 33)])
def test_gelu_i8_small(force_variant, R, K, T):
    """GELU between the two scales on the small kernel."""
    _gelu_case(force_variant, "smfmac_i8_2of4_small", "i8", "i8", 2, 4, R, K, T, 39)


def test_config1_runs_on_the_small_kernel():
    """The ViT-Tiny slice (T = 197, 197-byte rows) takes the small sparse
    kernel, not the generic fallback."""
    import torch
    import nm_inputs
    import semi_structured_sparse_nm_amd as nm
    L = nm_inputs.config1()[0]
    p = nm.pack(torch.zeros((L.R, L.K), dtype=torch.int8, device="cuda"), L.N, L.M)
    assert nm.variant(p, L.T, torch.int32) == "smfmac_i8_2of4_small"


FAST_H = ["smfmac_h_2of4_persistent"]


@pytest.mark.parametrize("variant", FAST_H)
@pytest.mark.parametrize("dt,out", [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("R,K,T", [(300, 192, 144), (17, 4, 16), (256, 96, 1008), (520, 768, 400),
                                   (259, 1280, 272), (64, 4100, 32)])
def test_fast_h_variants(force_variant, variant, dt, out, R, K, T):
    """fp16 / bf16 2:4 sparse-MFMA kernel forced on ragged rows, partial
    64-column blocks (K % 64 != 0), several token tiles and row strides."""
    import torch
    import semi_structured_sparse_nm_amd as nm
    from tests._parity import TORCH_DT, dev
    force_variant(variant)
    W, X, b, s = _inputs(dt, out, R, K, T, 2, 4, 9, f"fasth-{dt}-{out}-{R}-{K}-{T}")
    p = nm.pack(dev(W, dt), 2, 4)
    assert nm.variant(p, T, TORCH_DT[out]) == variant
    Y, _ = run(W, X, 2, 4, dt, out, bias=b, scale=s, ldx_pad=24, ldy_pad=8, sentinel=5)
    compare(Y[:, :T], reference(W, X, 2, 4, dt, out, bias=b, scale=s), out, variant)
    pad = Y[:, T:]
    want = 5 if out != "bf16" else oracle.round_to(np.array([5.0]), "bf16")[0]
    assert np.all(pad == want), "writes beyond T"


@pytest.mark.parametrize("dt,out", [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("R,K,T", [(16, 64, 16), (17, 4, 1), (300, 200, 3), (96, 4100, 16), (40, 512, 8),
                                   (33, 11008, 16)])
def test_decode_h_variant(force_variant, dt, out, R, K, T):
    """fp16 / bf16 2:4 decode kernel (K split over eight waves, partials summed
    in LDS): fewer blocks than waves, partial blocks, ragged rows, T < 16."""
    import semi_structured_sparse_nm_amd as nm
    from tests._parity import TORCH_DT, dev
    force_variant("smfmac_h_2of4_decode")
    W, X, b, s = _inputs(dt, out, R, K, T, 2, 4, 10, f"dec-{dt}-{out}-{R}-{K}-{T}")
    p = nm.pack(dev(W, dt), 2, 4)
    # nm_spmm_variant assumes dense rows (ldx = T); the run pads X rows to a
    # multiple of 8 elements, which the forced kernel needs
    if T % 8 == 0:
        assert nm.variant(p, T, TORCH_DT[out]) == "smfmac_h_2of4_decode"
    Y, _ = run(W, X, 2, 4, dt, out, bias=b, scale=s, ldx_pad=(-T) % 8 + 8, ldy_pad=3, sentinel=5)
    compare(Y[:, :T], reference(W, X, 2, 4, dt, out, bias=b, scale=s), out, "decode")
    pad = Y[:, T:]
    want = 5 if out != "bf16" else oracle.round_to(np.array([5.0]), "bf16")[0]
    assert np.all(pad == want), "writes beyond T"


@pytest.mark.parametrize("dt,out", [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("R,K,T", [(16, 64, 16), (17, 4, 1), (300, 200, 3), (96, 4100, 16), (40, 512, 8),
                                   (33, 11008, 16), (1100, 2048, 5), (64, 9000, 13)])
def test_stream24_variant(force_variant, dt, out, R, K, T):
    """fp16 / bf16 2:4 on the streaming decode schedule (one workgroup per
    CU walking row blocks, segments of 512 columns per wave, activation
    chunks of four segments): partial blocks and segments, ragged rows,
    several row blocks per workgroup, several chunks, T < 16."""
    import semi_structured_sparse_nm_amd as nm
    from tests._parity import TORCH_DT, dev
    force_variant("smfmac_h_2of4_stream_decode")
    W, X, b, s = _inputs(dt, out, R, K, T, 2, 4, 12, f"s24-{dt}-{out}-{R}-{K}-{T}")
    p = nm.pack(dev(W, dt), 2, 4)
    assert nm.variant(p, T, TORCH_DT[out]) == "smfmac_h_2of4_stream_decode"
    # odd T with dense rows: the last activation element's 4-byte piece ends past X
    Y, _ = run(W, X, 2, 4, dt, out, bias=b, scale=s, ldx_pad=0 if T % 2 else 3, ldy_pad=3, sentinel=5)
    compare(Y[:, :T], reference(W, X, 2, 4, dt, out, bias=b, scale=s), out, "stream24")
    pad = Y[:, T:]
    want = 5 if out != "bf16" else oracle.round_to(np.array([5.0]), "bf16")[0]
    assert np.all(pad == want), "writes beyond T"


EXPAND_NMS = [(1, 4), (3, 4), (4, 4), (1, 8), (2, 8), (4, 8), (8, 8)]
EXPAND_SHAPES = [(300, 192, 144), (17, 8, 16), (259, 1288, 272)]


EXPAND_VARIANTS = ["expand_mfma_persistent"]


def _expand_case(force_variant, variant, dt, out, N, M, R, K, T, seed):
    import semi_structured_sparse_nm_amd as nm
    from tests._parity import TORCH_DT, dev
    force_variant(variant)
    W, X, b, s = _inputs(dt, out, R, K, T, N, M, seed, f"expand-{dt}-{out}-{N}-{M}-{R}-{K}-{T}")
    p = nm.pack(dev(W, dt), N, M)
    assert nm.variant(p, T, TORCH_DT[out]) == variant
    narrow = out in ("i8", "f16", "bf16")
    Y, _ = run(W, X, N, M, dt, out, bias=b, scale=s, ldx_pad=32, ldy_pad=16 if narrow else 3, sentinel=5)
    compare(Y[:, :T], reference(W, X, N, M, dt, out, bias=b, scale=s), out, f"expand {N}:{M}")
    pad = Y[:, T:]
    want = 5 if out != "bf16" else oracle.round_to(np.array([5.0]), "bf16")[0]
    assert np.all(pad == want), "writes beyond T"


@pytest.mark.parametrize("variant", EXPAND_VARIANTS)
@pytest.mark.parametrize("dt,out", PAIRS)
@pytest.mark.parametrize("N,M", EXPAND_NMS)
@pytest.mark.parametrize("R,K,T", EXPAND_SHAPES)
def test_expand_variant(force_variant, variant, dt, out, N, M, R, K, T):
    """Dense-expand kernels (every N:M but 2:4, windows expanded in
    registers; 16 x 16 and 32 x 32 fragments) forced on ragged rows, partial
    column blocks, several token tiles and padded row strides, every dtype
    pair."""
    _expand_case(force_variant, variant, dt, out, N, M, R, K, T, 11)


@pytest.mark.parametrize("variant", EXPAND_VARIANTS)
@pytest.mark.parametrize("dt,out", [("i8", "i8"), ("f16", "f16"), ("bf16", "f32")])
@pytest.mark.parametrize("N,M", [(1, 4), (3, 4), (4, 8), (8, 8)])
@pytest.mark.parametrize("R,K,T", [(256, 96, 1008), (520, 768, 400), (64, 4104, 32)])
def test_expand_variant_more_shapes(force_variant, variant, dt, out, N, M, R, K, T):
    """More tiles per workgroup than one (1008 tokens), many column blocks
    (K = 4104) and several row tiles."""
    _expand_case(force_variant, variant, dt, out, N, M, R, K, T, 12)


# 1:4, 1:8 and 2:8 weights re-packed to 2:4 in the workspace, then multiplied
# by the 2:4 sparse-MFMA tile kernels
REPACK_NMS = [(1, 4), (1, 8), (2, 8)]
REPACK_CASES = [("smfmac_i8_2of4_persistent", "i8", "i8"), ("smfmac_i8_2of4_persistent", "i8", "i32"),
                ("smfmac_i8_2of4_persistent_w8", "i8", "i8"), ("smfmac_h_2of4_persistent", "f16", "f16"),
                ("smfmac_h_2of4_persistent", "bf16", "f32"), ("smfmac_h_2of4_persistent", "bf16", "bf16")]


@pytest.mark.parametrize("inner,dt,out", REPACK_CASES)
@pytest.mark.parametrize("N,M", REPACK_NMS)
@pytest.mark.parametrize("R,K,T", [(300, 192, 144), (17, 8, 16), (259, 1288, 272), (520, 776, 400)])
def test_repack24_variants(force_variant, inner, dt, out, N, M, R, K, T):
    """The re-packed path forced on ragged rows, partial column blocks,
    several token tiles and padded row strides: the result of the N:M
    product, element by element."""
    _expand_case(force_variant, "repack24_" + inner, dt, out, N, M, R, K, T, 13)


@pytest.mark.parametrize("dt", ["i8", "f16", "bf16"])
@pytest.mark.parametrize("N,M", REPACK_NMS)
@pytest.mark.parametrize("R,K", [(17, 96), (40, 264), (33, 520)])
def test_repack24_copy_describes_the_same_matrix(force_variant, dt, N, M, R, K):
    """The 2:4 copy in the workspace, decoded by the oracle, describes bit
    for bit the dense matrix the N:M packing describes (zeros, -0.0 and
    magnitude ties included), with two distinct ascending positions per
    group of four and padding slots as the packed format prescribes."""
    import torch
    import semi_structured_sparse_nm_amd as nm
    from tests._parity import TORCH_DT, dev
    inner = "smfmac_i8_2of4_persistent" if dt == "i8" else "smfmac_h_2of4_persistent"
    out = {"i8": "i32", "f16": "f16", "bf16": "bf16"}[dt]
    force_variant("repack24_" + inner)
    T = 16
    if dt == "i8":
        W = nm_inputs.uniform_int8((R, K), 2, "repack", dt, N, M, R, lo=-3, hi=3)
        W[0, :M] = -128
    else:
        W = nm_inputs.normal((R, K), 0.02, dt, 2, "repack", N, M, R)
        W[1, :M] = 0
        if dt == "f16":
            W[2, :M] = np.float16(-0.0)
    p = nm.pack(dev(W, dt), N, M)
    assert nm.variant(p, T, TORCH_DT[out]) == "repack24_" + inner
    need = nm.workspace_size(p, T, TORCH_DT[out])
    vb, mb = nm.pack_size(R, K, 2, 4, {"i8": nm.NM_I8, "f16": nm.NM_F16, "bf16": nm.NM_BF16}[dt])
    moff = (vb + 255) // 256 * 256
    assert need == moff + mb
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
    X = torch.zeros((K, T), dtype=TORCH_DT[dt], device="cuda")
    nm.spmm(p, X, out_dtype=TORCH_DT[out], workspace=ws)
    torch.cuda.synchronize()
    h = ws.cpu().numpy()
    v24, m24 = h[:vb], h[moff:moff + mb]
    vals, idx = oracle.read_packed(v24, m24, R, K, 2, 4, dt)
    assert np.all(idx[:, :, 0] < idx[:, :, 1])
    bits = np.uint8 if dt == "i8" else np.uint16
    cv, ci = oracle.compress(W, N, M, dt)
    want = oracle.decompress(cv, ci, R, K, N, M, dt)
    got = oracle.decompress(vals, idx, R, K, 2, 4, dt)
    assert np.array_equal(got.view(bits), want.view(bits))
    assert oracle.check_padding(v24, m24, R, K, 2, 4, dt) == 0


def test_repack24_small_workspace_runs_the_nm_kernel():
    """Given less workspace than the 2:4 copy needs, the call runs the N:M
    kernel instead, with the same result (int8: bit-exact)."""
    import ctypes
    import torch
    import semi_structured_sparse_nm_amd as nm
    R, K, T, N, M = 3072, 768, 1024, 1, 4
    W, X, b, s = _inputs("i8", "i8", R, K, T, N, M, 14, "repack-small-ws")
    p = nm.pack(torch.from_numpy(W).cuda(), N, M)
    assert nm.variant(p, T, torch.int8) == "repack24_smfmac_i8_2of4_persistent_w8"
    need = nm.workspace_size(p, T, torch.int8)
    assert need > 0
    Xd = torch.from_numpy(X).cuda()
    bd, sd = torch.from_numpy(b).cuda(), torch.from_numpy(s).cuda()
    ref = reference(W, X, N, M, "i8", "i8", bias=b, scale=s)
    small = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    for ws, wsb in ((None, 0), (small, need - 1)):
        Y = torch.full((R, T), 5, dtype=torch.int8, device="cuda")
        d = p.desc()
        st = nm.lib().nm_spmm(ctypes.byref(d), Xd.data_ptr(), T, T, Y.data_ptr(), T, nm.NM_I8, bd.data_ptr(),
                              sd.data_ptr(), None if ws is None else ws.data_ptr(), wsb, None)
        assert st == nm.NM_OK
        torch.cuda.synchronize()
        compare(Y.cpu().numpy(), ref, "i8", "small workspace")


# any int8 N:M split into two 2:4 layers in the workspace, then multiplied by
# the weight-stationary kernel over both layers (K in (640, 768])
SPLIT = "split24_smfmac_i8_stationary"
SPLIT_NMS = [(2, 4), (3, 4), (4, 4), (1, 8), (3, 8), (4, 8), (5, 8), (7, 8), (8, 8)]


@pytest.mark.parametrize("out", ["i8", "i32"])
@pytest.mark.parametrize("N,M", SPLIT_NMS)
@pytest.mark.parametrize("R,K,T", [(300, 768, 144), (520, 704, 400), (17, 648, 16), (1040, 768, 1008)])
def test_split24_variant(force_variant, out, N, M, R, K, T):
    """The two-layer path forced on ragged rows (partial row tiles and row
    blocks), a partial last column block (K 648, 704), partial last token
    steps, workgroups with no steps, and padded row strides: the result of
    the N:M product, element by element."""
    _expand_case(force_variant, SPLIT, "i8", out, N, M, R, K, T, 61)


@pytest.mark.parametrize("out", ["i8", "i32"])
@pytest.mark.parametrize("N,M", [(3, 4), (4, 8), (8, 8)])
def test_split24_many_steps(force_variant, out, N, M):
    """Eight row tiles of 256 rows over 256 workgroups: three 64-token steps
    per workgroup, so both stages alternate and each workgroup's steps
    follow its first."""
    _expand_case(force_variant, SPLIT, "i8", out, N, M, 2048, 768, 6144, 62)


DENSE = "dense24_smfmac_i8_stationary"


@pytest.mark.parametrize("out", ["i8", "i32"])
@pytest.mark.parametrize("N,M", [(4, 4), (8, 8)])
@pytest.mark.parametrize("R,K,T", [(300, 768, 144), (520, 704, 400), (17, 648, 16), (1040, 768, 1008),
                                   (2048, 768, 6144)])
def test_dense24_variant(force_variant, out, N, M, R, K, T):
    """Dense int8 weights through the two-layer kernel with the layers taken
    in registers (no copy): ragged rows, partial column blocks and steps,
    several steps per workgroup, padded strides; element by element."""
    _expand_case(force_variant, DENSE, "i8", out, N, M, R, K, T, 65)


def test_gelu_dense24(force_variant):
    """GELU fused into the dense form's epilogue."""
    _gelu_case(force_variant, DENSE, "i8", "i8", 8, 8, 300, 768, 144, 66)


@pytest.mark.parametrize("N,M", [(3, 4), (4, 4), (1, 8), (4, 8), (6, 8), (8, 8)])
@pytest.mark.parametrize("R,K", [(17, 648), (40, 768), (33, 704)])
def test_split24_copy_describes_the_same_matrix(force_variant, N, M, R, K):
    """The two 2:4 layers in the workspace, each decoded by the oracle as a
    2:4 packing, add up bit for bit to the dense matrix the N:M packing
    describes (ties, zeros and -128 included); each layer has two distinct
    ascending positions per group of four and clean padding; no position
    holds a nonzero in both layers."""
    import torch
    import semi_structured_sparse_nm_amd as nm
    force_variant(SPLIT)
    T = 16
    W = nm_inputs.uniform_int8((R, K), 5, "split", N, M, R, lo=-3, hi=3)
    W[0, :M] = -128
    W[1, :M] = 0
    p = nm.pack(torch.from_numpy(W).cuda(), N, M)
    assert nm.variant(p, T, torch.int32) == SPLIT
    vb, mb = nm.pack_size(R, K, 2, 4, nm.NM_I8)
    moff = (vb + 255) // 256 * 256
    layer = (moff + mb + 255) // 256 * 256
    need = nm.workspace_size(p, T, torch.int32)
    assert need == 2 * layer
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
    X = torch.zeros((K, T), dtype=torch.int8, device="cuda")
    nm.spmm(p, X, out_dtype=torch.int32, workspace=ws)
    torch.cuda.synchronize()
    h = ws.cpu().numpy()
    cv, ci = oracle.compress(W, N, M, "i8")
    want = oracle.decompress(cv, ci, R, K, N, M, "i8").astype(np.int32)
    got = np.zeros((R, K), np.int32)
    nonzero = np.zeros((R, K), np.int32)
    for l in range(2):
        v24, m24 = h[l * layer:l * layer + vb], h[l * layer + moff:l * layer + moff + mb]
        vals, idx = oracle.read_packed(v24, m24, R, K, 2, 4, "i8")
        assert np.all(idx[:, :, 0] < idx[:, :, 1]), l
        assert oracle.check_padding(v24, m24, R, K, 2, 4, "i8") == 0, l
        d = oracle.decompress(vals, idx, R, K, 2, 4, "i8").astype(np.int32)
        got += d
        nonzero += d != 0
    assert np.array_equal(got, want)
    assert nonzero.max() <= 1


@pytest.mark.parametrize("N,M", [(3, 4), (4, 8)])
def test_gelu_split24(force_variant, N, M):
    """GELU fused into the two-layer kernel's epilogue."""
    _gelu_case(force_variant, SPLIT, "i8", "i8", N, M, 300, 768, 144, 63)


def test_split24_small_workspace_runs_the_nm_kernel():
    """Given less workspace than the two layers need, the call runs the
    dense-expand kernel instead, with the same (bit-exact) result."""
    import ctypes
    import torch
    import semi_structured_sparse_nm_amd as nm
    R, K, T, N, M = 3072, 768, 1024, 4, 8
    W, X, b, s = _inputs("i8", "i8", R, K, T, N, M, 64, "split-small-ws")
    p = nm.pack(torch.from_numpy(W).cuda(), N, M)
    assert nm.variant(p, T, torch.int8) == SPLIT
    need = nm.workspace_size(p, T, torch.int8)
    assert need > 0
    Xd = torch.from_numpy(X).cuda()
    bd, sd = torch.from_numpy(b).cuda(), torch.from_numpy(s).cuda()
    ref = reference(W, X, N, M, "i8", "i8", bias=b, scale=s)
    small = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    full = torch.empty(need, dtype=torch.uint8, device="cuda")
    for ws, wsb in ((None, 0), (small, need - 1), (full, need)):
        Y = torch.full((R, T), 5, dtype=torch.int8, device="cuda")
        d = p.desc()
        st = nm.lib().nm_spmm(ctypes.byref(d), Xd.data_ptr(), T, T, Y.data_ptr(), T, nm.NM_I8, bd.data_ptr(),
                              sd.data_ptr(), None if ws is None else ws.data_ptr(), wsb, None)
        assert st == nm.NM_OK
        torch.cuda.synchronize()
        compare(Y.cpu().numpy(), ref, "i8", f"workspace {wsb}")


def _expand_decode_case(force_variant, dt, out, N, M, R, K, T, seed):
    import semi_structured_sparse_nm_amd as nm
    from tests._parity import TORCH_DT, dev
    force_variant("expand_mfma_decode")
    W, X, b, s = _inputs(dt, out, R, K, T, N, M, seed, f"expdec-{dt}-{out}-{N}-{M}-{R}-{K}-{T}")
    p = nm.pack(dev(W, dt), N, M)
    # nm_spmm_variant assumes dense rows (ldx = T); the run pads X rows to a
    # multiple of 16 elements, which the forced kernel needs
    if T % 16 == 0:
        assert nm.variant(p, T, TORCH_DT[out]) == "expand_mfma_decode"
    Y, _ = run(W, X, N, M, dt, out, bias=b, scale=s, ldx_pad=(-T) % 16 + 16, ldy_pad=3, sentinel=5)
    compare(Y[:, :T], reference(W, X, N, M, dt, out, bias=b, scale=s), out, f"expand decode {N}:{M}")
    pad = Y[:, T:]
    want = 5 if out != "bf16" else oracle.round_to(np.array([5.0]), "bf16")[0]
    assert np.all(pad == want), "writes beyond T"


@pytest.mark.parametrize("dt,out", PAIRS)
@pytest.mark.parametrize("N,M", NMS)
@pytest.mark.parametrize("R,K,T", [(17, 8, 1), (300, 200, 3), (96, 4104, 16)])
def test_expand_decode_variant(force_variant, dt, out, N, M, R, K, T):
    """Decode kernel (K split over eight waves, windows expanded in registers,
    partials summed in LDS in wave order) forced: fewer column blocks than
    waves, partial blocks, ragged rows, T < 16, every N:M and dtype pair."""
    _expand_decode_case(force_variant, dt, out, N, M, R, K, T, 13)


@pytest.mark.parametrize("dt,out", [("i8", "i8"), ("f16", "f16"), ("bf16", "f32")])
@pytest.mark.parametrize("N,M", [(1, 4), (3, 4), (4, 8), (8, 8)])
@pytest.mark.parametrize("R,K,T", [(16, 64, 16), (40, 512, 8), (33, 11008, 16)])
def test_expand_decode_variant_more_shapes(force_variant, dt, out, N, M, R, K, T):
    _expand_decode_case(force_variant, dt, out, N, M, R, K, T, 14)


@pytest.fixture
def force_ksplit():
    import os
    old = os.environ.get("NM_SPMM_VARIANT")
    yield lambda S: _set_forced(S=S)
    if old is None:
        os.environ.pop("NM_SPMM_VARIANT", None)
    else:
        os.environ["NM_SPMM_VARIANT"] = old


def _ksplit_case(force_variant, force_ksplit, variant, dt, out, N, M, R, K, T, S, ldy_pad, seed):
    import semi_structured_sparse_nm_amd as nm
    from tests._parity import TORCH_DT, dev
    force_variant(variant)
    force_ksplit(S)
    W, X, b, s = _inputs(dt, out, R, K, T, N, M, seed, f"ksplit-{variant}-{dt}-{out}-{N}-{M}-{R}-{K}-{T}-{S}")
    p = nm.pack(dev(W, dt), N, M)
    assert nm.variant(p, T, TORCH_DT[out]) == variant
    assert nm.ksplit(p, T, TORCH_DT[out]) == S
    assert nm.workspace_size(p, T, TORCH_DT[out]) == (S * R * T * 4 if S > 1 else 0)
    Y, _ = run(W, X, N, M, dt, out, bias=b, scale=s, ldx_pad=32, ldy_pad=ldy_pad, sentinel=5)
    compare(Y[:, :T], reference(W, X, N, M, dt, out, bias=b, scale=s), out, f"{variant} K split {S}")
    pad = Y[:, T:]
    want = 5 if out != "bf16" else oracle.round_to(np.array([5.0]), "bf16")[0]
    assert np.all(pad == want), "writes beyond T"


# (R, K, T, S): several row and token tiles with ragged edges; slices of one,
# two and several column blocks; a partial last column block (K = 1000)
KSPLIT_SHAPES = [(300, 1536, 400, 4), (520, 768, 144, 3), (64, 4096, 32, 8), (259, 1024, 272, 2),
                 (130, 1000, 160, 4)]


@pytest.mark.parametrize("variant", FAST_H)
@pytest.mark.parametrize("dt,out", [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("R,K,T,S", KSPLIT_SHAPES)
@pytest.mark.parametrize("ldy_pad", [8, 3])
def test_ksplit_h(force_variant, force_ksplit, variant, dt, out, R, K, T, S, ldy_pad):
    """fp16 / bf16 2:4 tile kernel with K cut into S slices across
    workgroups: fp32 partials in the workspace, reduced in slice order with
    the bias and the output rounding; aligned (vector) and unaligned
    (element) output rows."""
    _ksplit_case(force_variant, force_ksplit, variant, dt, out, 2, 4, R, K, T, S, ldy_pad, 21)


@pytest.mark.parametrize("dt,out", PAIRS)
@pytest.mark.parametrize("N,M", [(1, 4), (4, 8), (8, 8)])
@pytest.mark.parametrize("R,K,T,S", KSPLIT_SHAPES)
def test_ksplit_expand(force_variant, force_ksplit, dt, out, N, M, R, K, T, S):
    """Dense-expand kernel with K cut into S slices across workgroups; int32
    partials for int8 (exact, then bias and requantisation), fp32 otherwise."""
    nkb = -(-K // (128 if dt == "i8" else 64))
    if nkb % S:
        S = 2 if nkb % 2 == 0 else 1
    _ksplit_case(force_variant, force_ksplit, "expand_mfma_persistent", dt, out, N, M, R, K, T, S,
                 16 if out in ("i8", "f16", "bf16") else 3, 22)


# ---------------------------------------------------------------- fused GELU
# int8: the dequantising scale maps the layer's int8 output range onto about
# [-4, 4] (so the activation's curved part is exercised), out_scale maps it back
GELU_SPAN = 4.0


def _gelu_case(force_variant, variant, dt, out, N, M, R, K, T, seed, S=None, force_ksplit=None):
    import semi_structured_sparse_nm_amd as nm
    from tests._parity import TORCH_DT, compare_i8_open, dev
    force_variant(variant)
    if S is not None:
        force_ksplit(S)
    W, X, b, s = _inputs(dt, out, R, K, T, N, M, seed, f"gelu-{variant}-{dt}-{out}-{N}-{M}-{R}-{K}-{T}")
    p = nm.pack(dev(W, dt), N, M)
    # nm_spmm_variant assumes dense rows (ldx = T); the run pads X rows to a
    # multiple of 16 elements, which the forced kernels need
    if T % 16 == 0:
        assert nm.variant(p, T, TORCH_DT[out], act="gelu") == variant
    if S is not None:
        assert nm.ksplit(p, T, TORCH_DT[out], act="gelu") == S
    narrow = out in ("i8", "f16", "bf16")
    pad = dict(ldx_pad=(-T) % 16 + 16, ldy_pad=16 if narrow else 3, sentinel=5)
    if dt == "i8":
        sd = (np.asarray(s, np.float32) * np.float32(GELU_SPAN / 127.0)).astype(np.float32)
        osc = 127.0 / GELU_SPAN
        Y, _ = run(W, X, N, M, dt, out, bias=b, scale=sd, act="gelu", out_scale=osc, **pad)
        ref, near = reference(W, X, N, M, dt, out, bias=b, scale=sd, act="gelu", out_scale=osc)
        compare_i8_open(Y[:, :T], ref, near, f"{variant} gelu")
    else:
        Y, _ = run(W, X, N, M, dt, out, bias=b, act="gelu", **pad)
        compare(Y[:, :T], reference(W, X, N, M, dt, out, bias=b, act="gelu"), out, f"{variant} gelu")
    want = 5 if out != "bf16" else oracle.round_to(np.array([5.0]), "bf16")[0]
    assert np.all(Y[:, T:] == want), "writes beyond T"


@pytest.mark.parametrize("inner,dt,out", [("smfmac_i8_2of4_persistent", "i8", "i8"),
                                          ("smfmac_i8_2of4_persistent_w8", "i8", "i8"),
                                          ("smfmac_h_2of4_persistent", "f16", "f16")])
@pytest.mark.parametrize("N,M", [(1, 4), (2, 8)])
@pytest.mark.parametrize("R,K,T", [(300, 192, 144), (259, 1288, 272)])
def test_gelu_repack24(force_variant, inner, dt, out, N, M, R, K, T):
    """GELU fused into the re-packed path (the 2:4 kernel's epilogue)."""
    _gelu_case(force_variant, "repack24_" + inner, dt, out, N, M, R, K, T, 33)


GELU_FP = [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32")]
GELU_SHAPES = [(300, 192, 144), (259, 1280, 272)]


@pytest.mark.parametrize("dt,out", [("i8", "i8")] + GELU_FP)
@pytest.mark.parametrize("N,M", [(2, 4), (1, 4), (4, 8)])
@pytest.mark.parametrize("R,K,T", GELU_SHAPES)
def test_gelu_expand(force_variant, dt, out, N, M, R, K, T):
    """Dense-expand tile kernel with GELU fused; 2:4 included (with an
    activation it carries the int8 2:4 shapes the stationary kernel cannot)."""
    _gelu_case(force_variant, "expand_mfma_persistent", dt, out, N, M, R, K, T, 32)


@pytest.mark.parametrize("variant", FAST_H)
@pytest.mark.parametrize("dt,out", GELU_FP)
@pytest.mark.parametrize("R,K,T", GELU_SHAPES)
def test_gelu_h(force_variant, variant, dt, out, R, K, T):
    _gelu_case(force_variant, variant, dt, out, 2, 4, R, K, T, 33)


@pytest.mark.parametrize("dt,out", [("i8", "i8")] + GELU_FP)
@pytest.mark.parametrize("N,M", [(2, 4), (4, 8)])
@pytest.mark.parametrize("R,K,T", [(40, 512, 8), (33, 1280, 16)])
def test_gelu_decode(force_variant, dt, out, N, M, R, K, T):
    variant = "smfmac_h_2of4_decode" if (dt != "i8" and (N, M) == (2, 4)) else "expand_mfma_decode"
    _gelu_case(force_variant, variant, dt, out, N, M, R, K, T, 34)


@pytest.mark.parametrize("dt,out", GELU_FP)
@pytest.mark.parametrize("R,K,T", [(40, 512, 8), (600, 1280, 16)])
def test_gelu_stream24(force_variant, dt, out, R, K, T):
    _gelu_case(force_variant, "smfmac_h_2of4_stream_decode", dt, out, 2, 4, R, K, T, 36)


@pytest.mark.parametrize("dt,out", [("i8", "i8"), ("f16", "f16"), ("bf16", "f32")])
@pytest.mark.parametrize("R,K,T", [(70, 192, 197), (17, 64, 5)])
def test_gelu_generic(force_variant, dt, out, R, K, T):
    _gelu_case(force_variant, "generic_dense_expand", dt, out, 2, 4, R, K, T, 35)


@pytest.mark.parametrize("variant,dt,out", [("expand_mfma_persistent", "i8", "i8"),
                                            ("expand_mfma_persistent", "f16", "f16"),
                                            ("smfmac_h_2of4_persistent", "bf16", "bf16"),
                                            ("smfmac_h_2of4_persistent", "f16", "f32")])
def test_gelu_ksplit(force_variant, force_ksplit, variant, dt, out):
    """K split with GELU: the slices' partials are raw; the reduction applies
    bias, the activation and the output rounding or requantisation."""
    _gelu_case(force_variant, variant, dt, out, 2, 4, 300, 1536, 400, 36, S=4, force_ksplit=force_ksplit)


@pytest.mark.parametrize("R1,K1,T", [(3072, 768, 400), (520, 192, 144)])
def test_mlp_chain_fc1_gelu_fc2_int8(R1, K1, T):
    """ViT-B MLP in int8 without leaving the device: FC1 (2:4) with GELU
    fused requantises to int8, and its [R1][T] output is FC2's [K][T]
    activation as it stands.  FC1 against the oracle (closed decisions
    exact, open ones within a code); FC2 against the oracle chain, exact in
    every token column where both FC1 results agree, and elsewhere within the
    bound a one-code change of its inputs allows."""
    import torch
    import semi_structured_sparse_nm_amd as nm
    from tests._parity import compare_i8_open
    c = nm_inputs.mlp_chain(R1, K1, T, 2, 4, 0, f"chain-{R1}-{K1}-{T}")
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    p1, p2 = nm.pack(d(c.W1), 2, 4), nm.pack(d(c.W2), 2, 4)
    h = nm.spmm(p1, d(c.X), bias=d(c.b1), scale=d(c.s_deq1), out_dtype=torch.int8, act="gelu",
                out_scale=c.os1)
    y = nm.spmm(p2, h, bias=d(c.b2), scale=d(c.scale2), out_dtype=torch.int8)
    torch.cuda.synchronize()
    h_gpu, y_gpu = h.cpu().numpy(), y.cpu().numpy()
    h_ref, near = oracle.reference(c.W1, c.X, 2, 4, "i8", "i8", bias=c.b1, scale=c.s_deq1, act="gelu",
                                   out_scale=c.os1)
    ndiff = compare_i8_open(h_gpu, h_ref, near, "fc1 gelu")
    y_ref = oracle.reference(c.W2, h_ref, 2, 4, "i8", "i8", bias=c.b2, scale=c.scale2)
    cols = (h_gpu != h_ref).any(axis=0)
    assert ndiff == int((h_gpu != h_ref).sum())
    assert np.array_equal(y_gpu[:, ~cols], y_ref[:, ~cols])
    if cols.any():
        vals, idx = oracle.compress(c.W2, 2, 4, "i8")
        wm = np.abs(oracle.decompress(vals, idx, c.W2.shape[0], c.W2.shape[1], 2, 4, "i8").astype(np.int64))
        dh = np.abs(h_gpu[:, cols].astype(np.int64) - h_ref[:, cols].astype(np.int64))
        bound = np.ceil((wm @ dh) * c.scale2[:, None].astype(np.float64)) + 1
        assert np.all(np.abs(y_gpu[:, cols].astype(np.int64) - y_ref[:, cols]) <= bound)
    # the hidden activations are not degenerate (they use the int8 range)
    assert (np.abs(h_ref.astype(np.int64)) > 10).mean() > 0.05


def test_mlp_chain_full_size_sampled_columns():
    """The ViT-B MLP at batch 64 (T = 12608) in the launch configuration the
    chain benchmark times; token columns are independent, so the oracle chain
    on 48 sampled columns (the first, the last, the rest seeded) checks them
    exactly, under the same rule as the small chain test."""
    import torch
    import semi_structured_sparse_nm_amd as nm
    from tests._parity import compare_i8_open
    T = nm_inputs.VIT_B_TOKENS
    c = nm_inputs.mlp_chain(3072, 768, T, 2, 4, 0, "vitb_mlp")
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    p1, p2 = nm.pack(d(c.W1), 2, 4), nm.pack(d(c.W2), 2, 4)
    h = nm.spmm(p1, d(c.X), bias=d(c.b1), scale=d(c.s_deq1), out_dtype=torch.int8, act="gelu",
                out_scale=c.os1)
    y = nm.spmm(p2, h, bias=d(c.b2), scale=d(c.scale2), out_dtype=torch.int8)
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(3).integers(0, T, 46)]))
    h_gpu, y_gpu = h.cpu().numpy()[:, cols], y.cpu().numpy()[:, cols]
    Xs = np.ascontiguousarray(c.X[:, cols])
    h_ref, near = oracle.reference(c.W1, Xs, 2, 4, "i8", "i8", bias=c.b1, scale=c.s_deq1, act="gelu",
                                   out_scale=c.os1)
    compare_i8_open(h_gpu, h_ref, near, "fc1 gelu full size")
    y_ref = oracle.reference(c.W2, h_ref, 2, 4, "i8", "i8", bias=c.b2, scale=c.scale2)
    agree = ~(h_gpu != h_ref).any(axis=0)
    assert agree.sum() >= len(cols) // 2
    assert np.array_equal(y_gpu[:, agree], y_ref[:, agree])


@pytest.mark.parametrize("variant", FAST_I8)
@pytest.mark.parametrize("R,K,T", [(300, 192, 144), (520, 768, 400), (259, 1280, 272)])
def test_gelu_i8_persistent(force_variant, variant, R, K, T):
    """int8 2:4 persistent kernels (the ViT-B FC1 default) with GELU fused
    between the dequantising and the requantising scale."""
    _gelu_case(force_variant, variant, "i8", "i8", 2, 4, R, K, T, 37)


# ---------------------------------------------------------------- [T][K] layout
def _tk_case(dt, out, N, M, R, K, T, seed, act="none", xpad=24, variant=None):
    """nm_spmm_tk on padded row strides: Yt [T][R] against the oracle's
    [R][T] result, element by element; nothing written past R."""
    import torch
    import semi_structured_sparse_nm_amd as nm
    from tests._parity import TORCH_DT, compare_i8_open, dev, host
    W, X, b, s = _inputs(dt, out, R, K, T, N, M, seed, f"tk-{dt}-{out}-{N}-{M}-{R}-{K}-{T}-{act}")
    p = nm.pack(dev(W, dt), N, M)
    if variant is not None and K % 16 == 0:
        assert nm.variant_tk(p, T, TORCH_DT[out], act=act) == variant
    Xfull = torch.zeros((T, K + xpad), dtype=TORCH_DT[dt], device="cuda")
    Xfull[:, :K] = dev(np.ascontiguousarray(X.T), dt)
    Yfull = torch.full((T, R + 16), 5, dtype=TORCH_DT[out], device="cuda")
    kw = {}
    sd, osc = s, 1.0
    if dt == "i8" and act == "gelu":
        sd = (np.asarray(s, np.float32) * np.float32(GELU_SPAN / 127.0)).astype(np.float32)
        osc = 127.0 / GELU_SPAN
    bias = None if b is None else torch.from_numpy(np.asarray(b)).cuda()
    scale = None if sd is None else torch.from_numpy(np.asarray(sd, np.float32)).cuda()
    nm.linear(p, Xfull[:, :K], bias=bias, scale=scale, out_dtype=TORCH_DT[out], out=Yfull[:, :R], act=act,
              out_scale=osc)
    torch.cuda.synchronize()
    Y = host(Yfull, out)
    Yt = np.ascontiguousarray(Y[:, :R].T)
    if dt == "i8" and act == "gelu":
        ref, near = reference(W, X, N, M, dt, out, bias=b, scale=sd, act=act, out_scale=osc)
        compare_i8_open(Yt, ref, near, "tk gelu")
    else:
        compare(Yt, reference(W, X, N, M, dt, out, bias=b, scale=sd, act=act), out, f"tk {N}:{M}")
    want = 5 if out != "bf16" else oracle.round_to(np.array([5.0]), "bf16")[0]
    assert np.all(Y[:, R:] == want), "writes beyond R"


@pytest.mark.parametrize("out", ["i8", "i32"])
@pytest.mark.parametrize("N,M", [(3, 4), (4, 4), (1, 8), (4, 8), (7, 8), (8, 8)])
@pytest.mark.parametrize("R,K,T", [(304, 768, 144), (528, 704, 400), (16, 656, 16), (1040, 768, 1008)])
def test_tk_two_layer(force_variant, out, N, M, R, K, T):
    """The two-layer kernel in the [T][K] layout (split copy, or the dense
    form's layers in registers), forced on partial row tiles, partial column
    blocks and steps, padded strides: element by element, nothing written
    past R."""
    variant = ("dense24" if N == M else "split24") + "_smfmac_i8_stationary_tk"
    force_variant(variant)
    _tk_case("i8", out, N, M, R, K, T, 67, xpad=16, variant=variant)


@pytest.mark.parametrize("out", ["i8", "i32"])
@pytest.mark.parametrize("N,M", [(4, 8), (8, 8)])
def test_tk_two_layer_many_steps(force_variant, out, N, M):
    """Three 64-token steps per workgroup in the [T][K] layout."""
    variant = ("dense24" if N == M else "split24") + "_smfmac_i8_stationary_tk"
    force_variant(variant)
    _tk_case("i8", out, N, M, 2048, 768, 6144, 68, xpad=16, variant=variant)


@pytest.mark.parametrize("N,M", [(4, 8), (8, 8)])
def test_tk_two_layer_gelu(force_variant, N, M):
    variant = ("dense24" if N == M else "split24") + "_smfmac_i8_stationary_tk"
    force_variant(variant)
    _tk_case("i8", "i8", N, M, 528, 768, 400, 69, act="gelu", xpad=16, variant=variant)


def test_tk_split24_small_workspace_runs_another_kernel():
    """nm_spmm_tk on a 4:8 weight with less workspace than the two-layer split
    needs runs another kernel (no copy), with the same bit-exact result;
    with the full workspace it runs the split."""
    import ctypes
    import torch
    import semi_structured_sparse_nm_amd as nm
    R, K, T, N, M = 3072, 768, 1024, 4, 8
    W, X, b, s = _inputs("i8", "i8", R, K, T, N, M, 70, "tk-split-small-ws")
    p = nm.pack(torch.from_numpy(W).cuda(), N, M)
    assert nm.variant_tk(p, T, torch.int8) == "split24_smfmac_i8_stationary_tk"
    need = nm.workspace_size_tk(p, T, torch.int8)
    assert need > 0
    Xt = torch.from_numpy(np.ascontiguousarray(X.T)).cuda()
    bd, sd = torch.from_numpy(b).cuda(), torch.from_numpy(s).cuda()
    ref = reference(W, X, N, M, "i8", "i8", bias=b, scale=s)
    small = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    full = torch.empty(need, dtype=torch.uint8, device="cuda")
    for ws, wsb in ((None, 0), (small, need - 1), (full, need)):
        Yt = torch.full((T, R), 5, dtype=torch.int8, device="cuda")
        d = p.desc()
        st = nm.lib().nm_spmm_tk(ctypes.byref(d), Xt.data_ptr(), K, T, Yt.data_ptr(), R, nm.NM_I8, bd.data_ptr(),
                                 sd.data_ptr(), 0, 1.0, None if ws is None else ws.data_ptr(), wsb, None)
        assert st == nm.NM_OK
        torch.cuda.synchronize()
        compare(np.ascontiguousarray(Yt.cpu().numpy().T), ref, "i8", f"tk workspace {wsb}")


@pytest.mark.parametrize("dt,out", PAIRS)
@pytest.mark.parametrize("N,M", [(2, 4), (1, 4), (3, 4), (4, 8), (8, 8)])
@pytest.mark.parametrize("R,K,T", [(17, 8, 1), (300, 200, 37), (259, 1288, 144)])
def test_tk_layout(dt, out, N, M, R, K, T):
    """The PyTorch-linear layout (X [T][K], Y [T][R]) for every dtype pair,
    several N:M, ragged rows, tokens and column blocks, padded strides."""
    _tk_case(dt, out, N, M, R, K, T, 41)


@pytest.mark.parametrize("dt,out", [("i8", "i8"), ("f16", "f16"), ("bf16", "f32")])
def test_tk_layout_gelu(dt, out):
    _tk_case(dt, out, 2, 4, 300, 200, 37, 42, act="gelu")


@pytest.mark.parametrize("out", ["i8", "i32"])
@pytest.mark.parametrize("R,K,T", [(256, 192, 144), (3072, 768, 1008), (528, 1280, 272), (16, 128, 16),
                                   (304, 200, 37)])
def test_tk_fast_i8(force_variant, out, R, K, T):
    """The int8 2:4 persistent kernel of the [T][K] layout: several row and
    token tiles, tokens past T, K not a multiple of 128 (a token row's bytes
    past K meet zero weights), 16-byte-aligned padded strides."""
    force_variant("smfmac_i8_2of4_tk")
    _tk_case("i8", out, 2, 4, R, K, T, 43, xpad=(-K) % 16 + 16, variant="smfmac_i8_2of4_tk")


def test_tk_fast_i8_gelu(force_variant):
    force_variant("smfmac_i8_2of4_tk")
    _tk_case("i8", "i8", 2, 4, 528, 768, 400, 44, act="gelu", xpad=16, variant="smfmac_i8_2of4_tk")


# the weight-stationary int8 2:4 kernel of the [T][K] layout: K in (640, 768]
# (six column blocks in registers), R a multiple of 16
STAT_TK_SHAPES = [(528, 768, 400), (304, 700, 37), (16, 656, 16), (3072, 768, 1008), (2304, 768, 1040),
                  (3072, 768, 12608)]


@pytest.mark.parametrize("out", ["i8", "i32"])
@pytest.mark.parametrize("R,K,T", STAT_TK_SHAPES)
def test_tk_stationary_i8(force_variant, out, R, K, T):
    """The weight-stationary kernel in the [T][K] layout: several row tiles
    (rows of the last one past R), token steps with tokens past T, K not a
    multiple of 128 (a token row's bytes past K meet zero weights), padded
    strides, the full ViT-B FC1; nothing written past R."""
    force_variant("smfmac_i8_2of4_stationary_tk")
    _tk_case("i8", out, 2, 4, R, K, T, 51, xpad=(-K) % 16 + 16, variant="smfmac_i8_2of4_stationary_tk")


def test_tk_stationary_i8_gelu(force_variant):
    force_variant("smfmac_i8_2of4_stationary_tk")
    _tk_case("i8", "i8", 2, 4, 528, 768, 400, 52, act="gelu", xpad=16, variant="smfmac_i8_2of4_stationary_tk")


@pytest.mark.parametrize("N,M", [(1, 4), (2, 8)])
def test_tk_stationary_repack24(force_variant, N, M):
    force_variant("repack24_smfmac_i8_2of4_stationary_tk")
    _tk_case("i8", "i8", N, M, 528, 768, 400, 53, xpad=16, variant="repack24_smfmac_i8_2of4_stationary_tk")


@pytest.mark.parametrize("out", ["i8", "i32"])
@pytest.mark.parametrize("N,M", [(1, 4), (1, 8), (2, 8)])
@pytest.mark.parametrize("R,K,T", [(256, 192, 144), (528, 1288, 272), (304, 200, 37)])
def test_tk_repack24(force_variant, out, N, M, R, K, T):
    """1:4, 1:8 and 2:8 int8 in the [T][K] layout, re-packed to 2:4 in the
    workspace and multiplied by the layout's int8 2:4 kernel."""
    force_variant("repack24_smfmac_i8_2of4_tk")
    _tk_case("i8", out, N, M, R, K, T, 45, xpad=(-K) % 16 + 16, variant="repack24_smfmac_i8_2of4_tk")


TRANSPOSE_CASES = [("expand_mfma_persistent", "i8", "i8", 4, 8), ("expand_mfma_persistent", "f16", "f16", 1, 4),
                   ("expand_mfma_persistent", "bf16", "f32", 8, 8), ("smfmac_h_2of4_persistent", "f16", "f16", 2, 4),
                   ("smfmac_h_2of4_persistent", "bf16", "bf16", 2, 4),
                   ("smfmac_i8_2of4_persistent", "i8", "i32", 2, 4), ("smfmac_i8_2of4_persistent_w8", "i8", "i8", 2, 4)]


@pytest.mark.parametrize("inner,dt,out,N,M", TRANSPOSE_CASES)
@pytest.mark.parametrize("R,K,T", [(256, 192, 144), (304, 1288, 37), (520, 776, 400)])
def test_tk_transpose(force_variant, inner, dt, out, N, M, R, K, T):
    """[T][K] calls run as transpose, [K][T] product, transpose: every dtype
    pair and several kernels, T not a multiple of 16 (zero tokens pad the
    product), ragged rows and column blocks, padded strides; nothing written
    past R."""
    force_variant("transpose_" + inner)
    _tk_case(dt, out, N, M, R, K, T, 47, xpad=(-K) % 16 + 16, variant="transpose_" + inner)


def test_tk_transpose_decode(force_variant):
    force_variant("transpose_smfmac_h_2of4_decode")
    _tk_case("f16", "f16", 2, 4, 300, 1024, 7, 48, xpad=8, variant="transpose_smfmac_h_2of4_decode")


def test_tk_transpose_gelu_and_ksplit(force_variant, force_ksplit):
    import semi_structured_sparse_nm_amd as nm
    force_variant("transpose_expand_mfma_persistent")
    _tk_case("i8", "i8", 4, 8, 264, 1024, 144, 49, act="gelu", xpad=16, variant="transpose_expand_mfma_persistent")
    force_ksplit(4)
    _tk_case("f16", "f16", 1, 4, 264, 1024, 144, 50, xpad=16, variant="transpose_expand_mfma_persistent")


def test_tk_repack24_gelu(force_variant):
    force_variant("repack24_smfmac_i8_2of4_tk")
    _tk_case("i8", "i8", 1, 4, 528, 768, 400, 46, act="gelu", xpad=16, variant="repack24_smfmac_i8_2of4_tk")
