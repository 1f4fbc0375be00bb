"""Seeded synthetic inputs for the N:M sparse x dense product.

Shared by the tests, the benchmark and the smoke check on both sides (the CPU
oracle and the GPU library).  It holds no arithmetic of the product itself:
only random draws, the quantisation that turns synthetic fp64 data into int8
operands, and the workload shapes.

The workloads stand in for the paper's ViT / Swin image inference (arXiv
2607.12505, Sec. 2.1: time goes to the Q/K/V, attention-output and two FFN
linear layers) and for LLaMA-7B-sized projections; no dataset or trained
weight is needed because only shapes and value distributions matter to the
kernel.  Every stream is derived from (seed, name) so each tensor is
reproducible on its own.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import numpy as np


def rng(seed: int, *names) -> np.random.Generator:
    """Independent, reproducible generator for (seed, name, ...)."""
    key = [int(seed)] + [zlib.crc32(str(n).encode()) for n in names]
    return np.random.default_rng(np.random.SeedSequence(key))


def uniform_int8(shape, seed: int, *names, lo: int = -127, hi: int = 127) -> np.ndarray:
    """Integers uniform in [lo, hi] as int8."""
    return rng(seed, *names).integers(lo, hi + 1, size=shape).astype(np.int8)


def _bf16_bits(x64: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 raw bits, round half to even in one step."""
    m, e = np.frexp(x64)
    y = np.ldexp(np.rint(m * 256.0), e - 8).astype(np.float32)
    return (y.view(np.uint32) >> 16).astype(np.uint16)


def normal(shape, sigma: float, dt: str, seed: int, *names) -> np.ndarray:
    """N(0, sigma^2) in fp64, rounded to nearest-even in dtype 'f16' / 'bf16' / 'f32'.

    bf16 comes back as uint16 raw bits (numpy has no bfloat16)."""
    x = rng(seed, *names).standard_normal(size=shape) * sigma
    if dt == "f16":
        return x.astype(np.float16)
    if dt == "bf16":
        return _bf16_bits(x)
    if dt == "f32":
        return x.astype(np.float32)
    raise ValueError(dt)


@dataclass
class QuantLayer:
    """One int8 linear layer: W[R][K], X[K][T], bias int32[R], scale f32[R]."""
    W: np.ndarray
    X: np.ndarray
    bias: np.ndarray
    scale: np.ndarray
    s_w: np.ndarray = field(repr=False)
    s_x: float = 0.0


def quant_layer(R: int, K: int, T: int, N: int, M: int, seed: int, *names,
                w_sigma: float = 0.02, x_sigma: float = 1.0, b_sigma: float = 0.02) -> QuantLayer:
    """Synthetic int8 layer (ViT-B style).

    W ~ N(0, w_sigma^2) quantised per row: s_w[r] = max_k |w| / 127,
    q = clamp(rne(w / s_w), -127, 127); X ~ N(0, x_sigma^2) quantised per
    tensor the same way; bias_f ~ N(0, b_sigma^2) -> int32 rne(bias_f / (s_w s_x)).
    The output scale is chosen from input statistics only, so that four
    standard deviations of a row's expected output span the int8 range:
        scale[r] = f32(127 / (4 sqrt((N/M) sum_k q_w[r,k]^2 mean(q_x^2)) + 1)).
    Rare outliers therefore saturate, which the epilogue must handle.
    """
    w = rng(seed, *names, "W").standard_normal((R, K)) * w_sigma
    x = rng(seed, *names, "X").standard_normal((K, T)) * x_sigma
    bf = rng(seed, *names, "bias").standard_normal(R) * b_sigma
    s_w = np.abs(w).max(axis=1) / 127.0
    s_w[s_w == 0] = 1.0
    qw = np.clip(np.rint(w / s_w[:, None]), -127, 127).astype(np.int8)
    s_x = float(np.abs(x).max() / 127.0) or 1.0
    qx = np.clip(np.rint(x / s_x), -127, 127).astype(np.int8)
    bias = np.rint(bf / (s_w * s_x)).astype(np.int32)
    ex2 = float(np.mean(qx.astype(np.float64) ** 2))
    row = (N / M) * (qw.astype(np.float64) ** 2).sum(axis=1) * ex2
    scale = (127.0 / (4.0 * np.sqrt(row) + 1.0)).astype(np.float32)
    return QuantLayer(W=qw, X=qx, bias=bias, scale=scale, s_w=s_w, s_x=s_x)


@dataclass
class MlpChain:
    """Two int8 layers of a Transformer MLP with GELU between them:
    h = sat(rne(gelu(f32(W1 X + b1) * s_deq1[r]) * os1)), Y = requant(W2 h + b2, scale2)."""
    W1: np.ndarray
    X: np.ndarray
    b1: np.ndarray
    s_deq1: np.ndarray
    os1: float
    W2: np.ndarray
    b2: np.ndarray
    scale2: np.ndarray


def mlp_chain(R1: int, K1: int, T: int, N: int, M: int, seed: int, *names,
              w_sigma: float = 0.02, x_sigma: float = 1.0, b_sigma: float = 0.02) -> MlpChain:
    """Synthetic int8 MLP (ViT-B FC1 -> GELU -> FC2: R1 = 3072, K1 = 768),
    calibrated statically from input statistics (no pass over outputs).

    FC1 as quant_layer; its dequantising scale is the real one,
    s_deq1[r] = f32(s_w1[r] s_x), so FC1's real output p has per-row standard
    deviation sigma_p[r] = s_deq1[r] sqrt((N/M) sum_k q_w1^2 mean(q_x^2)).
    The hidden activation is quantised per tensor with s_h = 4 max_r sigma_p / 127
    (os1 = 1 / s_h).  FC2: W2 [K1][R1] ~ N(0, w_sigma^2) quantised per row;
    bias2 in the units s_w2 s_h; its requantising scale takes E[h^2] ~
    mean_r sigma_p^2 / (2 s_h^2) (GELU passes about the positive half) in
    quant_layer's formula."""
    fc1 = quant_layer(R1, K1, T, N, M, seed, *names, "fc1", w_sigma=w_sigma, x_sigma=x_sigma,
                      b_sigma=b_sigma)
    s_deq1 = (fc1.s_w * fc1.s_x).astype(np.float32)
    ex2 = float(np.mean(fc1.X.astype(np.float64) ** 2))
    sig_p = s_deq1.astype(np.float64) * np.sqrt((N / M) * (fc1.W.astype(np.float64) ** 2).sum(axis=1) * ex2)
    s_h = 4.0 * float(sig_p.max()) / 127.0
    w2 = rng(seed, *names, "fc2", "W").standard_normal((K1, R1)) * w_sigma
    bf2 = rng(seed, *names, "fc2", "bias").standard_normal(K1) * b_sigma
    s_w2 = np.abs(w2).max(axis=1) / 127.0
    s_w2[s_w2 == 0] = 1.0
    qw2 = np.clip(np.rint(w2 / s_w2[:, None]), -127, 127).astype(np.int8)
    b2 = np.rint(bf2 / (s_w2 * s_h)).astype(np.int32)
    eh2 = float(np.mean(sig_p ** 2)) / (2.0 * s_h * s_h)
    row = (N / M) * (qw2.astype(np.float64) ** 2).sum(axis=1) * eh2
    scale2 = (127.0 / (4.0 * np.sqrt(row) + 1.0)).astype(np.float32)
    return MlpChain(W1=fc1.W, X=fc1.X, b1=fc1.bias, s_deq1=s_deq1, os1=1.0 / s_h, W2=qw2, b2=b2,
                    scale2=scale2)


# ------------------------------------------------------------------ workloads
@dataclass(frozen=True)
class Layer:
    name: str
    R: int
    K: int
    T: int
    N: int
    M: int
    dt: str       # input dtype: 'i8' | 'f16' | 'bf16'
    out: str      # output dtype: 'i32' | 'i8' | 'f16' | 'bf16' | 'f32'


VIT_B_TOKENS = 64 * 197          # batch 64 of 197 tokens
VIT_B_LAYERS = {"qkv": (2304, 768), "proj": (768, 768), "fc1": (3072, 768), "fc2": (768, 3072)}


def config1():
    """Single int8 2:4 layer, W 192x192 (ViT-Tiny qkv slice), X 192x197, int32 out."""
    return [Layer("c1_vit_tiny_qkv_slice", 192, 192, 197, 2, 4, "i8", "i32")]


def config2():
    """ViT-B/16 linear layers, int8, batch 64, fused bias + requant to int8."""
    out = []
    for nm in ((1, 4), (2, 4), (2, 8), (4, 8)):
        for lname, (R, K) in VIT_B_LAYERS.items():
            out.append(Layer(f"c2_vitb_{lname}_{nm[0]}of{nm[1]}", R, K, VIT_B_TOKENS, nm[0], nm[1],
                             "i8", "i8"))
    return out


def headline():
    """ViT-B FC1, int8 2:4, batch 64: R=3072, K=768, T=12608, bias + requant to int8."""
    return Layer("vitb_fc1_2of4_i8", 3072, 768, VIT_B_TOKENS, 2, 4, "i8", "i8")


def config3():
    """Swin-T-style MLP shapes, fp16, batch 32, 2:4 and 1:4, fp16 out."""
    out = []
    for C, tok in ((96, 3136), (192, 784), (384, 196), (768, 49)):
        T = 32 * tok
        for nm in ((2, 4), (1, 4)):
            out.append(Layer(f"c3_swin_C{C}_fc1_{nm[0]}of{nm[1]}", 4 * C, C, T, nm[0], nm[1],
                             "f16", "f16"))
            out.append(Layer(f"c3_swin_C{C}_fc2_{nm[0]}of{nm[1]}", C, 4 * C, T, nm[0], nm[1],
                             "f16", "f16"))
    return out


def stack_nm(seed: int = 0):
    """Per-layer N:M of the 48-layer mixed ViT-B stack (block-major: qkv, proj, fc1, fc2)."""
    choices = [(1, 4), (2, 4), (4, 8), (8, 8)]
    draw = np.random.default_rng(seed).integers(0, 4, size=48)
    return [choices[int(i)] for i in draw]


def config4(seed: int = 0):
    """12 ViT-B blocks x {qkv, proj, fc1, fc2}, each with its own N:M, int8, batch 64."""
    nms = stack_nm(seed)
    out = []
    for i, (N, M) in enumerate(nms):
        blk, lname = divmod(i, 4)
        lname = list(VIT_B_LAYERS)[lname]
        R, K = VIT_B_LAYERS[lname]
        out.append(Layer(f"c4_b{blk}_{lname}_{N}of{M}", R, K, VIT_B_TOKENS, N, M, "i8", "i8"))
    return out


def config5():
    """LLaMA-7B projections, fp16 and bf16, 2:4 and 4:8, decode T=16 and prefill T=2048."""
    out = []
    for dt in ("f16", "bf16"):
        for (R, K), pname in (((4096, 4096), "qkvo"), ((11008, 4096), "up"), ((4096, 11008), "down")):
            for nm in ((2, 4), (4, 8)):
                for T in (16, 2048):
                    out.append(Layer(f"c5_llama_{pname}_{nm[0]}of{nm[1]}_T{T}_{dt}", R, K, T,
                                     nm[0], nm[1], dt, dt))
    return out


def all_configs():
    return {"1": config1(), "2": config2(), "3": config3(), "4": config4(), "5": config5()}


def make_inputs(layer: Layer, seed: int = 0):
    """Host operands for a layer: dict(W, X, bias, scale) (bias/scale may be None)."""
    L = layer
    if L.dt == "i8" and L.out == "i32":
        W = uniform_int8((L.R, L.K), seed, L.name, "W")
        X = uniform_int8((L.K, L.T), seed, L.name, "X")
        return dict(W=W, X=X, bias=None, scale=None)
    if L.dt == "i8":
        q = quant_layer(L.R, L.K, L.T, L.N, L.M, seed, L.name)
        return dict(W=q.W, X=q.X, bias=q.bias, scale=q.scale)
    W = normal((L.R, L.K), 0.02, L.dt, seed, L.name, "W")
    X = normal((L.K, L.T), 1.0, L.dt, seed, L.name, "X")
    return dict(W=W, X=X, bias=None, scale=None)


def ops_and_bytes(L: Layer):
    """(algorithmic ops, algorithmic bytes, dense-equivalent ops) of one product.

    ops = 2 R K T N/M; bytes = kept values + log2(M)-bit indices (none when
    N == M) + X + Y (+ bias and scale rows when an int8 epilogue runs)."""
    b = {"i8": 1, "f16": 2, "bf16": 2}[L.dt]
    by = {"i32": 4, "i8": 1, "f16": 2, "bf16": 2, "f32": 4}[L.out]
    kept = L.R * L.K * L.N // L.M
    w = {4: 2, 8: 3}[L.M]
    meta = 0 if L.N == L.M else kept * w / 8
    epi = L.R * 8 if L.out == "i8" else 0
    nbytes = kept * b + meta + L.K * L.T * b + L.R * L.T * by + epi
    return 2 * L.R * L.K * L.T * L.N / L.M, nbytes, 2 * L.R * L.K * L.T


def unstructured(R: int, K: int, density: float, dt: str, seed: int, *names) -> np.ndarray:
    """N(0, 0.02^2) weights pruned without structure to `density`: in every
    row the round(density K) entries of largest |w| stay (equal |w|: the lower
    column), the rest become +0 -- the moderately unstructured weights
    (about 50% kept) of LLM pruning by magnitude per output row.  Raw bits for
    bf16, as normal() returns them."""
    W = normal((R, K), 0.02, dt, seed, *names)
    mag = (W.view(np.uint16) & 0x7FFF) if dt in ("f16", "bf16") else np.abs(W)
    keep = int(round(density * K))
    order = np.argsort(-mag.astype(np.int64), axis=1, kind="stable")
    mask = np.zeros((R, K), bool)
    np.put_along_axis(mask, order[:, :keep], True, axis=1)
    out = W.copy()
    out[~mask] = 0
    return out


@dataclass
class HybridLayer:
    """A layer of the three-layer format product: weight pattern 'u50'
    (unstructured, 50% kept per row) or '4of8' (4:8), dtype, output dtype."""
    name: str
    R: int
    K: int
    T: int
    pattern: str
    dt: str
    out: str


def hybrid_workloads():
    """Layers of the three-layer format product: LLaMA-7B projections at 50%
    unstructured sparsity in decode (16 tokens), fp16 and bf16, and the
    ViT-B FC1 layer with 4:8 weights (a pattern the format holds in its first
    two layers) at 16 and 197 tokens (one image)."""
    out = []
    for dt in ("f16", "bf16"):
        for (R, K), pname in (((4096, 4096), "qkvo"), ((11008, 4096), "up"), ((4096, 11008), "down")):
            out.append(HybridLayer(f"hy_llama_{pname}_u50_T16_{dt}", R, K, 16, "u50", dt, dt))
    out.append(HybridLayer("hy_vitb_fc1_4of8_T16_f16", 3072, 768, 16, "4of8", "f16", "f16"))
    out.append(HybridLayer("hy_vitb_fc1_4of8_T197_f16", 3072, 768, 197, "4of8", "f16", "f16"))
    return out


def structured(R: int, K: int, n: int, m: int, dt: str, seed: int, *names) -> np.ndarray:
    """N(0, 0.02^2) weights with exactly n nonzeros in every group of m
    consecutive columns, at positions drawn uniformly (an n:m pattern as a
    pruned layer would carry it).  Raw bits for bf16."""
    W = normal((R, K), 0.02, dt, seed, *names)
    keys = rng(seed, *names, "mask").random((R, K // m, m))
    order = np.argsort(keys, axis=2, kind="stable")
    mask = np.zeros((R, K // m, m), bool)
    np.put_along_axis(mask, order[:, :, :n], True, axis=2)
    out = W.copy()
    out[~mask.reshape(R, K)] = 0
    return out


def hybrid_inputs(L: HybridLayer, seed: int = 0):
    """Host operands of a three-layer format layer: dict(W, X)."""
    if L.pattern == "u50":
        W = unstructured(L.R, L.K, 0.5, L.dt, seed, L.name, "W")
    elif L.pattern == "4of8":
        W = structured(L.R, L.K, 4, 8, L.dt, seed, L.name, "W")
    else:
        raise ValueError(L.pattern)
    X = normal((L.K, L.T), 1.0, L.dt, seed, L.name, "X")
    return dict(W=W, X=X)
