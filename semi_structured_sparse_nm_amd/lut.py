"""Profiling-based latency look-up table for nm_spmm.

The configuration side of "Realizable N:M Sparse Transformer Inference via
Search-Kernel Co-Design" (Sec. 3) predicts the latency of a layer-wise N:M
assignment with a calibrated look-up table (LUT) of measured kernel
latencies, so that a search can reject assignments that miss a latency
budget without running them.  This module is that predictor for this
library:

- an entry is the measured latency of one nm_spmm launch for one layer shape
  (R, K, N, M, input dtype, output dtype) at one token count T; between
  measured token counts the latency is interpolated linearly in T (and
  extrapolated from the two nearest entries outside them);
- a stack of layers run back to back is predicted as the sum of its layers'
  entries plus one calibrated gap per launch (what the back-to-back run
  costs beyond the isolated launches: launch spacing, cache state);
- ``calibrate`` fits that gap from one measured stack.

The table itself is plain data (JSON round trip); ``measure_layers`` and
``time_stack`` fill it and check it on the GPU through the library (HIP
graph replays on the current stream).
"""
from __future__ import annotations

import json
import math
from dataclasses import dataclass
from typing import Dict, Iterable, List, Sequence, Tuple

Key = Tuple[int, int, int, int, str, str]


@dataclass(frozen=True)
class LayerShape:
    """One linear layer as nm_spmm sees it."""
    R: int
    K: int
    T: int
    N: int
    M: int
    dt: str = "i8"      # weight / activation dtype: i8 | f16 | bf16
    out: str = "i8"     # output dtype: i8 | i32 | f16 | bf16 | f32

    @property
    def key(self) -> Key:
        return (self.R, self.K, self.N, self.M, self.dt, self.out)


class LatencyLUT:
    """Measured nm_spmm latencies (microseconds) per layer shape and T."""

    def __init__(self, gap_us: float = 0.0, device: str = ""):
        self._t: Dict[Key, List[Tuple[int, float]]] = {}
        self.gap_us = float(gap_us)
        self.device = device

    # ------------------------------------------------------------ entries
    def add(self, layer: LayerShape, us: float) -> None:
        if not (us > 0 and math.isfinite(us)):
            raise ValueError(f"latency must be positive and finite, got {us}")
        pts = [p for p in self._t.get(layer.key, []) if p[0] != layer.T]
        pts.append((int(layer.T), float(us)))
        pts.sort()
        self._t[layer.key] = pts

    def keys(self) -> List[Key]:
        return sorted(self._t)

    def __len__(self) -> int:
        return sum(len(v) for v in self._t.values())

    def __contains__(self, layer: LayerShape) -> bool:
        return layer.key in self._t

    def lookup(self, layer: LayerShape) -> float:
        """Latency of one launch of ``layer``: the entry at its T, else linear
        interpolation in T between the nearest entries (extrapolation from the
        two nearest outside them; a single entry scales in proportion to T).
        KeyError when the shape was never measured."""
        pts = self._t.get(layer.key)
        if not pts:
            raise KeyError(f"no latency measured for {layer.key}")
        T = layer.T
        for t, us in pts:
            if t == T:
                return us
        if len(pts) == 1:
            t, us = pts[0]
            return us * T / t
        if T < pts[0][0]:
            (t0, u0), (t1, u1) = pts[0], pts[1]
        elif T > pts[-1][0]:
            (t0, u0), (t1, u1) = pts[-2], pts[-1]
        else:
            i = next(i for i in range(1, len(pts)) if pts[i][0] > T)
            (t0, u0), (t1, u1) = pts[i - 1], pts[i]
        y = u0 + (u1 - u0) * (T - t0) / (t1 - t0)
        return max(y, 1e-3)

    # ------------------------------------------------------------ stacks
    def predict(self, layers: Sequence[LayerShape]) -> float:
        """Predicted latency of ``layers`` run back to back on one stream."""
        return sum(self.lookup(L) for L in layers) + len(layers) * self.gap_us

    def calibrate(self, layers: Sequence[LayerShape], measured_us: float) -> float:
        """Fit the per-launch gap so that ``predict(layers)`` equals the
        measured latency of that stack; returns the gap."""
        if not layers:
            raise ValueError("calibration needs at least one layer")
        self.gap_us = (float(measured_us) - sum(self.lookup(L) for L in layers)) / len(layers)
        return self.gap_us

    # ------------------------------------------------------------ persistence
    def to_json(self) -> str:
        return json.dumps({
            "device": self.device, "gap_us": self.gap_us,
            "entries": [{"R": k[0], "K": k[1], "N": k[2], "M": k[3], "dt": k[4], "out": k[5],
                         "points": [[t, us] for t, us in v]} for k, v in sorted(self._t.items())],
        }, indent=1)

    @classmethod
    def from_json(cls, text: str) -> "LatencyLUT":
        d = json.loads(text)
        lut = cls(gap_us=d.get("gap_us", 0.0), device=d.get("device", ""))
        for e in d["entries"]:
            for t, us in e["points"]:
                lut.add(LayerShape(e["R"], e["K"], int(t), e["N"], e["M"], e["dt"], e["out"]), us)
        return lut


# ---------------------------------------------------------------- GPU side
def _build(layer: LayerShape, seed: int, device):
    """Device operands of one layer (seeded; timing only)."""
    import torch

    from . import pack

    tdt = {"i8": torch.int8, "f16": torch.float16, "bf16": torch.bfloat16, "i32": torch.int32,
           "f32": torch.float32}
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    if layer.dt == "i8":
        W = torch.randint(-127, 128, (layer.R, layer.K), dtype=torch.int8, device=device, generator=gen)
        X = torch.randint(-127, 128, (layer.K, layer.T), dtype=torch.int8, device=device, generator=gen)
    else:
        W = (torch.randn((layer.R, layer.K), device=device, generator=gen) * 0.02).to(tdt[layer.dt])
        X = torch.randn((layer.K, layer.T), device=device, generator=gen).to(tdt[layer.dt])
    p = pack(W, layer.N, layer.M)
    bias = scale = None
    if layer.out == "i8":
        bias = torch.randint(-2000, 2000, (layer.R,), dtype=torch.int32, device=device, generator=gen)
        scale = torch.full((layer.R,), 1.0 / 4096, dtype=torch.float32, device=device)
    Y = torch.empty((layer.R, layer.T), dtype=tdt[layer.out], device=device)
    return (layer, p, X, bias, scale, Y, tdt[layer.out])


def _launch(item) -> None:
    from . import spmm
    layer, p, X, bias, scale, Y, odt = item
    spmm(p, X, bias=bias, scale=scale, out_dtype=odt, out=Y)


def _graph_time(items, reps: int) -> float:
    """Microseconds per pass of ``items`` launched in order, from a HIP graph
    of ``reps`` passes replayed once (after one warm replay)."""
    import torch

    for it in items:
        _launch(it)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for _ in range(reps):
                for it in items:
                    _launch(it)
    torch.cuda.current_stream().wait_stream(st)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def _footprint(layer: LayerShape) -> int:
    eb = {"i8": 1, "f16": 2, "bf16": 2}[layer.dt]
    ob = {"i8": 1, "i32": 4, "f16": 2, "bf16": 2, "f32": 4}[layer.out]
    return layer.R * layer.K * eb * layer.N // layer.M + layer.K * layer.T * eb + layer.R * layer.T * ob


def measure_layers(layers: Iterable[LayerShape], lut: LatencyLUT | None = None, reps: int = 20,
                   rotate_bytes: int = 1 << 30, max_copies: int = 32, seed: int = 0) -> LatencyLUT:
    """Measure every distinct layer shape of ``layers`` into ``lut`` (a new
    one by default).  Independent operand sets totalling at least
    ``rotate_bytes`` (more than the 256 MB Infinity Cache) are launched in
    turn, so no launch finds its inputs in the caches -- the state a layer
    meets in a stack of distinct layers."""
    import torch

    device = torch.device("cuda", torch.cuda.current_device())
    lut = lut or LatencyLUT(device=torch.cuda.get_device_name(device))
    seen = set()
    for L in layers:
        if (L.key, L.T) in seen:
            continue
        seen.add((L.key, L.T))
        copies = max(2, min(max_copies, -(-rotate_bytes // _footprint(L))))
        items = [_build(L, seed + 101 * c, device) for c in range(copies)]
        lut.add(L, _graph_time(items, max(reps, copies)) / copies)
        del items
        torch.cuda.empty_cache()
    return lut


def time_stack(layers: Sequence[LayerShape], reps: int = 3, seed: int = 0) -> float:
    """Measured microseconds of one back-to-back pass over ``layers`` (each
    with its own operands)."""
    import torch

    device = torch.device("cuda", torch.cuda.current_device())
    items = [_build(L, seed + 7 * i, device) for i, L in enumerate(layers)]
    us = _graph_time(items, reps)
    del items
    torch.cuda.empty_cache()
    return us
