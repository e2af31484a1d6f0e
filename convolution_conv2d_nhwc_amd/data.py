"""Seeded synthetic workloads: layer shapes and input tensors.

This module holds no convolution arithmetic. It lists the layer shapes of
the workloads the pages describe (written out by hand, including every
layer's input size) and draws their tensors from numpy's PCG64 generator.
It is the only code that both the HIP path's tests and the CPU oracle's
tests share.

Draw recipe (every workload, seed 0 unless a caller asks for another):
  * stream i of a workload is ``default_rng(SeedSequence([seed, i]))``;
    stream 0 draws the network input, stream i >= 1 draws layer i;
  * stream 1000 + i draws a fresh input for layer i when one layer of a
    chained workload is tested on its own;
  * a layer stream draws, in order: (its own input ``x`` when the workload
    gives each layer a fresh input), ``w``, ``b``, then ``s`` for int8;
  * float laws are drawn in float64 and cast to float32; bf16 tensors are
    float32 values rounded once to bf16 (round-to-nearest-even, by torch);
  * int8 laws are the discrete uniform on [-127, 127] inclusive; int8 bias
    is the discrete uniform on [-16129, 16129] (= +-127^2); requant scales
    are uniform on [0.001, 0.01].

Value laws per workload:
  mnist_f32      x, w ~ U[-1, 1], b ~ U[-0.1, 0.1]       (fp32)
  kws_int8       x, w int8 law, b int32 law, s scale law  (int8, chained)
  vww_bf16       x ~ N(0, 0.5), w ~ Kaiming normal, b ~ U[-0.1, 0.1]
  yolo640_bf16   four 320x320x3 tiles ~ U[0, 1) (fp32), then Kaiming w,
                 b ~ U[-0.1, 0.1]
  yolo_sweep_*   per-layer fresh x at the listed shape; int8 or bf16 laws
  dw_probe_*     per-layer fresh x; int8 or bf16 laws
Kaiming normal: sigma = sqrt(2 / fan_in), fan_in = (Cin/groups)*KH*KW.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, List, Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Layer:
    name: str
    n: int
    h: int
    w: int
    cin: int
    cout: int
    kh: int
    kw: int
    sh: int = 1
    sw: int = 1
    ph: int = 0
    pw: int = 0
    groups: int = 1
    dtype: str = "bf16"   # "f32" | "bf16" | "i8"
    out: str = "bf16"     # "f32" | "bf16" | "i8" | "i32"
    act: str = "none"     # "none" | "relu" | "relu6" | "mish"
    ho: int = 0           # expected output size, written out by hand
    wo: int = 0

    @property
    def depthwise(self) -> bool:
        return self.groups > 1 and self.groups == self.cin == self.cout

    def flops(self) -> int:
        """2 * N*Ho*Wo*Cout * KH*KW*(Cin/groups): every tap counted,
        padded ones included (the nanoinfer GPU section counts a 3x3
        depthwise layer at 128 channels, 28x28, as 1.8 MFLOP this way)."""
        return 2 * self.n * self.ho * self.wo * self.cout * self.kh * self.kw * (self.cin // self.groups)

    def bytes(self) -> int:
        """Algorithmic bytes: x read once, w once, y written once, bias (and
        scale) once."""
        esz = {"f32": 4, "bf16": 2, "i8": 1, "i32": 4}
        xb = self.n * self.h * self.w * self.cin * esz[self.dtype]
        wb = self.cout * self.kh * self.kw * (self.cin // self.groups) * esz[self.dtype]
        yb = self.n * self.ho * self.wo * self.cout * esz[self.out]
        bb = self.cout * 4 * (2 if (self.dtype == "i8" and self.out == "i8") else 1)
        return xb + wb + yb + bb


@dataclass(frozen=True)
class Workload:
    name: str
    law: str                 # "mnist" | "int8" | "bf16"
    layers: tuple
    chained: bool            # layer i+1 consumes layer i's output
    mosaic: Optional[tuple] = None   # (m, th, tw, c) tiles packed into layer 1's input
    description: str = ""

    def flops(self) -> int:
        return sum(l.flops() for l in self.layers)


def _dense(name, n, h, w, cin, cout, k, s, p, dtype, out, act, ho, wo):
    return Layer(name, n, h, w, cin, cout, k, k, s, s, p, p, 1, dtype, out, act, ho, wo)


def _dw(name, n, h, w, c, s, dtype, out, act, ho, wo):
    return Layer(name, n, h, w, c, c, 3, 3, s, s, 1, 1, c, dtype, out, act, ho, wo)


def _mnist() -> Workload:
    return Workload("mnist_f32", "mnist",
                    (_dense("conv3x3", 1, 28, 28, 1, 8, 3, 1, 1, "f32", "f32", "relu", 28, 28),),
                    chained=False,
                    description="fp32 NHWC 28x28x1 -> 8, 3x3 s1 p1, bias+ReLU, N=1")


def _kws() -> Workload:
    L = [Layer("stem10x4", 1, 49, 10, 1, 64, 10, 4, 2, 2, 5, 1, 1, "i8", "i8", "relu", 25, 5)]
    for i in range(4):
        L.append(_dw("dw%d" % (i + 1), 1, 25, 5, 64, 1, "i8", "i8", "relu", 25, 5))
        L.append(_dense("pw%d" % (i + 1), 1, 25, 5, 64, 64, 1, 1, 0, "i8", "i8", "relu", 25, 5))
    return Workload("kws_int8", "int8", tuple(L), chained=True,
                    description="KWS DS-CNN, int8, 49x10x1, stem 10x4 s2 pad(5,1) + 4x(dw3x3+pw1x1), ReLU")


def _vww() -> Workload:
    L = [_dense("stem", 1, 96, 96, 3, 8, 3, 2, 1, "bf16", "bf16", "relu6", 48, 48)]
    couts = [16, 32, 32, 64, 64, 128, 128, 128, 128, 128, 128, 256, 256]
    strides = [1, 2, 1, 2, 1, 2, 1, 1, 1, 1, 1, 2, 1]
    c, hw = 8, 48
    for i, (co, s) in enumerate(zip(couts, strides)):
        ohw = hw if s == 1 else {48: 24, 24: 12, 12: 6, 6: 3}[hw]
        L.append(_dw("dw%d" % (i + 1), 1, hw, hw, c, s, "bf16", "bf16", "relu6", ohw, ohw))
        L.append(_dense("pw%d" % (i + 1), 1, ohw, ohw, c, co, 1, 1, 0, "bf16", "bf16", "relu6", ohw, ohw))
        c, hw = co, ohw
    return Workload("vww_bf16", "bf16", tuple(L), chained=True,
                    description="VWW MobileNet-v1 0.25, bf16, 96x96x3, stem + 13 dw/pw blocks, ReLU6")


def _yolo640() -> Workload:
    b, m = "bf16", "mish"
    L = (
        _dense("L1_3x3_3to32", 1, 640, 640, 3, 32, 3, 1, 1, b, b, m, 640, 640),
        _dense("L2_3x3s2_32to64", 1, 640, 640, 32, 64, 3, 2, 1, b, b, m, 320, 320),
        _dense("L3_1x1_64to64", 1, 320, 320, 64, 64, 1, 1, 0, b, b, m, 320, 320),
        _dense("L4_3x3_64to64", 1, 320, 320, 64, 64, 3, 1, 1, b, b, m, 320, 320),
        _dense("L5_3x3s2_64to128", 1, 320, 320, 64, 128, 3, 2, 1, b, b, m, 160, 160),
        _dense("L6_1x1_128to64", 1, 160, 160, 128, 64, 1, 1, 0, b, b, m, 160, 160),
        _dense("L7_3x3s2_64to256", 1, 160, 160, 64, 256, 3, 2, 1, b, b, m, 80, 80),
        _dense("L8_3x3s2_256to512", 1, 80, 80, 256, 512, 3, 2, 1, b, b, m, 40, 40),
        _dense("L9_3x3s2_512to1024", 1, 40, 40, 512, 1024, 3, 2, 1, b, b, m, 20, 20),
    )
    return Workload("yolo640_bf16", "bf16", L, chained=True, mosaic=(1, 320, 320, 3),
                    description="YOLO 640x640 stack: 4x320 mosaic + 9 convs, bf16, Mish, N=1")


def _sweep(dtype: str) -> Workload:
    out = "i8" if dtype == "i8" else "bf16"
    d, m = dtype, "mish"
    L = (
        _dense("160sq_3x3_128to128", 16, 160, 160, 128, 128, 3, 1, 1, d, out, m, 160, 160),
        _dense("80sq_1x1_256to512", 16, 80, 80, 256, 512, 1, 1, 0, d, out, m, 80, 80),
        _dense("80sq_3x3_256to256", 16, 80, 80, 256, 256, 3, 1, 1, d, out, m, 80, 80),
        _dense("40sq_3x3_512to512", 16, 40, 40, 512, 512, 3, 1, 1, d, out, m, 40, 40),
        _dense("20sq_1x1_1024to512", 16, 20, 20, 1024, 512, 1, 1, 0, d, out, m, 20, 20),
        _dense("20sq_3x3_512to1024", 16, 20, 20, 512, 1024, 3, 1, 1, d, out, m, 20, 20),
    )
    law = "int8" if dtype == "i8" else "bf16"
    return Workload("yolo_sweep_%s" % ("int8" if dtype == "i8" else "bf16"), law, L, chained=False,
                    description="YOLO neck/backbone sweep, N=16, fused bias+Mish")


def _dw_probe(dtype: str) -> Workload:
    out = "i8" if dtype == "i8" else "bf16"
    L = tuple(_dw("dw_%dsq_%d" % (hw, c), 16, hw, hw, c, 1, dtype, out, "relu6", hw, hw)
              for hw, c in ((160, 128), (80, 256), (40, 512), (20, 1024)))
    law = "int8" if dtype == "i8" else "bf16"
    return Workload("dw_probe_%s" % ("int8" if dtype == "i8" else "bf16"), law, L, chained=False,
                    description="depthwise 3x3 s1 p1 probe on the sweep's maps, N=16, ReLU6")


WORKLOADS: Dict[str, Workload] = {w.name: w for w in (
    _mnist(), _kws(), _vww(), _yolo640(), _sweep("i8"), _sweep("bf16"),
    _dw_probe("bf16"), _dw_probe("i8"))}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


# ----------------------------------------------------------------- draws --

def rng_for(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream]))


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """float32 values -> torch.bfloat16 (round to nearest even, once)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _x(layer: Layer, law: str, rng) -> torch.Tensor:
    shape = (layer.n, layer.h, layer.w, layer.cin)
    if law == "mnist":
        return torch.from_numpy(rng.uniform(-1.0, 1.0, shape).astype(np.float32))
    if law == "int8":
        return torch.from_numpy(rng.integers(-127, 128, shape, dtype=np.int64).astype(np.int8))
    return to_bf16(rng.normal(0.0, 0.5, shape))


def _wbs(layer: Layer, law: str, rng) -> dict:
    wshape = (layer.cout, layer.kh, layer.kw, layer.cin // layer.groups)
    if law == "mnist":
        w = torch.from_numpy(rng.uniform(-1.0, 1.0, wshape).astype(np.float32))
        b = torch.from_numpy(rng.uniform(-0.1, 0.1, layer.cout).astype(np.float32))
        return {"w": w, "b": b}
    if law == "int8":
        w = torch.from_numpy(rng.integers(-127, 128, wshape, dtype=np.int64).astype(np.int8))
        b = torch.from_numpy(rng.integers(-16129, 16130, layer.cout, dtype=np.int64).astype(np.int32))
        s = torch.from_numpy(rng.uniform(0.001, 0.01, layer.cout).astype(np.float32))
        return {"w": w, "b": b, "s": s}
    fan_in = (layer.cin // layer.groups) * layer.kh * layer.kw
    w = to_bf16(rng.normal(0.0, np.sqrt(2.0 / fan_in), wshape))
    b = torch.from_numpy(rng.uniform(-0.1, 0.1, layer.cout).astype(np.float32))
    return {"w": w, "b": b}


def layer_params(wl: Workload, i: int, seed: int = 0) -> dict:
    """Tensors of layer i (0-based) of workload wl, on the CPU: keys w, b,
    (s for int8) and x when the workload gives each layer a fresh input."""
    layer = wl.layers[i]
    rng = rng_for(seed, i + 1)
    out = {}
    if not wl.chained:
        out["x"] = _x(layer, wl.law, rng)
    out.update(_wbs(layer, wl.law, rng))
    return out


def network_input(wl: Workload, seed: int = 0) -> torch.Tensor:
    """Input of layer 1 of a chained workload. For a mosaic workload these
    are the fp32 tiles [4m, th, tw, c] (values U[0, 1)), not the canvas."""
    rng = rng_for(seed, 0)
    if wl.mosaic is not None:
        m, th, tw, c = wl.mosaic
        return torch.from_numpy(rng.random((4 * m, th, tw, c)).astype(np.float32))
    return _x(wl.layers[0], wl.law, rng)


def fresh_input(wl: Workload, i: int, seed: int = 0) -> torch.Tensor:
    """A fresh seeded input of layer i's shape under the workload's value law
    (stream 1000 + i), for testing one layer of a chained stack on its own."""
    return _x(wl.layers[i], wl.law, rng_for(seed, 1000 + i))


def random_layer_tensors(layer: Layer, law: str, seed: int, stream: int = 1) -> dict:
    """x, w, b (and s) for an arbitrary layer spec from one stream (used by
    the shape-sweep tests)."""
    rng = rng_for(seed, stream)
    out = {"x": _x(layer, law, rng)}
    out.update(_wbs(layer, law, rng))
    return out


def with_batch(layer: Layer, n: int) -> Layer:
    return replace(layer, n=n)
