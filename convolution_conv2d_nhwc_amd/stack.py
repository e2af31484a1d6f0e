"""Stack executor: a chained workload as one sequence of launches on one
stream, each layer writing straight into the next layer's preallocated NHWC
input buffer, captured once into a HIP graph and replayed.

This is the host-side runtime of the layer stacks (the 640x640 YOLO stack
with its mosaic, the keyword-spotting and visual-wake-words stacks). It
follows the pages' runtime lessons: record the model work once and replay
it, and remove copies and moves between operations (zerolat.eu YOLOv4
report, section 10 "Runtime and I/O changes on the card", and its note on
why reducing the operation count matters); per-call host cost removed by
graph replay (nanoinfer README, GPU section: back-to-back launches against a
replayed graph). Every launch is a library call through the C ABI; the
executor only owns buffers and the order of the calls.
"""
from __future__ import annotations

from typing import Callable, List, Optional

import torch

from . import _lib
from .data import Workload, layer_params, network_input


class Stack:
    """Plans, resident weights and buffers of a workload on the current
    device. ``step()`` enqueues one pass on the current stream;
    ``capture()`` records one pass into a graph that ``replay()`` runs.

    With ``fuse``, a layer followed by a 1x1 layer that the library can run
    in the same launch (``conv_run_fused``: the first layer's output tile
    goes through the 1x1 layer before anything is stored) is launched as one
    node; the first layer's output buffer is then never written.

    With ``pad_canvas`` (a stack with a mosaic), the canvas carries 8 channel
    slots per pixel and the first layer reads it through the window stem
    kernel when the library accepts that layer with an 8-element pixel
    stride; otherwise the canvas is dense. With ``fuse`` as well, the mosaic
    is folded into that layer's input gather (``conv_run_mosaic``): one
    launch reads the tiles and the canvas is never written."""

    def __init__(self, wl: Workload, seed: int = 0, device: str = "cuda", fuse: bool = False,
                 pad_canvas: bool = True):
        if not wl.chained and len(wl.layers) != 1:
            raise ValueError("%s is neither a chained stack nor a single layer" % wl.name)
        self.wl = wl
        self.convs: List[_lib.Conv2d] = []
        self.params = []
        self.bufs: List[torch.Tensor] = []
        # with a mosaic, the canvas carries 8 channel slots per pixel when the
        # first layer can read them (the window stem kernel), else c_in
        self.canvas_c = wl.mosaic[3] if wl.mosaic is not None else 0
        for i, layer in enumerate(wl.layers):
            p = layer_params(wl, i, seed)
            conv = None
            if i == 0 and wl.mosaic is not None and pad_canvas and layer.cin <= 8:
                try:
                    conv = _lib.Conv2d.from_layer(layer, x_stride=8)
                    self.canvas_c = 8
                except _lib.ConvError:
                    conv = None
            if conv is None:
                conv = _lib.Conv2d.from_layer(layer)
            dev = {"w": p["w"].to(device)}
            if layer.dtype == "i8":
                dev["b"] = _lib.pack_bias_scale(p["b"], p.get("s") if layer.out == "i8" else None).to(device)
            else:
                dev["b"] = p["b"].to(device)
            self.convs.append(conv)
            self.params.append(dev)
            self.bufs.append(conv.empty_output(device))
        self.x0 = (network_input(wl, seed) if wl.chained else layer_params(wl, 0, seed)["x"]).to(device)
        self.canvas: Optional[torch.Tensor] = None
        if wl.mosaic is not None:
            m, th, tw, c = wl.mosaic
            self.canvas = torch.empty((m, 2 * th, 2 * tw, self.canvas_c), dtype=torch.bfloat16, device=device)
        self.graph: Optional[torch.cuda.CUDAGraph] = None
        self.mosaic_fused = bool(fuse and self.canvas is not None and self.canvas_c == 8)
        if self.mosaic_fused:
            self.canvas = None
        # fused[i]: layer i is launched together with layer i + 1
        self.fused = [False] * len(self.convs)
        if fuse:
            i = 0
            while i + 1 < len(self.convs):
                if _lib.fusable(self.convs[i], self.convs[i + 1]):
                    self.fused[i] = True
                    i += 2
                else:
                    i += 1

    # each layer's input: the canvas (or the network input), then the
    # previous layer's output buffer
    def layer_input(self, i: int) -> torch.Tensor:
        if i > 0:
            return self.bufs[i - 1]
        return self.canvas if self.canvas is not None else self.x0  # (the tiles when the mosaic is folded in)

    def nodes(self) -> List[tuple]:
        """The layers of each launch: (i,) or (i, i + 1) for a fused pair."""
        out, i = [], 0
        while i < len(self.convs):
            if self.fused[i]:
                out.append((i, i + 1))
                i += 2
            else:
                out.append((i,))
                i += 1
        return out

    def launches(self) -> List[Callable[[], None]]:
        """The pass as a list of library-call closures, in order (the mosaic,
        then one per node of ``nodes()``)."""
        seq: List[Callable[[], None]] = []
        if self.canvas is not None:
            seq.append(lambda: _lib.mosaic_pack(self.x0, self.canvas, c_pad=self.canvas_c, out_dtype=torch.bfloat16))
        for node in self.nodes():
            i = node[0]
            if len(node) == 2:
                seq.append(lambda i=i: _lib.run_fused(self.convs[i], self.convs[i + 1], self.layer_input(i),
                                                      self.params[i]["w"], self.params[i]["b"],
                                                      self.params[i + 1]["w"], self.params[i + 1]["b"],
                                                      self.bufs[i + 1]))
            elif i == 0 and self.mosaic_fused:
                seq.append(lambda: _lib.run_mosaic(self.convs[0], self.x0, self.params[0]["w"], self.params[0]["b"],
                                                   self.bufs[0]))
            else:
                seq.append(lambda i=i: self.convs[i].run(self.layer_input(i), self.params[i]["w"],
                                                         self.params[i]["b"], self.bufs[i]))
        return seq

    def mosaic_kernel(self) -> str:
        """The kernel symbol of the mosaic launch (see csrc/mosaic.hip)."""
        m, th, tw, c = self.wl.mosaic
        if self.canvas_c == 8:
            return "mosaic_px16_kernel"
        return "mosaic_vec8_kernel" if self.canvas_c == c and (tw * c) % 8 == 0 else "mosaic_pixel_kernel"

    def node_kernel(self, node) -> str:
        """The kernel symbol a node launches."""
        if node == (0,) and self.mosaic_fused:
            return "stem_window_kernel<1>"
        if len(node) == 2:
            d = _lib.describe_fused(self.convs[node[0]], self.convs[node[1]])
        else:
            d = self.convs[node[0]].describe()
        return d.split("kernel=")[-1]

    def step(self) -> torch.Tensor:
        for f in self.launches():
            f()
        return self.bufs[-1]

    def capture(self, warmup: int = 3) -> torch.cuda.CUDAGraph:
        """Run `warmup` eager passes on a side stream, then record one pass."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(warmup):
                self.step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def replay(self) -> torch.Tensor:
        if self.graph is None:
            raise RuntimeError("capture() first")
        self.graph.replay()
        return self.bufs[-1]

    @property
    def output(self) -> torch.Tensor:
        return self.bufs[-1]

    def close(self):
        self.graph = None
        for c in self.convs:
            c.close()
        self.convs = []
