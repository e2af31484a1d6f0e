"""ctypes binding of ``libconv_nhwc.so`` (declared in include/conv_nhwc.h).

Argument marshalling only: every step of the computation runs in the HIP
library. torch supplies device memory and the current stream. If the library
has not been built, the first call raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBPATH = os.path.join(_HERE, "libconv_nhwc.so")

DTYPES = {"f32": 0, "bf16": 1, "i8": 2, "i32": 3}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8, "i32": torch.int32}
ACTS = {"none": 0, "relu": 1, "relu6": 2, "mish": 3}
STATUS = {0: "CONV_OK", -1: "CONV_E_NULL", -2: "CONV_E_SHAPE", -3: "CONV_E_UNSUPPORTED",
          -4: "CONV_E_ALIGN", -5: "CONV_E_ALIAS", -6: "CONV_E_NOMEM", -7: "CONV_E_HIP",
          -8: "CONV_E_SCRATCH"}


class ConvError(RuntimeError):
    """A negative conv_status from the library; ``.code`` and ``.name``."""

    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code
        self.name = STATUS.get(code, "unknown")


class _Desc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("h", ctypes.c_int64), ("w", ctypes.c_int64),
                ("c_in", ctypes.c_int64), ("c_out", ctypes.c_int64),
                ("kh", ctypes.c_int32), ("kw", ctypes.c_int32),
                ("stride_h", ctypes.c_int32), ("stride_w", ctypes.c_int32),
                ("pad_h", ctypes.c_int32), ("pad_w", ctypes.c_int32),
                ("groups", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("act", ctypes.c_int32),
                ("algo", ctypes.c_int32), ("w_format", ctypes.c_int32), ("x_pixel_stride", ctypes.c_int32)]


W_FORMATS = {"plain": 0, "bfp8": 1}


_lib = None


def library_path() -> str:
    return _LIBPATH


def lib():
    """Load the HIP library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIBPATH):
        raise RuntimeError("libconv_nhwc.so is not built: run `python -m convolution_conv2d_nhwc_amd.build` "
                           "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(_LIBPATH)
    P = ctypes.c_void_p
    L.conv_prepare.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(P)]
    L.conv_prepare.restype = ctypes.c_int
    L.conv_run.argtypes = [P, P, P, P, P, P]
    L.conv_run.restype = ctypes.c_int
    L.conv_run_residual.argtypes = [P, P, P, P, P, P, P]
    L.conv_run_residual.restype = ctypes.c_int
    L.conv_run_noalloc.argtypes = [ctypes.POINTER(_Desc), P, P, P, P, P, P]
    L.conv_run_noalloc.restype = ctypes.c_int
    L.conv_destroy.argtypes = [P]
    L.conv_destroy.restype = ctypes.c_int
    L.conv_out_shape.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
    L.conv_out_shape.restype = ctypes.c_int
    L.conv_describe.argtypes = [P, ctypes.c_char_p, ctypes.c_int32]
    L.conv_describe.restype = ctypes.c_int
    L.conv_algo_count.argtypes = []
    L.conv_algo_count.restype = ctypes.c_int32
    L.conv_mosaic_pack.argtypes = [P, ctypes.c_int32, P, ctypes.c_int32] + [ctypes.c_int32] * 5 + [P]
    L.conv_mosaic_pack.restype = ctypes.c_int
    L.conv_spp_maxpool.argtypes = [P, ctypes.c_int32, P] + [ctypes.c_int32] * 4 + [P]
    L.conv_spp_maxpool.restype = ctypes.c_int
    I32 = ctypes.c_int32
    L.conv_upsample_concat.argtypes = [P, I32, I32, P, I32, I32, I32, P, I32, I32, I32, P]
    L.conv_upsample_concat.restype = ctypes.c_int
    L.conv_fuse_check.argtypes = [P, P]
    L.conv_fuse_check.restype = ctypes.c_int
    L.conv_describe_fused.argtypes = [P, P, ctypes.c_char_p, ctypes.c_int32]
    L.conv_describe_fused.restype = ctypes.c_int
    L.conv_run_fused.argtypes = [P] * 9
    L.conv_run_fused.restype = ctypes.c_int
    L.conv_run_mosaic.argtypes = [P, P, I32, I32, I32, P, P, P, P]
    L.conv_run_mosaic.restype = ctypes.c_int
    L.conv_run_upcat.argtypes = [P, P, I32, I32, P, I32, P, P, P, P]
    L.conv_run_upcat.restype = ctypes.c_int
    L.conv_bfp8_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64]
    L.conv_bfp8_bytes.restype = ctypes.c_int64
    L.conv_pack_bfp8.argtypes = [P, I32, ctypes.c_int64, ctypes.c_int64, P, P]
    L.conv_pack_bfp8.restype = ctypes.c_int
    L.conv_probe_mfma.argtypes = [I32, I32, P, ctypes.POINTER(ctypes.c_double), P]
    L.conv_probe_mfma.restype = ctypes.c_int
    L.conv_probe_copy.argtypes = [P, P, ctypes.c_int64, P]
    L.conv_probe_copy.restype = ctypes.c_int
    L.conv_status_str.argtypes = [ctypes.c_int32]
    L.conv_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(st: int, what: str):
    if st != 0:
        raise ConvError(st, "%s: %s" % (what, lib().conv_status_str(st).decode()))


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def conv_out_shape(h, w, kh, kw, stride=(1, 1), pad=(0, 0)):
    """Output (ho, wo) of a layer, as the library computes it (prepares a
    throw-away plan)."""
    c = Conv2d(1, h, w, 1, 1, kh, kw, stride, pad, dtype="bf16")
    try:
        return c.out_shape[1], c.out_shape[2]
    finally:
        c.close()


def pack_bias_scale(bias: torch.Tensor, scale: Optional[torch.Tensor]) -> torch.Tensor:
    """One int32 block [bias[c_out], scale bits[c_out]] as the int8 layers
    read it (scale may be None for the int32 checkpoint output)."""
    b = bias.to(torch.int32).contiguous()
    if scale is None:
        return b
    s = scale.to(torch.float32).contiguous().view(torch.int32)
    return torch.cat([b, s.to(b.device)])


class Conv2d:
    """A prepared layer (one conv_plan). ``run`` enqueues it on the current
    torch stream (or ``stream``)."""

    def __init__(self, n: int, h: int, w: int, c_in: int, c_out: int, kh: int, kw: int,
                 stride: Sequence[int] = (1, 1), pad: Sequence[int] = (0, 0), groups: int = 1,
                 dtype: str = "bf16", out_dtype: Optional[str] = None, act: str = "none",
                 algo: int = 0, w_format: str = "plain", x_stride: int = 0):
        out_dtype = out_dtype or dtype
        self.dtype, self.out_dtype, self.act = dtype, out_dtype, act
        self.groups = groups
        self.w_format = w_format
        d = _Desc(n, h, w, c_in, c_out, kh, kw, stride[0], stride[1], pad[0], pad[1], groups,
                  DTYPES[dtype], DTYPES[out_dtype], ACTS[act], algo, W_FORMATS[w_format], x_stride)
        self._desc = d
        self._plan = ctypes.c_void_p()
        _check(lib().conv_prepare(ctypes.byref(d), ctypes.byref(self._plan)), "conv_prepare")
        shp = (ctypes.c_int64 * 4)()
        _check(lib().conv_out_shape(self._plan, shp), "conv_out_shape")
        self.out_shape = tuple(int(v) for v in shp)
        # x_stride: elements per input pixel (channels past c_in ignored)
        self.in_shape = (n, h, w, x_stride or c_in)
        self.w_shape = (c_out, kh, kw, c_in // groups)
        if w_format == "bfp8":
            self.w_shape = (int(lib().conv_bfp8_bytes(c_out, kh * kw * (c_in // groups))),)

    @classmethod
    def from_layer(cls, layer, algo: int = 0, w_format: str = "plain", x_stride: int = 0) -> "Conv2d":
        return cls(layer.n, layer.h, layer.w, layer.cin, layer.cout, layer.kh, layer.kw,
                   (layer.sh, layer.sw), (layer.ph, layer.pw), layer.groups, layer.dtype,
                   layer.out, layer.act, algo, w_format, x_stride)

    def _w_dtype(self):
        return torch.uint8 if self.w_format == "bfp8" else TORCH_DT[self.dtype]

    def describe(self) -> str:
        buf = ctypes.create_string_buffer(256)
        _check(lib().conv_describe(self._plan, buf, 256), "conv_describe")
        return buf.value.decode()

    def empty_output(self, device="cuda") -> torch.Tensor:
        return torch.empty(self.out_shape, dtype=TORCH_DT[self.out_dtype], device=device)

    def _chk(self, t: torch.Tensor, name: str, dt, shape):
        if not t.is_cuda:
            raise ValueError("%s must be a device tensor" % name)
        if t.dtype != dt:
            raise ValueError("%s dtype %s, expected %s" % (name, t.dtype, dt))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError("%s shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))

    def run(self, x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor] = None,
            y: Optional[torch.Tensor] = None, stream=None, residual: Optional[torch.Tensor] = None) -> torch.Tensor:
        """x NHWC, w OHWI, b as the header describes (float32[c_out] or the
        packed int32 block for int8), y NHWC (allocated when None). With
        `residual` (y's dtype and shape; may be y itself) the layer computes
        act(conv + b) + residual through conv_run_residual."""
        self._chk(x, "x", TORCH_DT[self.dtype], self.in_shape)
        self._chk(w, "w", self._w_dtype(), self.w_shape)
        if b is not None:
            want = torch.int32 if self.dtype == "i8" else torch.float32
            self._chk(b, "b", want, None)
        if y is None:
            y = self.empty_output(x.device)
        self._chk(y, "y", TORCH_DT[self.out_dtype], self.out_shape)
        bp = None if b is None else b.data_ptr()
        if residual is None:
            st = lib().conv_run(self._plan, x.data_ptr(), w.data_ptr(), bp, y.data_ptr(), _stream_handle(stream))
            _check(st, "conv_run")
        else:
            self._chk(residual, "residual", TORCH_DT[self.out_dtype], self.out_shape)
            st = lib().conv_run_residual(self._plan, x.data_ptr(), w.data_ptr(), bp, residual.data_ptr(),
                                         y.data_ptr(), _stream_handle(stream))
            _check(st, "conv_run_residual")
        return y

    def run_noalloc(self, x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor], y: torch.Tensor,
                    stream=None, residual: Optional[torch.Tensor] = None) -> torch.Tensor:
        """The same layer through conv_run_noalloc (this object's description,
        not its plan): nothing is allocated, y must be given, and a split
        reduction uses the library's static scratch."""
        self._chk(x, "x", TORCH_DT[self.dtype], self.in_shape)
        self._chk(w, "w", self._w_dtype(), self.w_shape)
        if b is not None:
            self._chk(b, "b", torch.int32 if self.dtype == "i8" else torch.float32, None)
        self._chk(y, "y", TORCH_DT[self.out_dtype], self.out_shape)
        if residual is not None:
            self._chk(residual, "residual", TORCH_DT[self.out_dtype], self.out_shape)
        st = lib().conv_run_noalloc(ctypes.byref(self._desc), x.data_ptr(), w.data_ptr(),
                                    None if b is None else b.data_ptr(),
                                    None if residual is None else residual.data_ptr(), y.data_ptr(),
                                    _stream_handle(stream))
        _check(st, "conv_run_noalloc")
        return y

    def run_ptrs(self, x: int, w: int, b: Optional[int], y: int, stream=None) -> int:
        """Raw call with integer device addresses; returns the conv_status."""
        return lib().conv_run(self._plan, x, w, b, y, _stream_handle(stream) if stream is not False else None)

    def close(self):
        if self._plan is not None and self._plan.value:
            lib().conv_destroy(self._plan)
        self._plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def mosaic_pack(tiles: torch.Tensor, canvas: Optional[torch.Tensor] = None, c_pad: Optional[int] = None,
                out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """Pack tiles [4m, th, tw, c] into canvases [m, 2th, 2tw, c_pad]."""
    if tiles.dim() != 4 or tiles.shape[0] % 4:
        raise ValueError("tiles must be [4m, th, tw, c]")
    q, th, tw, c = tiles.shape
    m = q // 4
    c_pad = c if c_pad is None else c_pad
    rev = {torch.float32: 0, torch.bfloat16: 1}
    if tiles.dtype not in rev or out_dtype not in rev:
        raise ValueError("mosaic supports float32 and bfloat16")
    if not tiles.is_cuda or not tiles.is_contiguous():
        raise ValueError("tiles must be a contiguous device tensor")
    if canvas is None:
        canvas = torch.empty((m, 2 * th, 2 * tw, c_pad), dtype=out_dtype, device=tiles.device)
    if tuple(canvas.shape) != (m, 2 * th, 2 * tw, c_pad) or canvas.dtype != out_dtype or not canvas.is_contiguous():
        raise ValueError("canvas must be a contiguous [m, 2th, 2tw, c_pad] tensor of out_dtype")
    st = lib().conv_mosaic_pack(tiles.data_ptr(), rev[tiles.dtype], canvas.data_ptr(), rev[out_dtype],
                                m, th, tw, c, c_pad, _stream_handle(stream))
    _check(st, "conv_mosaic_pack")
    return canvas


def spp_maxpool(x: torch.Tensor, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """SPP max-pool block of x [n, h, w, c] (float32, bfloat16 or int8):
    y [n, h, w, 4c] = max13 | max9 | max5 | x along channels."""
    codes = {torch.float32: 0, torch.bfloat16: 1, torch.int8: 2}
    if x.dim() != 4 or x.dtype not in codes:
        raise ValueError("x must be a [n, h, w, c] float32, bfloat16 or int8 tensor")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous device tensor")
    n, h, w, c = x.shape
    if y is None:
        y = torch.empty((n, h, w, 4 * c), dtype=x.dtype, device=x.device)
    if tuple(y.shape) != (n, h, w, 4 * c) or y.dtype != x.dtype or not y.is_contiguous():
        raise ValueError("y must be a contiguous [n, h, w, 4c] tensor of x's dtype")
    st = lib().conv_spp_maxpool(x.data_ptr(), codes[x.dtype], y.data_ptr(), n, h, w, c, _stream_handle(stream))
    _check(st, "conv_spp_maxpool")
    return y


def upsample_concat(s0: torch.Tensor, up0: int, s1: torch.Tensor, up1: int, y: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """y [n, ho, wo, c0 + c1] = s0 | s1 along channels, each repeated 2x in
    rows and columns (nearest) where its up flag is 1."""
    codes = {torch.float32: 0, torch.bfloat16: 1, torch.int8: 2}
    for t in (s0, s1):
        if t.dim() != 4 or t.dtype not in codes or not t.is_cuda or not t.is_contiguous():
            raise ValueError("sources must be contiguous [n, h, w, c] device tensors (float32, bfloat16, int8)")
    if s0.dtype != s1.dtype:
        raise ValueError("sources must share a dtype")
    n, ho, wo = s0.shape[0], s0.shape[1] << up0, s0.shape[2] << up0
    if tuple(s1.shape[:3]) != (n, ho >> up1, wo >> up1) or (up1 and (s1.shape[1] << 1, s1.shape[2] << 1) != (ho, wo)):
        raise ValueError("source sizes do not match")
    c0, c1 = s0.shape[3], s1.shape[3]
    if y is None:
        y = torch.empty((n, ho, wo, c0 + c1), dtype=s0.dtype, device=s0.device)
    if tuple(y.shape) != (n, ho, wo, c0 + c1) or y.dtype != s0.dtype or not y.is_contiguous():
        raise ValueError("y must be a contiguous [n, ho, wo, c0 + c1] tensor of the sources' dtype")
    st = lib().conv_upsample_concat(s0.data_ptr(), c0, up0, s1.data_ptr(), c1, up1, codes[s0.dtype], y.data_ptr(),
                                    n, ho, wo, _stream_handle(stream))
    _check(st, "conv_upsample_concat")
    return y


# ---- measurement probes (include/conv_probe.h) ---------------------------------
PROBE_MFMA_WORKGROUPS = 1024  # kProbeMfmaWorkgroups


def probe_mfma(dtype: str, iters: int, out: Optional[torch.Tensor] = None, stream=None) -> float:
    """Enqueue the matrix-core probe (bf16 or i8) and return the operations
    (2 x multiply-adds) it performs; time it with events on the same stream."""
    if out is None:
        out = torch.empty(4 * PROBE_MFMA_WORKGROUPS, dtype=torch.float32, device="cuda")
    if not out.is_cuda or out.dtype != torch.float32 or out.numel() < 4 * PROBE_MFMA_WORKGROUPS:
        raise ValueError("out must be a device float32 tensor of at least %d values" % (4 * PROBE_MFMA_WORKGROUPS))
    ops = ctypes.c_double()
    _check(lib().conv_probe_mfma(DTYPES[dtype], iters, out.data_ptr(), ctypes.byref(ops), _stream_handle(stream)),
           "conv_probe_mfma")
    return ops.value


def probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> int:
    """Enqueue the read+write stream dst <- src (same byte size, contiguous
    device tensors); returns the bytes moved through memory (read + write)."""
    for t, n in ((src, "src"), (dst, "dst")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous device tensor" % n)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    _check(lib().conv_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream_handle(stream)), "conv_probe_copy")
    return 2 * nbytes


def bfp8_bytes(c_out: int, k: int) -> int:
    return int(lib().conv_bfp8_bytes(c_out, k))


def pack_bfp8(w: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Encode OHWI weights (device, bf16 or fp32, contiguous) into the bfp8
    image conv_run takes for w_format "bfp8" (uint8, conv_bfp8_bytes)."""
    if not w.is_cuda or not w.is_contiguous() or w.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("w must be a contiguous device bf16 or float32 tensor")
    c_out = w.shape[0]
    k = w.numel() // c_out
    nbytes = bfp8_bytes(c_out, k)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    if out.dtype != torch.uint8 or out.numel() != nbytes or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint8 tensor of %d bytes" % nbytes)
    _check(lib().conv_pack_bfp8(w.data_ptr(), DTYPES["f32" if w.dtype == torch.float32 else "bf16"], c_out, k,
                                out.data_ptr(), _stream_handle(stream)), "conv_pack_bfp8")
    return out


def fusable(c1: Conv2d, c2: Conv2d) -> bool:
    """Whether conv_run_fused takes the pair (c1's layer, then c2's 1x1)."""
    return lib().conv_fuse_check(c1._plan, c2._plan) == 0


def describe_fused(c1: Conv2d, c2: Conv2d) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().conv_describe_fused(c1._plan, c2._plan, buf, 256), "conv_describe_fused")
    return buf.value.decode()


def run_fused(c1: Conv2d, c2: Conv2d, x: torch.Tensor, w1: torch.Tensor, b1: Optional[torch.Tensor],
              w2: torch.Tensor, b2: Optional[torch.Tensor], y: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """c2(c1(x)) in one launch; c1's output is never stored."""
    c1._chk(x, "x", TORCH_DT[c1.dtype], c1.in_shape)
    c1._chk(w1, "w1", c1._w_dtype(), c1.w_shape)
    c2._chk(w2, "w2", c2._w_dtype(), c2.w_shape)
    for b, n in ((b1, "b1"), (b2, "b2")):
        if b is not None:
            c1._chk(b, n, torch.float32, None)
    if y is None:
        y = c2.empty_output(x.device)
    c2._chk(y, "y", TORCH_DT[c2.out_dtype], c2.out_shape)
    st = lib().conv_run_fused(c1._plan, c2._plan, x.data_ptr(), w1.data_ptr(), None if b1 is None else b1.data_ptr(),
                              w2.data_ptr(), None if b2 is None else b2.data_ptr(), y.data_ptr(),
                              _stream_handle(stream))
    _check(st, "conv_run_fused")
    return y


def run_mosaic(conv: Conv2d, tiles: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor] = None,
               y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """conv (a window-stem plan on the canvas) applied to the mosaic of tiles
    [4m, th, tw, c] (float32 or bfloat16) without packing the canvas."""
    if tiles.dim() != 4 or tiles.shape[0] % 4:
        raise ValueError("tiles must be [4m, th, tw, c]")
    conv._chk(tiles, "tiles", tiles.dtype if tiles.dtype in (torch.float32, torch.bfloat16) else torch.float32, None)
    conv._chk(w, "w", conv._w_dtype(), conv.w_shape)
    if b is not None:
        conv._chk(b, "b", torch.float32, None)
    if y is None:
        y = conv.empty_output(tiles.device)
    conv._chk(y, "y", TORCH_DT[conv.out_dtype], conv.out_shape)
    q, th, tw, c = tiles.shape
    n, h, wd = conv.in_shape[:3]
    if q != 4 * n or 2 * th != h or 2 * tw != wd or c != conv.w_shape[3]:
        raise ValueError("tiles %s do not make the layer's %s canvas" % (tuple(tiles.shape), conv.in_shape))
    st = lib().conv_run_mosaic(conv._plan, tiles.data_ptr(), DTYPES["f32" if tiles.dtype == torch.float32 else "bf16"],
                               th, tw, w.data_ptr(), None if b is None else b.data_ptr(), y.data_ptr(),
                               _stream_handle(stream))
    _check(st, "conv_run_mosaic")
    return y


def run_upcat(conv: Conv2d, s0: torch.Tensor, up0: int, s1: torch.Tensor, up1: int, w: torch.Tensor,
              b: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """conv (a 1x1 layer) applied to the channel concat of s0 and s1, each
    repeated 2x in rows and columns when its up flag is 1, without writing
    the joined map (conv_run_upcat)."""
    n, h, wd, c = conv.in_shape
    dt = TORCH_DT[conv.dtype]
    c0 = s0.shape[-1] if s0.dim() == 4 else -1
    conv._chk(s0, "s0", dt, (n, h >> up0, wd >> up0, c0))
    conv._chk(s1, "s1", dt, (n, h >> up1, wd >> up1, c - c0))
    conv._chk(w, "w", conv._w_dtype(), conv.w_shape)
    if b is not None:
        conv._chk(b, "b", torch.int32 if conv.dtype == "i8" else torch.float32, None)
    if y is None:
        y = conv.empty_output(s0.device)
    conv._chk(y, "y", TORCH_DT[conv.out_dtype], conv.out_shape)
    st = lib().conv_run_upcat(conv._plan, s0.data_ptr(), c0, up0, s1.data_ptr(), up1, w.data_ptr(),
                              None if b is None else b.data_ptr(), y.data_ptr(), _stream_handle(stream))
    _check(st, "conv_run_upcat")
    return y
