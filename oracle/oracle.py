"""Python front end of the CPU oracle (ctypes over ``liboracle.so``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product package. It
shares no code with the HIP library.

Every function here marshals numpy arrays into the C oracle
(``conv_oracle.c``), which evaluates the convolution by its definition
(nanoinfer README, naive nested-loop reference convolution; see the C file's
header for the full statement). Float results come back as float64 and are
not rounded to the output type.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "conv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ACT = {"none": 0, "relu": 1, "relu6": 2, "mish": 3}

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2 -fopenmp, no fast-math, no FMA
    contraction). Returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.oracle_conv_float.argtypes = [P, P, P] + [I64] * 12 + [I, P, P, I]
    lib.oracle_conv_float.restype = I
    lib.oracle_conv_float_at.argtypes = [P, P, P] + [I64] * 12 + [I, P, I64, P, P, I]
    lib.oracle_conv_float_at.restype = I
    lib.oracle_conv_i8.argtypes = [P, P, P, P] + [I64] * 12 + [I, I, P, P, P, I]
    lib.oracle_conv_i8.restype = I
    lib.oracle_conv_i8_at.argtypes = [P, P, P, P] + [I64] * 12 + [I, I, P, I64, P, P, P, I]
    lib.oracle_conv_i8_at.restype = I
    lib.oracle_mosaic.argtypes = [P] + [I64] * 5 + [I, P]
    lib.oracle_mosaic.restype = I
    lib.oracle_spp.argtypes = [P, I] + [I64] * 4 + [P]
    lib.oracle_spp.restype = I
    lib.oracle_upcat.argtypes = [P, I64, I, P, I64, I, I64, I64, I64, I64, P]
    lib.oracle_upcat.restype = I
    lib.oracle_mish.argtypes = [ctypes.c_double]
    lib.oracle_mish.restype = ctypes.c_double
    lib.oracle_act.argtypes = [ctypes.c_double, I]
    lib.oracle_act.restype = ctypes.c_double
    lib.oracle_requant.argtypes = [ctypes.c_int32, ctypes.c_float, I, P]
    lib.oracle_requant.restype = I
    lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_num_threads.argtypes = [I]
    lib.oracle_num_threads.restype = I
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def out_hw(h, w, kh, kw, sh, sw, ph, pw):
    """Output size under the floor rule ``(H + 2p - K) // s + 1``."""
    return (h + 2 * ph - kh) // sh + 1, (w + 2 * pw - kw) // sw + 1


def _geom(x, wt, stride, pad, groups):
    n, h, w, cin = x.shape
    cout, kh, kw, cg = wt.shape
    if cg * groups != cin:
        raise ValueError("weight inner dim %d != cin/groups" % cg)
    sh, sw = stride
    ph, pw = pad
    return [n, h, w, cin, cout, kh, kw, sh, sw, ph, pw, groups]


def num_threads(n: int = 0) -> int:
    """Set (n > 0) and report the OpenMP thread count the oracle uses."""
    return _load().oracle_num_threads(n)


def conv_float(x, wt, b=None, stride=(1, 1), pad=(0, 0), groups=1, act="none",
               want_abs=True, threads=0):
    """Float convolution by definition, in double.

    x: [N,H,W,Cin] float32 (bf16 data widened exactly); wt: [Cout,KH,KW,Cin/g]
    float32; b: [Cout] float32 or None. Returns (r, A) float64 NHWC arrays:
    r = act(pre), A = |b| + sum |x*w| (None when want_abs is False).
    """
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    wt = np.ascontiguousarray(wt, dtype=np.float32)
    b = None if b is None else np.ascontiguousarray(b, dtype=np.float32)
    g = _geom(x, wt, stride, pad, groups)
    ho, wo = out_hw(g[1], g[2], g[5], g[6], g[7], g[8], g[9], g[10])
    if ho <= 0 or wo <= 0:
        raise ValueError("empty output")
    r = np.empty((g[0], ho, wo, g[4]), np.float64)
    a = np.empty_like(r) if want_abs else None
    st = lib.oracle_conv_float(_ptr(x), _ptr(wt), _ptr(b), *g, ACT[act],
                               _ptr(r), _ptr(a), threads)
    if st:
        raise ValueError("oracle_conv_float failed: %d" % st)
    return r, a


def conv_float_at(x, wt, b, idx, stride=(1, 1), pad=(0, 0), groups=1,
                  act="none", threads=0):
    """The float definition evaluated at flat NHWC output indices ``idx``."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    wt = np.ascontiguousarray(wt, dtype=np.float32)
    b = None if b is None else np.ascontiguousarray(b, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    g = _geom(x, wt, stride, pad, groups)
    r = np.empty(idx.shape[0], np.float64)
    a = np.empty_like(r)
    st = lib.oracle_conv_float_at(_ptr(x), _ptr(wt), _ptr(b), *g, ACT[act],
                                  _ptr(idx), idx.shape[0], _ptr(r), _ptr(a), threads)
    if st:
        raise ValueError("oracle_conv_float_at failed: %d" % st)
    return r, a


def conv_i8(x, wt, b=None, s=None, stride=(1, 1), pad=(0, 0), groups=1,
            act="none", out="i8", threads=0):
    """int8 convolution by definition (int64 accumulation).

    out="i32": returns the int32 checkpoint R32 = acc + b (ReLU allowed).
    out="i8":  returns (q int8, m float64) where m is the value rounded.
    """
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.int8)
    wt = np.ascontiguousarray(wt, dtype=np.int8)
    b = None if b is None else np.ascontiguousarray(b, dtype=np.int32)
    s = None if s is None else np.ascontiguousarray(s, dtype=np.float32)
    g = _geom(x, wt, stride, pad, groups)
    ho, wo = out_hw(g[1], g[2], g[5], g[6], g[7], g[8], g[9], g[10])
    shape = (g[0], ho, wo, g[4])
    if out == "i32":
        y32 = np.empty(shape, np.int32)
        st = lib.oracle_conv_i8(_ptr(x), _ptr(wt), _ptr(b), _ptr(s), *g, ACT[act], 1,
                                _ptr(y32), None, None, threads)
        if st:
            raise ValueError("oracle_conv_i8 failed: %d" % st)
        return y32
    y8 = np.empty(shape, np.int8)
    m = np.empty(shape, np.float64)
    st = lib.oracle_conv_i8(_ptr(x), _ptr(wt), _ptr(b), _ptr(s), *g, ACT[act], 0,
                            None, _ptr(y8), _ptr(m), threads)
    if st:
        raise ValueError("oracle_conv_i8 failed: %d" % st)
    return y8, m


def conv_i8_at(x, wt, b, s, idx, stride=(1, 1), pad=(0, 0), groups=1,
               act="none", out="i8", threads=0):
    """int8 definition at flat NHWC output indices ``idx``."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.int8)
    wt = np.ascontiguousarray(wt, dtype=np.int8)
    b = None if b is None else np.ascontiguousarray(b, dtype=np.int32)
    s = None if s is None else np.ascontiguousarray(s, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    g = _geom(x, wt, stride, pad, groups)
    cnt = idx.shape[0]
    if out == "i32":
        y32 = np.empty(cnt, np.int32)
        st = lib.oracle_conv_i8_at(_ptr(x), _ptr(wt), _ptr(b), _ptr(s), *g, ACT[act], 1,
                                   _ptr(idx), cnt, _ptr(y32), None, None, threads)
        if st:
            raise ValueError("oracle_conv_i8_at failed: %d" % st)
        return y32
    y8 = np.empty(cnt, np.int8)
    m = np.empty(cnt, np.float64)
    st = lib.oracle_conv_i8_at(_ptr(x), _ptr(wt), _ptr(b), _ptr(s), *g, ACT[act], 0,
                               _ptr(idx), cnt, None, _ptr(y8), _ptr(m), threads)
    if st:
        raise ValueError("oracle_conv_i8_at failed: %d" % st)
    return y8, m


def mosaic(tiles, c_pad=None, out="bf16"):
    """Pack tiles [4m,th,tw,c] (float32) into canvases [m,2th,2tw,c_pad].

    out="bf16" returns uint16 bf16 bit patterns (RNE); out="f32" float32.
    """
    lib = _load()
    tiles = np.ascontiguousarray(tiles, dtype=np.float32)
    q, th, tw, c = tiles.shape
    if q % 4:
        raise ValueError("tile count must be a multiple of 4")
    m = q // 4
    c_pad = c if c_pad is None else c_pad
    dt = np.uint16 if out == "bf16" else np.float32
    canvas = np.empty((m, 2 * th, 2 * tw, c_pad), dt)
    st = lib.oracle_mosaic(_ptr(tiles), m, th, tw, c, c_pad, 1 if out == "bf16" else 0,
                           _ptr(canvas))
    if st:
        raise ValueError("oracle_mosaic failed: %d" % st)
    return canvas


_SPP_DT = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.int8): 2}


def spp(x):
    """SPP max-pool block of x [n,h,w,c] (float32, bf16 bit patterns as
    uint16, or int8): returns [n,h,w,4c] of the same dtype, channel blocks
    max13, max9, max5, x (see oracle_spp in the C file)."""
    lib = _load()
    x = np.ascontiguousarray(x)
    if x.dtype not in _SPP_DT or x.ndim != 4:
        raise ValueError("spp takes a 4-d float32, uint16 (bf16) or int8 array")
    n, h, w, c = x.shape
    y = np.empty((n, h, w, 4 * c), x.dtype)
    st = lib.oracle_spp(_ptr(x), _SPP_DT[x.dtype], n, h, w, c, _ptr(y))
    if st:
        raise ValueError("oracle_spp failed: %d" % st)
    return y


def upcat(s0, up0, s1, up1):
    """Concatenate s0 and s1 ([n,h,w,c] arrays of one dtype) along channels
    at the output size, each repeated 2x in rows and columns where its up
    flag is set (see oracle_upcat in the C file)."""
    lib = _load()
    s0, s1 = np.ascontiguousarray(s0), np.ascontiguousarray(s1)
    if s0.dtype != s1.dtype or s0.ndim != 4 or s1.ndim != 4:
        raise ValueError("two 4-d arrays of one dtype")
    n, ho, wo = s0.shape[0], s0.shape[1] << up0, s0.shape[2] << up0
    if s1.shape[:3] != (n, ho >> up1, wo >> up1):
        raise ValueError("source sizes do not match")
    y = np.empty((n, ho, wo, s0.shape[3] + s1.shape[3]), s0.dtype)
    st = lib.oracle_upcat(_ptr(s0), s0.shape[3], up0, _ptr(s1), s1.shape[3], up1, s0.itemsize, n, ho, wo, _ptr(y))
    if st:
        raise ValueError("oracle_upcat failed: %d" % st)
    return y


def add_residual_float(r, a, res):
    """Residual-add epilogue for float outputs (zerolat.eu YOLOv4 report,
    section 9 "Four custom Tensix kernels", K2: the activation, then the skip tensor added,
    the sum written once). r, a: the oracle's unrounded activation output and
    absolute-value convolution; res: the residual's values (fp32, or bf16
    widened exactly). Returns (r + res, a + |res|) in float64, unrounded."""
    res = np.asarray(res, np.float64)
    return np.asarray(r, np.float64) + res, np.asarray(a, np.float64) + np.abs(res)


def add_residual_i8(m, res):
    """Residual-add epilogue for int8 outputs: res is int8 in the output's
    units, added to the activation's unrounded value m (float64) before the
    rounding: Q = clamp(round_half_even(m + res), -127, 127). Returns
    (Q int8, m + res)."""
    t = np.asarray(m, np.float64) + np.asarray(res, np.float64)
    return np.clip(np.rint(t), -127, 127).astype(np.int8), t


def mish(x: float) -> float:
    return _load().oracle_mish(float(x))


def act(x: float, name: str) -> float:
    return _load().oracle_act(float(x), ACT[name])


def requant(r32: int, s: float, act_name: str = "none"):
    """Requantise one int32 value; returns (q, m)."""
    m = ctypes.c_double()
    q = _load().oracle_requant(int(r32), float(s), ACT[act_name], ctypes.byref(m))
    return q, m.value


def f32_to_bf16_bits(v: float) -> int:
    return _load().oracle_f32_to_bf16(float(v))


def mish_tie_mask(m):
    """Elements whose pre-rounding value lies within 1e-5*max(1,|m|) of a
    half-integer: the only place a correct fp32 Mish may round differently
    from the double-precision one."""
    m = np.asarray(m, np.float64)
    frac = np.abs(m - np.floor(m) - 0.5)
    return frac <= 1e-5 * np.maximum(1.0, np.abs(m))
