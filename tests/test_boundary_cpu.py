"""The C-ABI boundary, on the CPU: the library loads, exports every symbol the
header declares, and rejects every malformed call with a named error before
anything would be enqueued (no GPU is touched by these tests)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

from convolution_conv2d_nhwc_amd import _lib
from convolution_conv2d_nhwc_amd._lib import Conv2d, ConvError, _Desc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv_nhwc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.library_path()),
                                reason="libconv_nhwc.so not built")


def header_functions():
    src = "".join(open(h).read() for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(conv_[a-z_0-9]+)\s*\(", src)))


def test_header_symbols_are_exported():
    names = header_functions()
    assert {"conv_prepare", "conv_run", "conv_destroy", "conv_out_shape", "conv_mosaic_pack",
            "conv_status_str", "conv_describe", "conv_algo_count", "conv_spp_maxpool",
            "conv_upsample_concat", "conv_run_residual", "conv_run_noalloc", "conv_probe_mfma",
            "conv_probe_copy"} <= set(names)
    L = ctypes.CDLL(_lib.library_path())
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (conv_[a-z_0-9]+)$", out, flags=re.M))
    assert set(names) <= exported


def desc(**kw):
    base = dict(n=1, h=8, w=8, c_in=16, c_out=16, kh=3, kw=3, stride_h=1, stride_w=1, pad_h=1,
                pad_w=1, groups=1, dtype=1, out_dtype=1, act=0, algo=0)
    base.update(kw)
    return _Desc(**base)


def prepare(d):
    p = ctypes.c_void_p()
    st = _lib.lib().conv_prepare(ctypes.byref(d), ctypes.byref(p))
    return st, p


@pytest.mark.parametrize("kw,code", [
    (dict(n=0), -2), (dict(h=-1), -2), (dict(c_in=0), -2), (dict(kh=0), -2),
    (dict(stride_w=0), -2), (dict(pad_h=-1), -2),
    (dict(h=2, pad_h=0), -2),                      # kernel larger than padded input
    (dict(groups=3), -2),                          # 16 % 3 != 0
    (dict(groups=4), -3),                          # grouped, not depthwise
    (dict(groups=16, kh=5, kw=5, pad_h=2, pad_w=2), -3),  # depthwise must be 3x3
    (dict(groups=16, c_out=32), -3),               # depthwise needs c_out == c_in (32 % 16 == 0)
    (dict(dtype=0, out_dtype=1), -3),              # f32 -> bf16 not offered
    (dict(dtype=1, out_dtype=2), -3),
    (dict(dtype=2, out_dtype=1), -3),
    (dict(dtype=5, out_dtype=5), -3),
    (dict(act=7), -3),
    (dict(dtype=2, out_dtype=3, act=3), -3),       # int32 checkpoint: NONE/RELU only
    (dict(dtype=2, out_dtype=3, act=2), -3),
    (dict(algo=99), -3),
    (dict(dtype=0, out_dtype=0, algo=1), -3),      # algo only for the MFMA path
    (dict(n=1, h=1 << 15, w=1 << 15, c_in=8), -3),  # x over 2^31 bytes
    # a reduction of 2^24 bytes per output (kh*kw*c_in*esz): the kernels'
    # (tap, channel) split of a reduction index is exact only below that
    (dict(n=1, h=1, w=1, c_in=1 << 23, c_out=1, kh=1, kw=1, pad_h=0, pad_w=0), -3),
    (dict(n=1, h=1, w=1, c_in=1 << 24, c_out=1, kh=1, kw=1, pad_h=0, pad_w=0, dtype=2, out_dtype=2), -3),
])
def test_prepare_rejects(kw, code):
    st, p = prepare(desc(**kw))
    assert st == code
    assert not p.value
    assert _lib.lib().conv_status_str(st).decode().startswith(_lib.STATUS[code])


def test_prepare_null():
    p = ctypes.c_void_p()
    assert _lib.lib().conv_prepare(None, ctypes.byref(p)) == -1
    d = desc()
    assert _lib.lib().conv_prepare(ctypes.byref(d), None) == -1


@pytest.mark.parametrize("layer,expect", [
    (dict(c_in=3, c_out=32, dtype="bf16"), "smallk dtype=bf16 out=bf16"),
    (dict(c_in=61, c_out=32, dtype="bf16"), "igemm dtype=bf16 out=bf16 loader=generic"),
    (dict(c_in=32, c_out=64, dtype="bf16"), "loader=vec16"),
    (dict(c_in=64, c_out=64, kh=1, kw=1, pad=(0, 0), dtype="bf16"), "loader=1x1"),
    (dict(c_in=64, c_out=64, kh=1, kw=1, pad=(0, 0), stride=(2, 2), dtype="bf16"), "loader=tap"),
    (dict(c_in=64, c_out=64, dtype="bf16"), "loader=tap"),
    (dict(c_in=128, c_out=64, kh=5, kw=5, pad=(2, 2), dtype="i8"), "loader=tap"),
    (dict(c_in=128, c_out=64, kh=7, kw=5, pad=(3, 3), dtype="i8"), "loader=vec16"),  # 35 taps > 32
    (dict(c_in=8, c_out=8, dtype="i8", out_dtype="i8"), "smallk dtype=i8"),  # 8 bytes per pixel, K=72
    (dict(c_in=24, c_out=8, dtype="i8", out_dtype="i8"), "loader=generic"),  # K = 216 bytes
    (dict(c_in=40, c_out=8, dtype="i8", out_dtype="i8"), "loader=generic"),  # K = 360 bytes
    (dict(c_in=16, c_out=16, dtype="i8", out_dtype="i32"), "out=i32 loader=vec16"),
    (dict(c_in=64, c_out=64, groups=64, dtype="i8"), "dw3x3 dtype=i8"),
    (dict(c_in=1, c_out=8, dtype="f32"), "direct_f32"),
    (dict(c_in=4, c_out=4, groups=4, dtype="f32"), "dw3x3 dtype=f32 out=f32 stride=1x1 rows"),
    (dict(c_in=4, c_out=4, groups=4, dtype="f32", stride=(2, 2)), "dw3x3 dtype=f32 out=f32 loader=vec16"),
    (dict(c_in=6, c_out=6, groups=6, dtype="bf16"), "dw3x3 dtype=bf16 out=bf16 loader=generic"),
    # long reductions over 128-byte channel blocks: the large-layer kernel
    (dict(n=16, h=40, w=40, c_in=512, c_out=512, dtype="bf16"), "igemm_xl dtype=bf16 out=bf16 loader=tap tile=8"),
    (dict(n=16, h=20, w=20, c_in=512, c_out=1024, dtype="bf16"), "igemm_xl dtype=bf16 out=bf16 loader=tap tile=9"),
    (dict(n=16, h=40, w=40, c_in=512, c_out=512, dtype="i8"), "igemm_xl dtype=i8 out=i8 loader=tap tile=8"),
    (dict(n=16, h=80, w=80, c_in=256, c_out=256, dtype="i8"), "igemm_xl dtype=i8 out=i8 loader=tap tile=8"),
    (dict(n=16, h=80, w=80, c_in=128, c_out=128, dtype="i8"), "igemm dtype=i8 out=i8 loader=tap"),  # short K, 128 channels
    (dict(n=16, h=160, w=160, c_in=128, c_out=128, dtype="bf16"), "loader=tap tile=2 co128xpx128"),
    (dict(n=16, h=40, w=40, c_in=512, c_out=320, dtype="bf16"), "igemm dtype=bf16"),  # Cout % 128
    # reductions of at most 256 bytes on the 64x64 tile: the weight-stationary kernel
    (dict(c_in=64, c_out=64, kh=1, kw=1, pad=(0, 0), dtype="bf16"), "igemm_ws dtype=bf16 out=bf16 loader=1x1"),
    (dict(c_in=128, c_out=64, kh=1, kw=1, pad=(0, 0), dtype="i8"), "igemm_ws dtype=i8 out=i8 loader=1x1"),
    (dict(c_in=24, c_out=64, kh=1, kw=1, pad=(0, 0), stride=(2, 2), dtype="bf16"),
     "igemm_ws dtype=bf16 out=bf16 loader=vec16"),
    (dict(c_in=64, c_out=64, dtype="bf16"), "igemm dtype=bf16 out=bf16 loader=tap"),  # K = 1152 bytes
    (dict(c_in=192, c_out=64, kh=1, kw=1, pad=(0, 0), dtype="bf16"), "igemm dtype=bf16 out=bf16 loader=1x1"),
])
def test_path_selection(layer, expect):
    args = dict(n=1, h=16, w=16, kh=3, kw=3, stride=(1, 1), pad=(1, 1), groups=1, act="relu")
    args.update(layer)
    c = Conv2d(args["n"], args["h"], args["w"], args["c_in"], args["c_out"], args["kh"], args["kw"],
               args["stride"], args["pad"], args["groups"], args["dtype"], args.get("out_dtype"), args["act"])
    assert expect in c.describe()
    c.close()


def test_out_shape_floor_rule_and_per_axis_pads():
    # the keyword-spotting stem: 49x10, 10x4 kernel, stride 2, pad (5, 1)
    c = Conv2d(1, 49, 10, 1, 64, 10, 4, (2, 2), (5, 1), dtype="i8")
    assert c.out_shape == (1, 25, 5, 64)
    c.close()
    c = Conv2d(1, 49, 10, 1, 64, 10, 4, (2, 2), (1, 5), dtype="i8")
    assert c.out_shape == (1, 21, 9, 64)
    c.close()


def test_forced_algo_and_count():
    """Every algo id forces its own kernel configuration: all but the last on
    a layer all of them accept (1x1 over one 128-byte channel block, Cout =
    256), the last (the halo kernel) on a 3x3 layer over 64 channels. The
    large-layer kernel refuses a Cout that is not a multiple of its channel
    tile, the weight-stationary kernel a reduction over 256 bytes, the halo
    kernel anything but a 3x3 bf16 layer over 32 or 64 channels at stride 1
    or 2."""
    n = _lib.lib().conv_algo_count()
    assert n >= 2
    kinds = set()
    for a in range(1, n):
        c = Conv2d(1, 20, 20, 64, 256, 1, 1, (1, 1), (0, 0), dtype="bf16", algo=a)
        d = c.describe()
        assert "tile=%d " % a in d
        kinds.add(d.split()[0])
        c.close()
    assert kinds == {"igemm", "igemm_xl", "igemm_ws"}
    c = Conv2d(1, 20, 20, 64, 256, 3, 3, (1, 1), (1, 1), dtype="bf16", algo=n)
    assert c.describe().startswith("halo ") and "tile=%d " % n in c.describe(), c.describe()
    c.close()
    ws = n - 1
    with pytest.raises(ConvError):
        Conv2d(1, 20, 20, 64, 256, 3, 3, (1, 1), (1, 1), dtype="bf16", algo=ws)  # 1152-byte reduction
    for kw in (dict(cin=64, k=1), dict(cin=48, k=3), dict(cin=128, k=3), dict(cin=64, k=5), dict(cin=64, k=3, s=3),
               dict(cin=64, k=3, dtype="i8", out_dtype="i8"), dict(cin=64, k=3, w_format="bfp8"),
               dict(cin=64, k=3, cout=62)):
        a = dict(kw)
        cin, k, s = a.pop("cin"), a.pop("k"), a.pop("s", 1)
        cout = a.pop("cout", 64)
        with pytest.raises(ConvError):
            Conv2d(1, 20, 20, cin, cout, k, k, (s, s), (k // 2, k // 2), **dict(dict(dtype="bf16"), **a), algo=n)
    xl = [a for a in range(1, n)
          if Conv2d(1, 20, 20, 64, 256, 1, 1, (1, 1), (0, 0), dtype="bf16", algo=a).describe().startswith("igemm_xl")]
    for a in xl:
        with pytest.raises(ConvError):
            Conv2d(1, 20, 20, 64, 64, 3, 3, (1, 1), (1, 1), dtype="bf16", algo=a)   # Cout 64
        with pytest.raises(ConvError):
            Conv2d(1, 20, 20, 48, 256, 3, 3, (1, 1), (1, 1), dtype="bf16", algo=a)  # 96-byte channel blocks


def test_depthwise_forced_rows():
    """algo 1..4 on a stride-1 depthwise layer forces 1, 2, 4, 8 rows per lane
    of the row-window kernel; other algos, strided layers and channel counts
    that are not a multiple of 4 are refused."""
    for a, th in ((1, 1), (2, 2), (3, 4), (4, 8)):
        for dt, out, pat in (("bf16", None, r"dw3x3_rows_kernel<unsigned short, 4, \d+, %d, "),
                             ("i8", "i8", r"dw3x3_i8_kernel<\d+, %d, "), ("f32", None, r"dw3x3_rows_kernel<float, 4, \d+, %d, ")):
            c = Conv2d(1, 9, 9, 16, 16, 3, 3, (1, 1), (1, 1), groups=16, dtype=dt, out_dtype=out, algo=a)
            assert re.search(pat % th, c.describe()), c.describe()
            c.close()
    for kw in (dict(algo=5), dict(algo=1, stride=(2, 2)), dict(algo=1, c=6)):
        ch = kw.pop("c", 16)
        st = kw.pop("stride", (1, 1))
        with pytest.raises(ConvError):
            Conv2d(1, 9, 9, ch, ch, 3, 3, st, (1, 1), groups=ch, dtype="bf16", **kw)


def fake(addr):
    return ctypes.c_void_p(addr)


def test_residual_argument_checks_before_launch():
    """conv_run_residual refuses a NULL or misaligned residual, one that
    partly overlaps y, and int32-checkpoint plans, before any launch."""
    c = Conv2d(1, 8, 8, 16, 16, 3, 3, (1, 1), (1, 1), dtype="bf16")
    L = _lib.lib()
    P = c._plan
    X, W, B, Y, R = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
    assert L.conv_run_residual(P, X, W, B, None, Y, None) == -1
    assert L.conv_run_residual(None, X, W, B, R, Y, None) == -1
    assert L.conv_run_residual(P, X, W, B, R + 8, Y, None) == -4
    assert L.conv_run_residual(P, X, W, B, Y + 16, Y, None) == -5
    c.close()
    c32 = Conv2d(1, 8, 8, 16, 16, 3, 3, (1, 1), (1, 1), dtype="i8", out_dtype="i32")
    assert L.conv_run_residual(c32._plan, X, W, B, R, Y, None) == -3
    c32.close()


def test_upcat_argument_checks_before_launch():
    """conv_upsample_concat refuses bad arguments on the host."""
    L = _lib.lib()
    A, B, Y = 0x10000000, 0x20000000, 0x40000000
    ok = (1, 40, 40, None)
    assert L.conv_upsample_concat(None, 256, 1, B, 256, 0, 1, Y, *ok) == -1
    assert L.conv_upsample_concat(A, 256, 1, B, 256, 0, 1, None, *ok) == -1
    assert L.conv_upsample_concat(A, 256, 1, B, 256, 0, 1, Y, 1, 41, 40, None) == -2   # odd height, upsampled
    assert L.conv_upsample_concat(A, 256, 2, B, 256, 0, 1, Y, *ok) == -2               # up flag not 0/1
    assert L.conv_upsample_concat(A, 0, 1, B, 256, 0, 1, Y, *ok) == -2
    assert L.conv_upsample_concat(A, 256, 1, B, 256, 0, 3, Y, *ok) == -3               # int32
    assert L.conv_upsample_concat(A, 12, 1, B, 256, 0, 1, Y, *ok) == -3                # 24-byte pixel
    assert L.conv_upsample_concat(A, 8, 1, B, 16, 0, 2, Y, *ok) == -3                  # int8, 8 bytes
    assert L.conv_upsample_concat(A + 8, 256, 1, B, 256, 0, 1, Y, *ok) == -4
    assert L.conv_upsample_concat(A, 256, 1, B, 256, 0, 1, B + 64, *ok) == -5          # y overlaps s1
    assert L.conv_upsample_concat(A, 8, 0, B, 8, 0, 1, Y, 70000, 1, 2, None) == -3     # n * ho > 65535


def test_spp_argument_checks_before_launch():
    """conv_spp_maxpool refuses bad arguments on the host, before any device
    call; the fake addresses are never dereferenced."""
    L = _lib.lib()
    X, Y = 0x10000000, 0x20000000
    ok = (1, 20, 20, 512)
    assert L.conv_spp_maxpool(None, 1, Y, *ok, None) == -1
    assert L.conv_spp_maxpool(X, 1, None, *ok, None) == -1
    assert L.conv_spp_maxpool(X, 1, Y, 0, 20, 20, 512, None) == -2
    assert L.conv_spp_maxpool(X, 1, Y, 1, 20, -1, 512, None) == -2
    assert L.conv_spp_maxpool(X, 3, Y, *ok, None) == -3             # int32 is not a map dtype
    assert L.conv_spp_maxpool(X, 1, Y, 1, 20, 20, 12, None) == -3    # bf16 channels not a multiple of 8
    assert L.conv_spp_maxpool(X, 0, Y, 1, 20, 20, 6, None) == -3     # fp32 channels not a multiple of 4
    assert L.conv_spp_maxpool(X, 1, Y, 1, 64, 33, 8, None) == -3     # 2112 pixels
    assert L.conv_spp_maxpool(X + 8, 1, Y, *ok, None) == -4
    assert L.conv_spp_maxpool(X, 1, Y + 4, *ok, None) == -4
    assert L.conv_spp_maxpool(X, 1, X + 1024 * 16, *ok, None) == -5  # y overlaps x


def test_run_pointer_checks_before_launch():
    """NULL, misaligned and overlapping pointers are refused on the host;
    the fake addresses are never dereferenced or handed to a kernel."""
    c = Conv2d(1, 8, 8, 16, 16, 3, 3, (1, 1), (1, 1), dtype="bf16")
    L = _lib.lib()
    P = c._plan
    X, W, B, Y = 0x10000000, 0x20000000, 0x30000000, 0x40000000
    assert L.conv_run(None, X, W, B, Y, None) == -1
    assert L.conv_run(P, None, W, B, Y, None) == -1
    assert L.conv_run(P, X, None, B, Y, None) == -1
    assert L.conv_run(P, X, W, B, None, None) == -1
    assert L.conv_run(P, X + 8, W, B, Y, None) == -4
    assert L.conv_run(P, X, W + 2, B, Y, None) == -4
    assert L.conv_run(P, X, W, B, Y + 4, None) == -4
    assert L.conv_run(P, X, W, B + 2, Y, None) == -4
    xbytes = 8 * 8 * 16 * 2
    assert L.conv_run(P, X, W, B, X + xbytes - 16 * 4, None) == -5  # y starts inside x
    assert L.conv_run(P, Y + 2048 - 1024, W, B, Y, None) == -5      # x starts inside y
    assert L.conv_run(P, X, W, Y + 64, Y, None) == -5               # b inside y
    c.close()
    ci = Conv2d(1, 8, 8, 16, 16, 3, 3, (1, 1), (1, 1), dtype="i8", out_dtype="i8")
    assert L.conv_run(ci._plan, X, W, None, Y, None) == -1  # int8 output needs the scale block
    ci.close()


def test_mosaic_argument_checks():
    L = _lib.lib()
    T, C = 0x10000000, 0x50000000
    assert L.conv_mosaic_pack(None, 0, C, 1, 1, 4, 4, 3, 3, None) == -1
    assert L.conv_mosaic_pack(T, 0, C, 1, 0, 4, 4, 3, 3, None) == -2
    assert L.conv_mosaic_pack(T, 0, C, 1, 1, 4, 4, 3, 2, None) == -2   # c_pad < c
    assert L.conv_mosaic_pack(T, 2, C, 1, 1, 4, 4, 3, 3, None) == -3   # int8 tiles
    assert L.conv_mosaic_pack(T + 4, 0, C, 1, 1, 4, 4, 3, 3, None) == -4
    assert L.conv_mosaic_pack(T, 0, T + 64, 1, 1, 4, 4, 3, 3, None) == -5


def test_noalloc_null_desc_and_status_text():
    # a NULL description is refused before any device call
    assert _lib.lib().conv_run_noalloc(None, 16, 16, None, None, 16, None) == -1
    assert _lib.lib().conv_status_str(-8).decode().startswith("CONV_E_SCRATCH")
    assert _lib.STATUS[-8] == "CONV_E_SCRATCH"


def test_bfp8_sizes_and_plan_checks():
    L = _lib.lib()
    assert L.conv_bfp8_bytes(64, 576) == 64 * 576 + 64 * 36
    assert L.conv_bfp8_bytes(5, 20) == 5 * 32 + 5 * 2
    assert L.conv_bfp8_bytes(0, 5) == 0 and L.conv_bfp8_bytes(3, -1) == 0
    st, p = prepare(desc(c_in=64, c_out=64, w_format=1))
    assert st == 0
    buf = ctypes.create_string_buffer(256)
    L.conv_describe(p, buf, 256)
    assert b"w=bfp8" in buf.value and buf.value.startswith(b"igemm "), buf.value
    L.conv_destroy(p)
    for kw in (dict(c_in=3, c_out=32, w_format=1),                       # stem: generic loader
               dict(c_in=64, c_out=64, dtype=2, out_dtype=2, w_format=1),  # int8
               dict(c_in=64, c_out=64, groups=64, w_format=1),             # depthwise
               dict(c_in=64, c_out=256, algo=5, w_format=1),               # a large-layer tile
               dict(c_in=64, c_out=64, w_format=2)):                       # no such format
        st, p = prepare(desc(**kw))
        assert st == -3 and not p.value, kw


def test_bfp8_pack_argument_checks_before_launch():
    L = _lib.lib()
    assert L.conv_pack_bfp8(None, 1, 4, 16, 4096, None) == -1
    assert L.conv_pack_bfp8(4096, 1, 0, 16, 8192, None) == -2
    assert L.conv_pack_bfp8(4096, 2, 4, 16, 8192, None) == -3      # int8 weights
    assert L.conv_pack_bfp8(4096, 1, 4, 16, 8200, None) == -4      # packed not 16-byte aligned
    assert L.conv_pack_bfp8(4096, 1, 4, 16, 4096 + 64, None) == -5  # overlapping


def test_destroy_null_is_noop():
    assert _lib.lib().conv_destroy(None) == 0


def test_python_binding_validates_tensors():
    import torch
    c = Conv2d(1, 8, 8, 16, 16, 3, 3, (1, 1), (1, 1), dtype="bf16")
    x = torch.zeros(1, 8, 8, 16, dtype=torch.bfloat16)
    w = torch.zeros(16, 3, 3, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        c.run(x, w)   # host tensors are refused before any library call
    c.close()


def _shape(c):
    return " %dx%d" % (c.w_shape[1], c.w_shape[2])


def _halo_fusable(c):
    cout, kh, kw, cin = c.w_shape
    stride = 2 if c.out_shape[1] * 2 <= c.in_shape[1] else 1
    return kh == kw == 3 and cin in (32, 64) and cout in (64, 128) and not (cout == 64 and stride == 2 and cin == 64)


def test_fuse_check_pairs():
    """conv_fuse_check accepts a KxK bf16 layer with 64 or 128 output channels
    followed by a 1x1 bf16 layer on its output with at most 64 channels (a
    multiple of 4), and refuses everything else."""
    def C(h, w, cin, cout, k, s=1, **kw):
        return Conv2d(1, h, w, cin, cout, k, k, (s, s), (k // 2, k // 2), **dict(dict(dtype="bf16"), **kw))

    ok = [(C(20, 20, 64, 64, 3), C(20, 20, 64, 64, 1)),
          (C(20, 20, 64, 128, 3, s=2), C(10, 10, 128, 32, 1)),
          (C(17, 9, 32, 64, 3), C(17, 9, 64, 4, 1)),
          (C(12, 12, 128, 64, 5), C(12, 12, 64, 60, 1))]
    bad = [(C(20, 20, 64, 96, 3), C(20, 20, 96, 64, 1)),            # 96 intermediate channels
           (C(20, 20, 64, 64, 3), C(20, 20, 64, 128, 1)),           # 128 output channels
           (C(20, 20, 64, 64, 3), C(20, 20, 64, 62, 1)),            # not a multiple of 4
           (C(20, 20, 64, 64, 3), C(20, 20, 64, 64, 3)),            # second layer 3x3
           (C(20, 20, 64, 64, 3), C(10, 10, 64, 64, 1, s=2)),       # wrong shape / stride
           (C(20, 20, 64, 64, 3), C(20, 20, 64, 64, 1, act="none", dtype="f32")),
           (C(20, 20, 3, 64, 3), C(20, 20, 64, 64, 1)),             # stem gather
           (C(20, 20, 64, 64, 3, dtype="i8", out_dtype="i8"), C(20, 20, 64, 64, 1, dtype="i8", out_dtype="i8")),
           (C(20, 20, 64, 64, 3, groups=64), C(20, 20, 64, 64, 1)),  # depthwise
           (C(20, 20, 64, 64, 3, w_format="bfp8"), C(20, 20, 64, 64, 1)),
           (C(20, 20, 64, 64, 3), C(20, 20, 64, 64, 1, w_format="bfp8"))]
    for a, b in ok:
        assert _lib.fusable(a, b), (a.describe(), b.describe())
        d = _lib.describe_fused(a, b)
        # 3x3 first layers over 32 / 64 channels fuse on the halo kernel
        # (except 64 -> 64 at stride 2), the rest on the implicit GEMM
        assert d.startswith("halo fused_1x1 " if " 3x3" in _shape(a) and _halo_fusable(a) else "igemm fused_1x1 "), d
        assert d.endswith(", 1>"), d
    # a first layer forced onto an implicit-GEMM tile keeps that kernel
    a, b = C(20, 20, 64, 64, 3, algo=1), C(20, 20, 64, 64, 1)
    assert _lib.describe_fused(a, b).startswith("igemm fused_1x1 ")
    a.close()
    b.close()
    for a, b in bad:
        assert not _lib.fusable(a, b), (a.describe(), b.describe())
        with pytest.raises(ConvError):
            _lib.describe_fused(a, b)
    L = _lib.lib()
    assert L.conv_fuse_check(None, ok[0][1]._plan) == -1
    assert L.conv_fuse_check(ok[0][0]._plan, None) == -1
    for a, b in ok + bad:
        a.close()
        b.close()


def test_run_fused_pointer_checks_before_launch():
    a = Conv2d(1, 8, 8, 64, 64, 3, 3, (1, 1), (1, 1), dtype="bf16")
    b = Conv2d(1, 8, 8, 64, 64, 1, 1, (1, 1), (0, 0), dtype="bf16")
    bad = Conv2d(1, 8, 8, 64, 128, 1, 1, (1, 1), (0, 0), dtype="bf16")
    L = _lib.lib()
    X, W1, B1, W2, B2, Y = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000, 0x60000000
    P1, P2 = a._plan, b._plan
    assert L.conv_run_fused(None, P2, X, W1, B1, W2, B2, Y, None) == -1
    assert L.conv_run_fused(P1, P2, None, W1, B1, W2, B2, Y, None) == -1
    assert L.conv_run_fused(P1, P2, X, W1, B1, None, B2, Y, None) == -1
    assert L.conv_run_fused(P1, P2, X, W1, B1, W2, B2, None, None) == -1
    assert L.conv_run_fused(P1, bad._plan, X, W1, B1, W2, B2, Y, None) == -3
    assert L.conv_run_fused(P1, P2, X + 8, W1, B1, W2, B2, Y, None) == -4
    assert L.conv_run_fused(P1, P2, X, W1, B1, W2 + 4, B2, Y, None) == -4
    assert L.conv_run_fused(P1, P2, X, W1, B1, W2, B2 + 2, Y, None) == -4
    assert L.conv_run_fused(P1, P2, X, W1, B1, W2, B2, Y + 8, None) == -4
    assert L.conv_run_fused(P1, P2, X, W1, B1, W2, B2, X + 1024, None) == -5  # y inside x
    assert L.conv_run_fused(P1, P2, X, W1, B1, Y + 256, B2, Y, None) == -5    # w2 inside y
    assert L.conv_run_fused(P1, P2, X, W1, Y + 64, W2, B2, Y, None) == -5     # b1 inside y
    for c in (a, b, bad):
        c.close()


def test_pixel_stride_checks():
    """x_pixel_stride: 8 with c_in <= 8 on a 3x3 stride-1 bf16 layer is the
    window stem kernel; every other non-dense stride is refused."""
    base = dict(n=1, h=20, w=20, c_in=3, c_out=32, kh=3, kw=3, stride=(1, 1), pad=(1, 1), dtype="bf16",
                act="mish", x_stride=8)
    c = Conv2d(**base)
    assert c.describe().startswith("stem_window ") and c.in_shape == (1, 20, 20, 8), c.describe()
    c.close()
    c = Conv2d(**dict(base, c_in=16, x_stride=16))  # dense
    assert not c.describe().startswith("stem_window ")
    c.close()
    for kw, code in ((dict(stride=(2, 2)), "CONV_E_UNSUPPORTED"), (dict(kh=5, kw=5, pad=(2, 2)), "CONV_E_UNSUPPORTED"),
                     (dict(c_in=16, x_stride=8), "CONV_E_SHAPE"), (dict(x_stride=4), "CONV_E_UNSUPPORTED"),
                     (dict(dtype="i8", out_dtype="i8"), "CONV_E_UNSUPPORTED"), (dict(algo=1), "CONV_E_UNSUPPORTED"),
                     (dict(pad=(2, 2)), "CONV_E_UNSUPPORTED"), (dict(w_format="bfp8"), "CONV_E_UNSUPPORTED")):
        with pytest.raises(ConvError) as e:
            Conv2d(**dict(base, **kw))
        assert e.value.name == code, (kw, e.value.name)


def test_run_mosaic_checks_before_launch():
    L = _lib.lib()
    stem = Conv2d(1, 20, 30, 3, 32, 3, 3, (1, 1), (1, 1), dtype="bf16", act="mish", x_stride=8)
    dense = Conv2d(1, 20, 30, 3, 32, 3, 3, (1, 1), (1, 1), dtype="bf16", act="mish")
    T, W, B, Y = 0x10000000, 0x20000000, 0x30000000, 0x40000000
    P = stem._plan
    assert L.conv_run_mosaic(None, T, 0, 10, 15, W, B, Y, None) == -1
    assert L.conv_run_mosaic(P, None, 0, 10, 15, W, B, Y, None) == -1
    assert L.conv_run_mosaic(P, T, 0, 10, 15, W, B, None, None) == -1
    assert L.conv_run_mosaic(P, T, 2, 10, 15, W, B, Y, None) == -3          # int8 tiles
    assert L.conv_run_mosaic(dense._plan, T, 0, 10, 15, W, B, Y, None) == -3  # not a window-stem plan
    assert L.conv_run_mosaic(P, T, 0, 10, 16, W, B, Y, None) == -3          # tiles do not make the canvas
    assert L.conv_run_mosaic(P, T + 2, 0, 10, 15, W, B, Y, None) == -4      # fp32 tiles need 4-byte alignment
    assert L.conv_run_mosaic(P, T + 2, 1, 10, 15, W, B, T + 64, None) == -5  # bf16 tiles: 2 is enough (then alias)
    assert L.conv_run_mosaic(P, T, 0, 10, 15, W + 8, B, Y, None) == -4
    assert L.conv_run_mosaic(P, T, 0, 10, 15, W, B, T + 64, None) == -5     # y inside the tiles
    stem.close()
    dense.close()


def test_run_upcat_checks_before_launch():
    """conv_run_upcat refuses, before any launch, missing pointers, plans that
    are not a dense 1x1 stride-1 unpadded bf16/int8 layer, bad up flags and
    channel splits, splits that are not whole 128-byte blocks, misalignment
    and an output overlapping an input."""
    L = _lib.lib()
    c = Conv2d(1, 40, 40, 512, 256, 1, 1, (1, 1), (0, 0), dtype="bf16", act="mish")
    odd = Conv2d(1, 41, 40, 512, 256, 1, 1, (1, 1), (0, 0), dtype="bf16", act="mish")
    k3 = Conv2d(1, 40, 40, 512, 256, 3, 3, (1, 1), (1, 1), dtype="bf16", act="mish")
    S0, S1, W, B, Y = 0x10000000, 0x20000000, 0x30000000, 0x38000000, 0x40000000
    P = c._plan
    assert L.conv_run_upcat(None, S0, 256, 1, S1, 0, W, B, Y, None) == -1
    assert L.conv_run_upcat(P, None, 256, 1, S1, 0, W, B, Y, None) == -1
    assert L.conv_run_upcat(P, S0, 256, 1, None, 0, W, B, Y, None) == -1
    assert L.conv_run_upcat(P, S0, 256, 1, S1, 0, W, B, None, None) == -1
    assert L.conv_run_upcat(k3._plan, S0, 256, 1, S1, 0, W, B, Y, None) == -3   # not a 1x1 layer
    assert L.conv_run_upcat(P, S0, 256, 2, S1, 0, W, B, Y, None) == -2         # up flag
    assert L.conv_run_upcat(odd._plan, S0, 256, 1, S1, 0, W, B, Y, None) == -2  # odd height, upsampled
    assert L.conv_run_upcat(P, S0, 0, 1, S1, 0, W, B, Y, None) == -2           # empty first map
    assert L.conv_run_upcat(P, S0, 512, 1, S1, 0, W, B, Y, None) == -2         # empty second map
    assert L.conv_run_upcat(P, S0, 96, 1, S1, 0, W, B, Y, None) == -3          # 192-byte channel split
    assert L.conv_run_upcat(P, S0 + 8, 256, 1, S1, 0, W, B, Y, None) == -4
    assert L.conv_run_upcat(P, S0, 256, 1, S1, 0, W, B + 2, Y, None) == -4
    assert L.conv_run_upcat(P, S0, 256, 1, S1, 0, W, B, S1 + 4096, None) == -5  # y inside s1
    for x in (c, odd, k3):
        x.close()
