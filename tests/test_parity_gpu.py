"""GPU parity: the HIP path through the C ABI against the CPU oracle, element
by element on the same seeded inputs (small shapes that span several tiles
with ragged tails, every tile configuration of the MFMA kernel forced in
turn), plus the hygiene checks: canary-filled outputs, guard bands,
determinism, a non-default stream and HIP-graph replay."""
import re
from dataclasses import replace

import numpy as np
import pytest
import torch

from convolution_conv2d_nhwc_amd import _lib
from convolution_conv2d_nhwc_amd.data import Layer, random_layer_tensors
from oracle import oracle
from tests import helpers as H

pytestmark = pytest.mark.gpu

ALGO_COUNT = _lib.lib().conv_algo_count()


def _algo_describe(algo):
    # a layer every forced algorithm but the halo kernel accepts: 1x1 over one
    # 128-byte channel block (a 128-byte reduction), Cout = 256; the halo
    # kernel's is a 3x3 layer over 64 channels
    try:
        return _lib.Conv2d(1, 20, 20, 64, 256, 1, 1, (1, 1), (0, 0), dtype="bf16", algo=algo).describe()
    except _lib.ConvError:
        return _lib.Conv2d(1, 20, 20, 64, 256, 3, 3, (1, 1), (1, 1), dtype="bf16", algo=algo).describe()


ALGO_DESC = {a: _algo_describe(a) for a in range(1, ALGO_COUNT + 1)}
TILE_ALGOS = [a for a, d in ALGO_DESC.items() if d.startswith("igemm ")]
XL_ALGOS = [a for a, d in ALGO_DESC.items() if d.startswith("igemm_xl ")]
WS_ALGOS = [a for a, d in ALGO_DESC.items() if d.startswith("igemm_ws ")]
HALO_ALGOS = [a for a, d in ALGO_DESC.items() if d.startswith("halo ")]
assert len(TILE_ALGOS) + len(XL_ALGOS) + len(WS_ALGOS) + len(HALO_ALGOS) == ALGO_COUNT and WS_ALGOS and HALO_ALGOS


def halo_accepts(layer):
    return (layer.dtype == "bf16" and layer.groups == 1 and layer.kh == 3 and layer.kw == 3 and layer.sh == layer.sw
            and layer.sh in (1, 2) and layer.cin in (32, 64) and layer.ph <= 2 and layer.pw <= 2
            and layer.cout % 4 == 0)

# Tiles wider than 256 rows on either side need a 16-byte-vector loader; the
# element-wise gather refuses them at prepare time.
BIG_TILES = {a for a in TILE_ALGOS if max(map(int, re.search(r"co(\d+)xpx(\d+)", ALGO_DESC[a]).groups())) > 256}


def forced_tiles(layer):
    """Every forced MFMA tile the layer accepts. Only the generic loader may
    refuse a tile wider than 256; the direct-to-LDS kernel refuses layers
    without 128-byte channel blocks or with Cout not a multiple of its tile;
    the weight-stationary kernel refuses element-wise gathers and reductions
    over 256 bytes."""
    out = []
    for a in TILE_ALGOS + XL_ALGOS + WS_ALGOS + HALO_ALGOS:
        try:
            _lib.Conv2d.from_layer(layer, algo=a).close()
            out.append(a)
        except _lib.ConvError as e:
            assert "CONV_E_UNSUPPORTED" in str(e), (layer.name, a, str(e))
            d = _lib.Conv2d.from_layer(layer).describe()
            cbytes = layer.cin * (2 if layer.dtype == "bf16" else 1)
            if a in BIG_TILES:
                assert "loader=generic" in d or "smallk" in d, (layer.name, a, d)
            elif a in WS_ALGOS:
                assert cbytes % 16 or layer.kh * layer.kw * cbytes > 256 or layer.groups > 1, (layer.name, a, d)
            elif a in HALO_ALGOS:
                assert not halo_accepts(layer), (layer.name, a, d)
            else:
                assert a in XL_ALGOS, (layer.name, a, d)
                tco = int(re.search(r"co(\d+)x", ALGO_DESC[a]).group(1))
                assert cbytes % 128 or layer.cout % tco or layer.kh * layer.kw > 32, (layer.name, a, d)
    return out


def L(name, n, h, w, cin, cout, kh, kw, s=(1, 1), p=(0, 0), groups=1, dtype="bf16", out=None, act="mish"):
    ho, wo = oracle.out_hw(h, w, kh, kw, s[0], s[1], p[0], p[1])
    out = out or dtype
    return Layer(name, n, h, w, cin, cout, kh, kw, s[0], s[1], p[0], p[1], groups, dtype, out, act, ho, wo)


LAW = {"f32": "mnist", "bf16": "bf16", "i8": "int8"}

# Dense layers for the MFMA kernel: every loader (vec16, 1x1, generic), ragged
# pixel counts and channel counts, strides, per-axis padding.
DENSE = [
    L("bf16_3x3_vec", 2, 19, 23, 32, 80, 3, 3, (1, 1), (1, 1)),
    L("bf16_3x3s2_vec", 1, 37, 29, 64, 72, 3, 3, (2, 2), (1, 1), act="relu6"),
    L("bf16_1x1", 2, 17, 13, 64, 136, 1, 1, act="none"),
    L("bf16_1x1_s2", 1, 18, 18, 48, 40, 1, 1, (2, 2), act="relu"),
    L("bf16_stem_c3", 1, 41, 45, 3, 32, 3, 3, (1, 1), (1, 1)),
    L("bf16_c61_cout61", 1, 21, 19, 61, 61, 3, 3, (1, 1), (1, 1)),
    L("bf16_5x3_pad21", 1, 23, 17, 16, 24, 5, 3, (2, 1), (2, 1), act="relu"),
    L("bf16_deepK", 1, 9, 9, 512, 96, 3, 3, (1, 1), (1, 1)),
    L("i8_3x3_vec_i8", 2, 19, 23, 32, 80, 3, 3, (1, 1), (1, 1), dtype="i8", out="i8", act="relu"),
    L("i8_3x3_vec_i32", 1, 21, 17, 64, 72, 3, 3, (2, 2), (1, 1), dtype="i8", out="i32", act="none"),
    L("i8_1x1_i8_mish", 2, 15, 13, 128, 96, 1, 1, dtype="i8", out="i8", act="mish"),
    L("i8_1x1_i32_relu", 1, 16, 16, 64, 64, 1, 1, dtype="i8", out="i32", act="relu"),
    L("i8_stem10x4", 1, 49, 10, 1, 64, 10, 4, (2, 2), (5, 1), dtype="i8", out="i8", act="relu"),
    L("i8_c24_generic", 1, 20, 20, 24, 40, 3, 3, (1, 1), (1, 1), dtype="i8", out="i32", act="none"),
    L("i8_cout61", 1, 19, 21, 32, 61, 3, 3, (1, 1), (1, 1), dtype="i8", out="i8", act="relu6"),
    L("i8_deepK", 1, 8, 8, 512, 64, 3, 3, (1, 1), (1, 1), dtype="i8", out="i32", act="none"),
    # tap loader (Cin * elem_size a multiple of 128 bytes)
    L("bf16_tap_5x3_pad21", 1, 23, 17, 64, 40, 5, 3, (2, 1), (2, 1), act="relu"),
    L("bf16_tap_1x1_s2", 1, 18, 18, 128, 40, 1, 1, (2, 2), act="relu6"),
    L("bf16_tap_pad3", 2, 9, 9, 64, 16, 3, 3, (1, 1), (3, 3)),
    L("i8_tap_3x3_s2_mish", 1, 19, 21, 128, 72, 3, 3, (2, 2), (1, 1), dtype="i8", out="i8", act="mish"),
    L("i8_tap_5x5_i32", 1, 13, 11, 128, 24, 5, 5, (1, 1), (2, 2), dtype="i8", out="i32", act="none"),
    L("i8_vec_7x7_i32", 1, 13, 11, 128, 24, 7, 7, (1, 1), (3, 3), dtype="i8", out="i32", act="none"),
]

# Short-K layers with odd channel counts: the LDS-free small-K kernel (auto).
SMALLK = [
    L("sk_bf16_c3_s1", 1, 41, 45, 3, 32, 3, 3, (1, 1), (1, 1)),
    L("sk_bf16_c3_s2_cout8", 2, 33, 30, 3, 8, 3, 3, (2, 2), (1, 1), act="relu6"),
    L("sk_bf16_c1_5x5_cout70", 1, 20, 17, 1, 70, 5, 5, (1, 2), (2, 1), act="relu"),
    L("sk_bf16_c7_k63", 1, 19, 23, 7, 40, 3, 3, (1, 1), (1, 1), act="none"),
    L("sk_i8_stem10x4", 1, 49, 10, 1, 64, 10, 4, (2, 2), (5, 1), dtype="i8", out="i8", act="relu"),
    L("sk_i8_c3_i32", 2, 15, 17, 3, 24, 3, 3, (1, 1), (1, 1), dtype="i8", out="i32", act="none"),
    L("sk_i8_c8_mish", 1, 21, 19, 8, 130, 3, 3, (2, 1), (0, 1), dtype="i8", out="i8", act="mish"),
    # wide images: several 64-pixel tiles per output row with a ragged last
    # one, image rows whose byte length is not a multiple of 16, stride 2,
    # and a pad wider than the kernel
    L("sk_bf16_w300", 1, 9, 300, 3, 32, 3, 3, (1, 1), (1, 1)),
    L("sk_bf16_w530_s2", 1, 11, 530, 3, 32, 3, 3, (2, 2), (1, 1), act="relu6"),
    L("sk_bf16_w100_n2", 2, 7, 100, 3, 16, 3, 3, (1, 1), (1, 1), act="relu"),
    L("sk_i8_w277_pad4", 1, 6, 277, 3, 48, 3, 3, (1, 1), (4, 4), dtype="i8", out="i8", act="mish"),
    L("sk_bf16_c2_w131_cout20", 1, 5, 131, 2, 20, 3, 5, (1, 2), (1, 2), act="none"),
]


@pytest.mark.parametrize("layer", SMALLK, ids=[l.name for l in SMALLK])
def test_smallk(layer):
    t = random_layer_tensors(layer, LAW[layer.dtype], seed=18)
    y, conv = H.gpu_run(layer, t["x"], t)
    assert "smallk" in conv.describe(), conv.describe()
    H.check_layer_full(layer, t["x"], t, y, "%s [%s]" % (layer.name, conv.describe()))


@pytest.mark.parametrize("layer", DENSE, ids=[l.name for l in DENSE])
def test_dense_all_tiles(layer):
    t = random_layer_tensors(layer, LAW[layer.dtype], seed=11)
    ref = H.oracle_full(layer, t["x"], t)
    xg = t["x"].cuda()
    for algo in [0] + forced_tiles(layer):
        y, conv = H.gpu_run(layer, xg, t, algo=algo)
        what = "%s algo=%d [%s]" % (layer.name, algo, conv.describe())
        yc = y.cpu()
        if layer.dtype == "i8":
            H.check_int(yc.numpy(), ref, layer, what)
        else:
            H.check_float(yc.float().numpy(), ref[0], ref[1], layer.dtype, what)
        conv.close()


# Layers for the large-layer kernel: 128-byte channel blocks, Cout a multiple
# of 128 or 256, one, two and many K-tiles, stride and padding, int8 outputs,
# and a layer small enough to be split along K.
XL = [
    L("xl_bf16_3x3_c64", 1, 19, 23, 64, 256, 3, 3, (1, 1), (1, 1)),
    L("xl_bf16_1x1_nkt1", 2, 15, 17, 64, 128, 1, 1, act="none"),
    L("xl_bf16_1x1_nkt2", 1, 20, 20, 128, 256, 1, 1, act="relu"),
    L("xl_bf16_s2_pad", 1, 33, 31, 128, 256, 3, 3, (2, 2), (1, 1), act="relu6"),
    L("xl_bf16_5x3_pad21", 1, 23, 17, 64, 128, 5, 3, (2, 1), (2, 1), act="relu"),
    L("xl_i8_3x3_mish", 1, 21, 19, 128, 256, 3, 3, (1, 1), (1, 1), dtype="i8", out="i8", act="mish"),
    L("xl_i8_3x3_i32", 2, 11, 13, 256, 128, 3, 3, (1, 1), (1, 1), dtype="i8", out="i32", act="none"),
    L("xl_i8_1x1_relu", 1, 17, 18, 256, 512, 1, 1, dtype="i8", out="i8", act="relu"),
    L("xl_bf16_splitk", 1, 10, 10, 512, 256, 3, 3, (1, 1), (1, 1)),
]


@pytest.mark.parametrize("layer", XL, ids=[l.name for l in XL])
def test_xl_all_tiles(layer):
    t = random_layer_tensors(layer, LAW[layer.dtype], seed=19)
    ref = H.oracle_full(layer, t["x"], t)
    xg = t["x"].cuda()
    algos = [a for a in forced_tiles(layer) if a in XL_ALGOS]
    assert algos, layer.name
    for algo in algos:
        y, conv = H.gpu_run(layer, xg, t, algo=algo)
        what = "%s algo=%d [%s]" % (layer.name, algo, conv.describe())
        assert "igemm_xl" in conv.describe()
        if layer.name.endswith("splitk"):
            assert "ksplit=1 " not in conv.describe(), what
        yc = y.cpu()
        if layer.dtype == "i8":
            H.check_int(yc.numpy(), ref, layer, what)
        else:
            H.check_float(yc.float().numpy(), ref[0], ref[1], layer.dtype, what)
        conv.close()


DW = [
    L("dw_bf16_s1", 2, 17, 19, 64, 64, 3, 3, (1, 1), (1, 1), groups=64, act="relu6"),
    L("dw_bf16_s2", 1, 24, 23, 32, 32, 3, 3, (2, 2), (1, 1), groups=32, act="mish"),
    L("dw_bf16_c12_generic", 1, 13, 11, 12, 12, 3, 3, (1, 1), (1, 1), groups=12, act="none"),
    L("dw_i8_s1", 1, 25, 5, 64, 64, 3, 3, (1, 1), (1, 1), groups=64, dtype="i8", out="i8", act="relu"),
    L("dw_i8_s2_i32", 2, 15, 16, 32, 32, 3, 3, (2, 2), (1, 1), groups=32, dtype="i8", out="i32", act="none"),
    L("dw_i8_c8_generic", 1, 12, 9, 8, 8, 3, 3, (1, 1), (1, 1), groups=8, dtype="i8", out="i8", act="mish"),
    L("dw_f32_c4", 1, 14, 13, 4, 4, 3, 3, (1, 1), (1, 1), groups=4, dtype="f32", act="relu"),
    L("dw_f32_c6_s2", 1, 15, 15, 6, 6, 3, 3, (2, 2), (1, 1), groups=6, dtype="f32", act="mish"),
    L("dw_bf16_pad0", 1, 10, 11, 16, 16, 3, 3, (1, 1), (0, 0), groups=16, act="relu"),
]


@pytest.mark.parametrize("layer", DW, ids=[l.name for l in DW])
def test_depthwise(layer):
    t = random_layer_tensors(layer, LAW[layer.dtype], seed=12)
    y, conv = H.gpu_run(layer, t["x"], t)
    assert "dw3x3" in conv.describe()
    H.check_layer_full(layer, t["x"], t, y, "%s [%s]" % (layer.name, conv.describe()))


# Stride-1 depthwise layers through the row-window kernels with every forced
# rows-per-lane count (algo 1..4 = 1, 2, 4, 8 rows): output heights that no
# row count divides, widths ragged against the lane's 2 (bf16, fp32) or 4
# (int8) columns, both paddings, every int8 output kind.
DW_ROWS = [
    L("dwr_bf16_mish", 2, 19, 21, 32, 32, 3, 3, (1, 1), (1, 1), groups=32, act="mish"),
    L("dwr_bf16_pad0_relu6", 1, 14, 9, 16, 16, 3, 3, (1, 1), (0, 0), groups=16, act="relu6"),
    L("dwr_i8_mish", 2, 19, 18, 64, 64, 3, 3, (1, 1), (1, 1), groups=64, dtype="i8", out="i8", act="mish"),
    L("dwr_i8_relu6", 1, 13, 7, 32, 32, 3, 3, (1, 1), (1, 1), groups=32, dtype="i8", out="i8", act="relu6"),
    L("dwr_i8_i32_relu", 1, 11, 10, 16, 16, 3, 3, (1, 1), (1, 1), groups=16, dtype="i8", out="i32", act="relu"),
    L("dwr_i8_none_pad0", 1, 12, 13, 8, 8, 3, 3, (1, 1), (0, 0), groups=8, dtype="i8", out="i8", act="none"),
    L("dwr_f32_mish", 1, 17, 10, 8, 8, 3, 3, (1, 1), (1, 1), groups=8, dtype="f32", act="mish"),
]


@pytest.mark.parametrize("layer", DW_ROWS, ids=[l.name for l in DW_ROWS])
def test_depthwise_rows_per_lane(layer):
    t = random_layer_tensors(layer, LAW[layer.dtype], seed=14)
    ref = H.oracle_full(layer, t["x"], t)
    xg = t["x"].cuda()
    for algo, th in ((1, 1), (2, 2), (3, 4), (4, 8)):
        y, conv = H.gpu_run(layer, xg, t, algo=algo)
        d = conv.describe()
        what = "%s algo=%d [%s]" % (layer.name, algo, d)
        m = re.search(r"kernel=dw3x3_(rows|i8)_kernel<(.*)>", d)
        assert m, what
        args = [a.strip() for a in m.group(2).split(",")]
        assert int(args[3 if m.group(1) == "rows" else 1]) == th, what
        yc = y.cpu()
        if layer.dtype == "i8":
            H.check_int(yc.numpy(), ref, layer, what)
        else:
            H.check_float(yc.float().numpy(), ref[0], ref[1], layer.dtype, what)
        conv.close()


F32 = [
    L("f32_mnist_like", 1, 28, 28, 1, 8, 3, 3, (1, 1), (1, 1), dtype="f32", act="relu"),
    L("f32_ragged", 2, 11, 9, 5, 7, 3, 2, (2, 1), (1, 0), dtype="f32", act="mish"),
    L("f32_1x1", 1, 7, 7, 16, 10, 1, 1, dtype="f32", act="relu6"),
]


@pytest.mark.parametrize("layer", F32, ids=[l.name for l in F32])
def test_fp32_direct(layer):
    t = random_layer_tensors(layer, "mnist", seed=13)
    y, conv = H.gpu_run(layer, t["x"], t)
    assert "direct_f32" in conv.describe()
    H.check_layer_full(layer, t["x"], t, y, layer.name)


def test_zero_bias_pointer():
    layer = L("nobias", 1, 9, 9, 16, 16, 3, 3, (1, 1), (1, 1), act="none")
    t = random_layer_tensors(layer, "bf16", seed=14)
    conv = _lib.Conv2d.from_layer(layer)
    y = conv.run(t["x"].cuda(), t["w"].cuda(), None)
    r, a = oracle.conv_float(H.to_np_f32(t["x"]), H.to_np_f32(t["w"]), None, (1, 1), (1, 1))
    H.check_float(y.cpu().float().numpy(), r, a, "bf16", "null bias")


# Few output tiles, long reduction: the plan splits K over workgroups and a
# second kernel sums the partials in split order (the allocation-free entry
# keeps them in the static scratch instead: the same bits).
SPLITK = [
    L("splitk_bf16_mish", 1, 20, 20, 512, 1024, 3, 3, (2, 2), (1, 1)),
    L("splitk_bf16_1x1", 1, 12, 12, 2048, 96, 1, 1, act="relu"),
    L("splitk_i8_i8", 2, 10, 10, 256, 72, 3, 3, (1, 1), (1, 1), dtype="i8", out="i8", act="relu6"),
    L("splitk_i8_i32", 1, 9, 9, 512, 64, 3, 3, (1, 1), (1, 1), dtype="i8", out="i32", act="relu"),
    L("splitk_i8_mish_vec", 1, 11, 13, 96, 40, 5, 5, (1, 1), (2, 2), dtype="i8", out="i8", act="mish"),
]


@pytest.mark.parametrize("layer", SPLITK, ids=[l.name for l in SPLITK])
def test_split_k(layer):
    t = random_layer_tensors(layer, LAW[layer.dtype], seed=19)
    ref = H.oracle_full(layer, t["x"], t)
    conv = _lib.Conv2d.from_layer(layer)
    desc = conv.describe()
    assert "ksplit=1 " not in desc, desc
    x, w, b = t["x"].cuda(), t["w"].cuda(), H.bias_arg(layer, t)
    ys = []
    for _ in range(2):
        y = conv.empty_output()
        y.fill_(float("nan") if y.dtype.is_floating_point else -77)
        conv.run(x, w, b, y)
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0].view(torch.uint8), ys[1].view(torch.uint8)), "split-K run-to-run difference"
    # many launches back to back on the one workspace
    yb = conv.empty_output()
    for _ in range(20):
        conv.run(x, w, b, yb)
    yn = conv.empty_output()
    yn.fill_(float("nan") if yn.dtype.is_floating_point else -77)
    conv.run_noalloc(x, w, b, yn)
    torch.cuda.synchronize()
    assert torch.equal(yb.view(torch.uint8), ys[0].view(torch.uint8)), "split-K after 20 launches"
    assert torch.equal(yn.view(torch.uint8), ys[0].view(torch.uint8)), "plan workspace vs static scratch"
    what = "%s [%s]" % (layer.name, desc)
    if layer.dtype == "i8":
        H.check_int(ys[0].cpu().numpy(), ref, layer, what)
    else:
        H.check_float(ys[0].cpu().float().numpy(), ref[0], ref[1], layer.dtype, what)
    # graph replays reuse the plan's workspace
    g = torch.cuda.CUDAGraph()
    yg = conv.empty_output()
    with torch.cuda.graph(g):
        conv.run(x, w, b, yg)
    for _ in range(3):
        yg.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg.view(torch.uint8), ys[0].view(torch.uint8)), "graph replay differs"


# ------------------------------------------------------------------ mosaic

@pytest.mark.parametrize("th,tw,c,c_pad,in_dt,out_dt", [
    (320, 320, 3, 3, torch.float32, torch.bfloat16),   # the 640x640 workload (vector path)
    (320, 320, 3, 4, torch.float32, torch.bfloat16),   # channel padding (pixel path)
    (7, 5, 3, 3, torch.float32, torch.float32),        # odd sizes
    (16, 8, 4, 8, torch.bfloat16, torch.bfloat16),
])
def test_mosaic_bit_exact(th, tw, c, c_pad, in_dt, out_dt):
    g = np.random.default_rng(15)
    tiles32 = g.random((8, th, tw, c)).astype(np.float32) * 3 - 1
    tiles = torch.from_numpy(tiles32).to(in_dt)
    can = _lib.mosaic_pack(tiles.cuda(), c_pad=c_pad, out_dtype=out_dt).cpu()
    ref = oracle.mosaic(tiles.float().numpy(), c_pad=c_pad, out="bf16" if out_dt == torch.bfloat16 else "f32")
    got = can.view(torch.int16).numpy().view(np.uint16) if out_dt == torch.bfloat16 else can.numpy()
    assert np.array_equal(got, ref)


# ----------------------------------------------------------------- hygiene

def _guarded_run(layer, t, algo=0):
    """Output placed in the middle of a larger buffer whose margins hold a
    pattern that must survive the run."""
    conv = _lib.Conv2d.from_layer(layer, algo=algo)
    dt = _lib.TORCH_DT[layer.out]
    numel = int(np.prod(conv.out_shape))
    esz = torch.tensor([], dtype=dt).element_size()
    guard = 4096 // esz
    buf = torch.empty(numel + 2 * guard, dtype=dt, device="cuda")
    if dt.is_floating_point:
        buf.fill_(-4096.0)
    else:
        buf.fill_(-99)
    y = buf[guard:guard + numel].view(conv.out_shape)
    conv.run(t["x"].cuda(), t["w"].cuda(), H.bias_arg(layer, t), y)
    torch.cuda.synchronize()
    head, tail = buf[:guard], buf[guard + numel:]
    fill = -4096.0 if dt.is_floating_point else -99
    assert torch.all(head == fill) and torch.all(tail == fill), "write outside y"
    return y


@pytest.mark.parametrize("layer", [DENSE[0], DENSE[5], DENSE[8], DENSE[14], DW[0], DW[3], F32[1], SMALLK[2],
                                   SMALLK[6], XL[0], XL[8]],
                         ids=lambda l: l.name)
def test_guard_bands_and_determinism(layer):
    t = random_layer_tensors(layer, LAW[layer.dtype], seed=16)
    algos = [0] + (forced_tiles(layer) if layer.groups == 1 and layer.dtype != "f32" else [])
    for algo in algos:
        y1 = _guarded_run(layer, t, algo).clone()
        y2 = _guarded_run(layer, t, algo)
        assert torch.equal(y1.cpu().view(torch.uint8), y2.cpu().view(torch.uint8)), "run-to-run difference"
        if algo == 0:
            H.check_layer_full(layer, t["x"], t, y2, "%s guarded" % layer.name)


def test_side_stream_and_graph_replay():
    layer = DENSE[0]
    t = random_layer_tensors(layer, "bf16", seed=17)
    ref = H.oracle_full(layer, t["x"], t)
    conv = _lib.Conv2d.from_layer(layer)
    x, w, b = t["x"].cuda(), t["w"].cuda(), H.bias_arg(layer, t)
    y = conv.empty_output()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y.fill_(float("nan"))
        conv.run(x, w, b, y)
    s.synchronize()
    H.check_float(y.cpu().float().numpy(), ref[0], ref[1], "bf16", "side stream")
    # capture into a graph, replay several times with eager work between
    g = torch.cuda.CUDAGraph()
    yg = conv.empty_output()
    with torch.cuda.graph(g):
        conv.run(x, w, b, yg)
    for i in range(4):
        yg.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        H.check_float(yg.cpu().float().numpy(), ref[0], ref[1], "bf16", "graph replay %d" % i)
        _ = (x.float() * 2).sum().item()  # unrelated eager work between replays


# SPP max-pool block against the oracle, bit for bit (values: the oracle keeps
# the first of equal values, the kernel the larger key, which differ only for
# -0 against +0): the 320- and 640-input maps of YOLOv4's SPP, maps smaller
# than the windows, a single pixel, odd sizes, all three dtypes, and the
# chunk counts per workgroup that batch and channel count select.
SPP = [
    ((1, 10, 10, 512), "bf16"), ((1, 20, 20, 512), "bf16"), ((16, 20, 20, 512), "bf16"),
    ((2, 13, 7, 24), "bf16"), ((1, 1, 1, 8), "bf16"), ((3, 3, 5, 16), "i8"), ((1, 19, 19, 256), "i8"),
    ((2, 9, 14, 12), "f32"), ((1, 45, 45, 8), "bf16"), ((4, 6, 40, 64), "f32"),
]


def _spp_input(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    if dtype == "i8":
        return torch.randint(-127, 128, shape, generator=g, dtype=torch.int8)
    x = torch.randn(shape, generator=g) * 0.5
    return x.to(torch.bfloat16) if dtype == "bf16" else x


@pytest.mark.parametrize("shape,dtype", SPP, ids=["%s_%s" % ("x".join(map(str, s)), d) for s, d in SPP])
def test_spp_maxpool(shape, dtype):
    x = _spp_input(shape, dtype, seed=31)
    xn = x.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else x.numpy()
    ref = oracle.spp(xn)
    y = _lib.spp_maxpool(x.cuda())
    torch.cuda.synchronize()
    yc = y.cpu()
    yn = yc.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else yc.numpy()
    if dtype == "bf16":
        yv = (yn.astype(np.uint32) << 16).view(np.float32)
        rv = (ref.astype(np.uint32) << 16).view(np.float32)
        assert np.array_equal(yv, rv), "values differ"
        same_bits = yn == ref
        assert np.all(same_bits | (yv == 0)), "bits differ on a nonzero value"
    else:
        assert np.array_equal(yn, ref)


# Upsample x2 + concat against the oracle, byte for byte: YOLOv4's two neck
# joins at 640 input (20x20x256 upsampled beside a 40x40x256 lateral map,
# 40x40x128 beside 80x80x128) in both channel orders, both or neither source
# upsampled, every dtype, odd chunk counts per pixel.
UPCAT = [
    ((1, 20, 20, 256), 1, (1, 40, 40, 256), 0, "bf16"), ((1, 80, 80, 128), 0, (1, 40, 40, 128), 1, "bf16"),
    ((2, 5, 7, 24), 1, (2, 10, 14, 8), 0, "bf16"), ((3, 4, 6, 16), 0, (3, 4, 6, 48), 0, "i8"),
    ((1, 3, 3, 32), 1, (1, 3, 3, 16), 1, "i8"), ((2, 6, 5, 12), 1, (2, 12, 10, 4), 0, "f32"),
    ((16, 20, 20, 256), 1, (16, 40, 40, 256), 0, "bf16"),
]


@pytest.mark.parametrize("a_shape,up0,b_shape,up1,dtype", UPCAT,
                         ids=["%s_up%d_%s_up%d_%s" % ("x".join(map(str, a)), u0, "x".join(map(str, b)), u1, d)
                              for a, u0, b, u1, d in UPCAT])
def test_upsample_concat(a_shape, up0, b_shape, up1, dtype):
    a = _spp_input(a_shape, dtype, seed=41)
    b = _spp_input(b_shape, dtype, seed=42)
    to_np = (lambda t: t.view(torch.int16).numpy()) if dtype == "bf16" else (lambda t: t.numpy())
    ref = oracle.upcat(to_np(a), up0, to_np(b), up1)
    y = _lib.upsample_concat(a.cuda(), up0, b.cuda(), up1)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(y.cpu()), ref)


# Residual-add epilogue (conv_run_residual): y = act(conv + b) + r written
# once, against the oracle's unrounded activation plus r, on every kernel
# path: implicit GEMM (tap, vec16 and element-wise loaders, Cout not a
# multiple of 4), the large-layer kernel, the small-K stem kernel, the halo-
# persistent kernel, split K, the fp32 direct kernel and the three depthwise
# kernels; in place (r is y) for a bf16 and an int8 layer.
RES = [
    L("res_bf16_tap", 1, 12, 13, 64, 64, 3, 3, (1, 1), (1, 1), act="mish"),
    L("res_bf16_xl", 1, 11, 9, 128, 256, 3, 3, (1, 1), (1, 1), act="mish"),
    L("res_bf16_vec", 1, 9, 10, 32, 48, 3, 3, (2, 2), (1, 1), act="relu6"),
    L("res_bf16_cout6", 1, 9, 8, 24, 6, 3, 3, (1, 1), (1, 1), act="relu"),
    L("res_bf16_stem", 1, 17, 15, 3, 32, 3, 3, (1, 1), (1, 1), act="mish"),
    L("res_bf16_xl_c128", 1, 14, 12, 64, 128, 3, 3, (1, 1), (1, 1), act="none"),
    L("res_i8_xl_splitk", 1, 9, 9, 512, 256, 3, 3, (1, 1), (1, 1), dtype="i8", out="i8", act="relu"),
    L("res_bf16_splitk", 1, 10, 10, 512, 256, 3, 3, (1, 1), (1, 1), act="mish"),
    L("res_i8_tap", 1, 12, 11, 128, 64, 3, 3, (1, 1), (1, 1), dtype="i8", out="i8", act="mish"),
    L("res_i8_xl", 1, 13, 9, 128, 256, 3, 3, (1, 1), (1, 1), dtype="i8", out="i8", act="relu6"),
    L("res_i8_cout5", 1, 7, 9, 16, 5, 3, 3, (1, 1), (1, 1), dtype="i8", out="i8", act="none"),
    L("res_f32", 1, 10, 10, 4, 8, 3, 3, (1, 1), (1, 1), dtype="f32", act="relu"),
    L("res_dw_bf16", 2, 11, 13, 32, 32, 3, 3, (1, 1), (1, 1), groups=32, act="relu6"),
    L("res_dw_bf16_s2", 1, 12, 11, 32, 32, 3, 3, (2, 2), (1, 1), groups=32, act="mish"),
    L("res_dw_i8", 1, 9, 10, 64, 64, 3, 3, (1, 1), (1, 1), groups=64, dtype="i8", out="i8", act="mish"),
    L("res_dw_i8_s2", 1, 12, 12, 32, 32, 3, 3, (2, 2), (1, 1), groups=32, dtype="i8", out="i8", act="relu"),
    L("res_dw_f32", 1, 9, 9, 8, 8, 3, 3, (1, 1), (1, 1), groups=8, dtype="f32", act="mish"),
]
RES_KERNEL = {"res_bf16_xl": "igemm_xl", "res_i8_xl": "igemm_xl", "res_bf16_xl_c128": "igemm_xl",
              "res_i8_xl_splitk": "ksplit=",
              "res_bf16_stem": "smallk", "res_bf16_splitk": "ksplit=", "res_dw_bf16": "dw3x3_rows_kernel",
              "res_dw_bf16_s2": "dw3x3_kernel", "res_dw_i8": "dw3x3_i8_kernel", "res_dw_i8_s2": "dw3x3_kernel",
              "res_f32": "direct_f32"}


def _residual(layer, shape, seed):
    g = torch.Generator().manual_seed(seed)
    if layer.dtype == "i8":
        return torch.randint(-127, 128, shape, generator=g, dtype=torch.int8)
    r = torch.randn(shape, generator=g)
    return r.to(torch.bfloat16) if layer.dtype == "bf16" else r


@pytest.mark.parametrize("layer", RES, ids=[l.name for l in RES])
def test_residual_epilogue(layer):
    t = random_layer_tensors(layer, LAW[layer.dtype], seed=23)
    ref = H.oracle_full(layer, t["x"], t)
    algo = 0
    if layer.name.endswith("_xl"):
        algo = next(a for a in forced_tiles(layer) if a in XL_ALGOS)
    elif "_xl_c128" in layer.name or "_xl_splitk" in layer.name:
        algo = next(a for a in forced_tiles(layer) if a in XL_ALGOS)
    conv = _lib.Conv2d.from_layer(layer, algo=algo)
    d = conv.describe()
    want = RES_KERNEL.get(layer.name)
    assert want is None or want in d, (layer.name, d)
    if layer.name.endswith("splitk"):
        assert "ksplit=1 " not in d, d
    w = t["w"].cuda()
    b = (_lib.pack_bias_scale(t["b"], t.get("s")) if layer.dtype == "i8" else t["b"]).cuda()
    res = _residual(layer, conv.out_shape, seed=24)
    for inplace in ((False, True) if layer.name in ("res_bf16_tap", "res_i8_tap") else (False,)):
        rg = res.cuda()
        y = rg if inplace else conv.empty_output()
        conv.run(t["x"].cuda(), w, b, y, residual=rg)
        torch.cuda.synchronize()
        what = "%s inplace=%s [%s]" % (layer.name, inplace, d)
        yc = y.cpu()
        if layer.dtype == "i8":
            q, m = oracle.add_residual_i8(ref[1], res.numpy())
            H.check_int(yc.numpy(), (q, m), layer, what)
        else:
            rv = res.float().numpy()
            r, a = oracle.add_residual_float(ref[0], ref[1], rv)
            H.check_float(yc.float().numpy(), r, a, layer.dtype, what)
    conv.close()
