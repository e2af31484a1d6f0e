"""The window stem kernel (3x3 stride-1 bf16 first layer on inputs padded to
8 channels per pixel) against the oracle, and the mosaic packer's padded
canvas.

The input handed to the kernel is the dense NHWC tensor with channels c_in
.. 7 of every pixel filled with NaN: the kernel must ignore them (a NaN that
reached a sum would show up as a non-finite output). The oracle runs the
dense layer; every output is compared under the bf16 rule. Cases: 1, 3, 5 and
8 input channels, ragged patch rows and columns, several images, a partial
32-channel tile, pad 0 and 1, every activation, a residual, more patches than the
persistent grid holds (a workgroup walks two); the 640x640x3 -> 32 stem of
the YOLO stack at full size on sampled outputs (plus one full band of rows
element by element).
"""
import numpy as np
import pytest
import torch

from convolution_conv2d_nhwc_amd import _lib
from convolution_conv2d_nhwc_amd.data import Layer, layer_params, random_layer_tensors, workload
from oracle import oracle
from tests import helpers as H

pytestmark = pytest.mark.gpu


def L(name, n, h, w, cin, cout, p=1, act="mish"):
    ho, wo = oracle.out_hw(h, w, 3, 3, 1, 1, p, p)
    return Layer(name, n, h, w, cin, cout, 3, 3, 1, 1, p, p, 1, "bf16", "bf16", act, ho, wo)


def padded(x: torch.Tensor) -> torch.Tensor:
    n, h, w, c = x.shape
    xp = torch.full((n, h, w, 8), float("nan"), dtype=torch.bfloat16)
    xp[..., :c] = x
    return xp


def run_stem(layer, t, residual=None):
    conv = _lib.Conv2d.from_layer(layer, x_stride=8)
    d = conv.describe()
    assert d.startswith("stem_window "), d
    y = conv.empty_output()
    y.fill_(float("nan"))
    conv.run(padded(t["x"]).cuda(), t["w"].cuda(), t["b"].cuda(), y,
             residual=None if residual is None else residual.cuda())
    torch.cuda.synchronize()
    conv.close()
    return y.cpu(), d


CASES = [
    L("st_c3_ragged", 1, 37, 150, 3, 32),
    L("st_c3_n2_cout48", 2, 9, 70, 3, 48, act="relu"),
    L("st_c8", 1, 20, 64, 8, 32, act="none"),
    L("st_c1_pad0_cout64", 1, 16, 33, 1, 64, p=0, act="relu6"),
    L("st_c5_n3", 3, 5, 17, 5, 32),
]


@pytest.mark.parametrize("layer", CASES, ids=[c.name for c in CASES])
def test_stem_vs_oracle(layer):
    print("stem", layer.name, flush=True)
    t = random_layer_tensors(layer, "bf16", seed=81)
    y, d = run_stem(layer, t)
    H.check_layer_full(layer, t["x"], t, y, "%s [%s]" % (layer.name, d))


def test_stem_residual():
    layer = L("st_res", 1, 12, 40, 3, 32)
    t = random_layer_tensors(layer, "bf16", seed=82)
    r = (0.5 * torch.randn((1, 12, 40, 32), generator=torch.Generator().manual_seed(83))).to(torch.bfloat16)
    y, d = run_stem(layer, t, residual=r)
    rr, a = H.oracle_full(layer, t["x"], t)
    want, asum = oracle.add_residual_float(rr, a, r.float().numpy().astype(np.float64))
    H.check_float(y.float().numpy(), want, asum, "bf16", "stem residual [%s]" % d)


def test_mosaic_padded_canvas_bit_exact():
    g = np.random.default_rng(84)
    tiles = torch.from_numpy(g.standard_normal((8, 17, 23, 3)).astype(np.float32))
    can = _lib.mosaic_pack(tiles.cuda(), c_pad=8, out_dtype=torch.bfloat16).cpu()
    bits = can.view(torch.int16).numpy().view(np.uint16)
    ref = oracle.mosaic(tiles.numpy(), out="bf16")
    assert np.array_equal(bits[..., :3], ref)
    assert not np.any(bits[..., 3:])


def test_stem_yolo640_full_size():
    wl = workload("yolo640_bf16")
    layer = wl.layers[0]
    t = dict(layer_params(wl, 0))
    t["x"] = (torch.rand((1, 640, 640, 3), generator=torch.Generator().manual_seed(85))).to(torch.bfloat16)
    print("stem full size", layer.name, flush=True)
    y, d = run_stem(layer, t)
    H.check_layer_sampled(layer, t["x"], t, y, count=3000, what="%s [%s]" % (layer.name, d))
    # a band of 6 output rows, every element: the rows' inputs and outputs
    band = Layer(layer.name + "_band", 1, 8, 640, 3, 32, 3, 3, 1, 1, 1, 1, 1, "bf16", "bf16", layer.act, 8, 640)
    xb = t["x"][:, 300:308].contiguous()
    rb, ab = H.oracle_full(band, xb, t)
    # output rows 301..306 depend only on input rows 300..307
    H.check_float(y[:, 301:307].float().numpy(), rb[:, 1:7], ab[:, 1:7], "bf16", "stem band rows 301-306")


def test_stem_several_patches_per_workgroup():
    """More patches than the persistent grid holds (two workgroups per CU),
    with ragged patch rows and columns: workgroups walk two patches, the
    second window copied during the first patch; every output against the
    oracle, and the folded-mosaic form of the same layer bit-equal to it."""
    layer = L("st_multi_ragged", 1, 130, 1000, 3, 32)
    t = random_layer_tensors(layer, "bf16", seed=89)
    print("stem", layer.name, flush=True)
    y, d = run_stem(layer, t)
    H.check_layer_full(layer, t["x"], t, y, "%s [%s]" % (layer.name, d))
    # the same canvas as four 65 x 500 bf16 tiles
    x = t["x"][0]
    tiles = torch.stack([x[:65, :500], x[:65, 500:], x[65:, :500], x[65:, 500:]]).contiguous()
    conv = _lib.Conv2d.from_layer(layer, x_stride=8)
    ym = _lib.run_mosaic(conv, tiles.cuda(), t["w"].cuda(), t["b"].cuda())
    torch.cuda.synchronize()
    conv.close()
    assert torch.equal(ym.cpu().view(torch.int16), y.view(torch.int16)), "folded mosaic vs padded canvas"


def _mosaic_layer(name, m, th, tw, c, cout, act):
    return L(name, m, 2 * th, 2 * tw, c, cout, act=act)


@pytest.mark.parametrize("tdt", ["f32", "bf16"])
def test_mosaic_folded_vs_oracle_and_packed(tdt):
    """conv_run_mosaic on four tiles per canvas: against the oracle's
    mosaic + convolution, and bit-equal to packing the canvas first."""
    layer = _mosaic_layer("mos_" + tdt, 2, 13, 37, 3, 48, "mish")
    g = np.random.default_rng(86)
    tiles = torch.from_numpy(g.random((8, 13, 37, 3)).astype(np.float32))
    if tdt == "bf16":
        tiles = tiles.to(torch.bfloat16)
    t = random_layer_tensors(layer, "bf16", seed=87)
    conv = _lib.Conv2d.from_layer(layer, x_stride=8)
    tg, wg, bg = tiles.cuda(), t["w"].cuda(), t["b"].cuda()
    y = conv.empty_output()
    y.fill_(float("nan"))
    _lib.run_mosaic(conv, tg, wg, bg, y)
    can = _lib.mosaic_pack(tg, c_pad=8, out_dtype=torch.bfloat16)
    y2 = conv.run(can, wg, bg)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu().view(torch.int16), y2.cpu().view(torch.int16)), "folded vs packed"
    if tdt == "f32":
        bits = oracle.mosaic(tiles.numpy(), out="bf16")
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    else:
        # bf16 tiles are copied as they are: the canvas is the tiles placed 2x2
        x = torch.cat([torch.cat([tiles[0::4], tiles[1::4]], 2), torch.cat([tiles[2::4], tiles[3::4]], 2)], 1)
    H.check_layer_full(layer, x, t, y.cpu(), "%s [%s]" % (layer.name, conv.describe()))
    conv.close()


def test_mosaic_folded_yolo640_bit_equal_to_packed():
    wl = workload("yolo640_bf16")
    layer = wl.layers[0]
    p = layer_params(wl, 0)
    tiles = (torch.rand((4, 320, 320, 3), generator=torch.Generator().manual_seed(88))).cuda()
    conv = _lib.Conv2d.from_layer(layer, x_stride=8)
    w, b = p["w"].cuda(), p["b"].cuda()
    y = _lib.run_mosaic(conv, tiles, w, b)
    y2 = conv.run(_lib.mosaic_pack(tiles, c_pad=8, out_dtype=torch.bfloat16), w, b)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    conv.close()
