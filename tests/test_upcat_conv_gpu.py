"""The YOLOv4 neck join read straight by the 1x1 convolution after it
(conv_run_upcat) against the oracle chain (upsample x2 + concat, then the
convolution) and against the two-step path on the GPU (conv_upsample_concat,
then conv_run with the same plan).

* The 640x640 network's joins: a 20x20x256 map upsampled beside a 40x40x256
  lateral map into a 1x1 512 -> 256 layer, and the 40x40x128 / 80x80x128
  join into 256 -> 128; bf16 with Mish on the 64x64 implicit-GEMM tile
  (forced, unsplit: bit-equal to the two-step path) and with the automatic
  plan (against the oracle).
* The upsampled map second, two images, a ragged pixel count, ReLU.
* int8 with requantised int8 output (exact integer sums: bit-equal to the
  two-step path whatever the plan, and to the oracle under the int8 rule).
"""
import numpy as np
import pytest
import torch

from convolution_conv2d_nhwc_amd import _lib
from convolution_conv2d_nhwc_amd.data import Layer, random_layer_tensors
from oracle import oracle
from tests import helpers as H

pytestmark = pytest.mark.gpu


def layer(name, n, h, w, c0, c1, cout, dtype="bf16", out=None, act="mish"):
    return Layer(name, n, h, w, c0 + c1, cout, 1, 1, 1, 1, 0, 0, 1, dtype, out or dtype, act, h, w)


def maps(lay, c0, up0, up1, seed):
    g = torch.Generator().manual_seed(seed)
    n, h, w = lay.n, lay.h, lay.w
    shapes = [(n, h >> up0, w >> up0, c0), (n, h >> up1, w >> up1, lay.cin - c0)]
    if lay.dtype == "i8":
        return [torch.randint(-127, 128, s, generator=g, dtype=torch.int8) for s in shapes]
    return [(0.5 * torch.randn(s, generator=g)).to(torch.bfloat16) for s in shapes]


def two_step_and_fused(lay, c0, up0, up1, seed, algo=0):
    s0, s1 = maps(lay, c0, up0, up1, seed)
    t = random_layer_tensors(lay, "int8" if lay.dtype == "i8" else "bf16", seed=seed + 1)
    conv = _lib.Conv2d.from_layer(lay, algo=algo)
    d = conv.describe()
    s0g, s1g, w, b = s0.cuda(), s1.cuda(), t["w"].cuda(), H.bias_arg(lay, t)
    x = _lib.upsample_concat(s0g, up0, s1g, up1)
    y2 = conv.run(x, w, b)
    yf = conv.empty_output()
    yf.fill_(float("nan") if yf.dtype.is_floating_point else -77)
    _lib.run_upcat(conv, s0g, up0, s1g, up1, w, b, yf)
    torch.cuda.synchronize()
    conv.close()
    to_np = (lambda u: u.view(torch.int16).numpy()) if lay.dtype == "bf16" else (lambda u: u.numpy())
    xc = oracle.upcat(to_np(s0), up0, to_np(s1), up1)
    return xc, t, y2.cpu(), yf.cpu(), d


def same_bits(a, b, what):
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), what


CASES = [
    # name, n, h, w, c0, c1, cout, up0, up1, act
    ("yolo640_join_40", 1, 40, 40, 256, 256, 256, 1, 0, "mish"),
    ("yolo640_join_80", 1, 80, 80, 128, 128, 128, 1, 0, "mish"),
    ("second_up_n2_ragged", 2, 18, 26, 64, 128, 96, 0, 1, "relu"),
    # a 256-byte reduction: the automatic plan is the weight-stationary
    # kernel, so the join runs on the 64x64 tile
    ("ws_plan_join", 1, 32, 34, 64, 64, 64, 1, 0, "relu6"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_upcat_conv_bf16(case):
    name, n, h, w, c0, c1, cout, up0, up1, act = case
    lay = layer(name, n, h, w, c0, c1, cout, act=act)
    print("upcat conv", name, flush=True)
    # the 64x64 tile, unsplit on these sizes: the fused read is the two-step path bit for bit
    xc, t, y2, yf, d = two_step_and_fused(lay, c0, up0, up1, seed=91, algo=1)
    assert "ksplit=1 " in d, d
    same_bits(yf, y2, "%s fused vs two-step [%s]" % (name, d))
    xt = torch.from_numpy(xc.view(np.int16)).view(torch.bfloat16)
    H.check_layer_full(lay, xt, t, yf, "%s [%s]" % (name, d))
    # the automatic plan (any kernel for the two-step path; the fused read on
    # its implicit-GEMM tile, or the 64x64 tile)
    xc, t, y2, yf, d = two_step_and_fused(lay, c0, up0, up1, seed=92)
    if name == "ws_plan_join":
        assert d.startswith("igemm_ws "), d
    xt = torch.from_numpy(xc.view(np.int16)).view(torch.bfloat16)
    H.check_layer_full(lay, xt, t, yf, "%s auto [%s]" % (name, d))


def test_upcat_conv_int8():
    lay = layer("i8_join", 1, 40, 40, 256, 128, 128, dtype="i8", out="i8", act="relu")
    print("upcat conv int8", flush=True)
    xc, t, y2, yf, d = two_step_and_fused(lay, 256, 1, 0, seed=93)
    same_bits(yf, y2, "int8 fused vs two-step [%s]" % d)
    H.check_layer_full(lay, torch.from_numpy(xc), t, yf, "int8 join [%s]" % d)
