"""The halo kernel (3x3 bf16 layers over 32 or 64 input channels, stride 1
or 2; forced with the last algo id) against the oracle and the
implicit-GEMM kernel.

* Each case runs the layer on the halo kernel and on the 64x64 implicit-GEMM
  tile: both sum each output's products in the same order (tap by tap, 32
  channels per MFMA step) with the same epilogue, so they must agree bit for
  bit; the halo output is also checked against the oracle's fp64 result
  under the bf16 rule (every element). Cases: both strides and channel
  counts, ragged patch rows and columns, several images, two channel tiles
  with a partial one, pad 0 and 2, a residual, no bias, every activation,
  more patches than workgroups with some workgroups left without a patch.
* The 320x320x64 -> 64 layer of the 640x640 stack at full size (bit-equal to
  the implicit-GEMM kernel, plus sampled outputs against the oracle) and its
  160x160x64 -> 256 stride-2 layer.
* Fused 1x1 pairs through the halo kernel (the first layer forced onto it):
  bit-equal to the two layers run separately and to the implicit-GEMM fused
  launch, and against the oracle chain.
"""
import numpy as np
import pytest
import torch

from convolution_conv2d_nhwc_amd import _lib
from convolution_conv2d_nhwc_amd.data import Layer, layer_params, random_layer_tensors, workload
from oracle import oracle
from tests import helpers as H

pytestmark = pytest.mark.gpu

HALO = _lib.lib().conv_algo_count()


def L(name, n, h, w, cin, cout, s=1, p=1, act="mish"):
    ho, wo = oracle.out_hw(h, w, 3, 3, s, s, p, p)
    return Layer(name, n, h, w, cin, cout, 3, 3, s, s, p, p, 1, "bf16", "bf16", act, ho, wo)


def run(layer, t, algo, bias=True, residual=None):
    conv = _lib.Conv2d.from_layer(layer, algo=algo)
    y = conv.empty_output()
    y.fill_(float("nan"))
    conv.run(t["x"].cuda(), t["w"].cuda(), t["b"].cuda() if bias else None, y,
             residual=None if residual is None else residual.cuda())
    torch.cuda.synchronize()
    d = conv.describe()
    conv.close()
    return y.cpu(), d


def same_bits(a, b, what):
    x, y = a.view(torch.int16).reshape(-1).numpy(), b.view(torch.int16).reshape(-1).numpy()
    bad = np.nonzero(x != y)[0]
    assert bad.size == 0, "%s: %d of %d differ, first at %s: %s vs %s" % (
        what, bad.size, x.size, bad[:6], a.reshape(-1)[bad[:6]].tolist(), b.reshape(-1)[bad[:6]].tolist())


CASES = [
    L("h_s1_c64_ragged", 1, 19, 37, 64, 64),
    L("h_s1_c32_n2_cout128", 2, 13, 20, 32, 128, act="relu"),
    L("h_s2_c64_cout72", 1, 21, 34, 64, 72, s=2, act="relu6"),
    L("h_s2_c32_wide", 1, 10, 70, 32, 64, s=2, act="none"),
    L("h_s1_pad0", 1, 18, 18, 64, 64, p=0),
    L("h_s1_pad2_c32", 2, 9, 17, 32, 40, p=2, act="relu"),
    L("h_s2_pad0_n3", 3, 12, 15, 64, 64, s=2, p=0),
    # 513 patches for 512 workgroups: the last XCD's range is shorter than
    # its workgroup count, so some workgroups get no patch
    L("h_s1_xcd_ranges_empty", 1, 36, 912, 64, 64, act="relu"),
]


@pytest.mark.parametrize("layer", CASES, ids=[c.name for c in CASES])
def test_halo_vs_oracle_and_igemm(layer):
    print("halo", layer.name, flush=True)
    t = random_layer_tensors(layer, "bf16", seed=71)
    yh, dh = run(layer, t, HALO)
    assert dh.startswith("halo "), dh
    yi, di = run(layer, t, 1)
    same_bits(yh, yi, "%s [%s] vs [%s]" % (layer.name, dh, di))
    H.check_layer_full(layer, t["x"], t, yh, "%s [%s]" % (layer.name, dh))


def test_halo_residual_and_no_bias():
    layer = L("h_res", 1, 14, 21, 64, 64)
    t = random_layer_tensors(layer, "bf16", seed=72)
    r = (0.5 * torch.randn((1, 14, 21, 64), generator=torch.Generator().manual_seed(73))).to(torch.bfloat16)
    yh, dh = run(layer, t, HALO, residual=r)
    yi, _ = run(layer, t, 1, residual=r)
    same_bits(yh, yi, "residual [%s]" % dh)
    rr, a = H.oracle_full(layer, t["x"], t)
    want, asum = oracle.add_residual_float(rr, a, r.float().numpy().astype(np.float64))
    H.check_float(yh.float().numpy(), want, asum, "bf16", "halo residual")
    yh, _ = run(layer, t, HALO, bias=False)
    yi, _ = run(layer, t, 1, bias=False)
    same_bits(yh, yi, "no bias")


@pytest.mark.parametrize("idx", [3, 6])
def test_halo_yolo640_layers_full_size(idx):
    """L4 (320x320x64 -> 64, stride 1) and L7 (160x160x64 -> 256, stride 2)."""
    wl = workload("yolo640_bf16")
    layer = wl.layers[idx]
    t = dict(layer_params(wl, idx))
    t["x"] = torch.randn((layer.n, layer.h, layer.w, layer.cin),
                         generator=torch.Generator().manual_seed(74)).to(torch.bfloat16)
    print("halo full size", layer.name, flush=True)
    yh, dh = run(layer, t, HALO)
    yi, di = run(layer, t, 1)
    same_bits(yh, yi, "%s [%s]" % (layer.name, dh))
    H.check_layer_sampled(layer, t["x"], t, yh, count=2000, what="%s [%s]" % (layer.name, dh))


def pair(name, n, h, w, cin, cmid, cout, s=1, act1="mish", act2="mish"):
    a = L(name + "_a", n, h, w, cin, cmid, s=s, act=act1)
    b = Layer(name + "_b", n, a.ho, a.wo, cmid, cout, 1, 1, 1, 1, 0, 0, 1, "bf16", "bf16", act2, a.ho, a.wo)
    return a, b


PAIRS = [
    pair("hf_s1_c64_64to32", 1, 17, 35, 64, 64, 32),
    pair("hf_s2_c32_64to64", 2, 19, 36, 32, 64, 64, s=2, act1="relu", act2="relu6"),
    pair("hf_s2_c64_128to64", 1, 21, 33, 64, 128, 64, s=2),
    pair("hf_s1_c32_128to60", 1, 9, 20, 32, 128, 60, act1="none", act2="relu"),
    # 261 patches for 256 workgroups (one per CU with 128 channels): empty
    # XCD ranges in the fused launch
    pair("hf_s1_c64_128to64_xcd", 1, 36, 464, 64, 128, 64),
]


def fused_runs(a, b, ta, tb):
    """(separate, halo fused, implicit-GEMM fused, description)."""
    ch, c1, c2 = _lib.Conv2d.from_layer(a, algo=HALO), _lib.Conv2d.from_layer(a), _lib.Conv2d.from_layer(b)
    ci = _lib.Conv2d.from_layer(a, algo=1)
    assert _lib.fusable(ch, c2) and _lib.fusable(ci, c2)
    d = _lib.describe_fused(ch, c2)
    assert d.startswith("halo fused_1x1 "), d
    x, w1, b1, w2, b2 = ta["x"].cuda(), ta["w"].cuda(), ta["b"].cuda(), tb["w"].cuda(), tb["b"].cuda()
    t = c1.run(x, w1, b1)
    ys = c2.run(t, w2, b2)
    outs = []
    for cc in (ch, ci):
        y = c2.empty_output()
        y.fill_(float("nan"))
        _lib.run_fused(cc, c2, x, w1, b1, w2, b2, y)
        outs.append(y)
    torch.cuda.synchronize()
    for c in (ch, c1, c2, ci):
        c.close()
    return ys.cpu(), outs[0].cpu(), outs[1].cpu(), d


@pytest.mark.parametrize("case", PAIRS, ids=[c[0].name[:-2] for c in PAIRS])
def test_halo_fused_pairs(case):
    a, b = case
    print("halo fused", a.name, flush=True)
    ta = random_layer_tensors(a, "bf16", seed=75)
    tb = random_layer_tensors(b, "bf16", seed=76)
    ys, yh, yi, d = fused_runs(a, b, ta, tb)
    same_bits(ys, yh, "%s separate vs halo fused [%s]" % (a.name, d))
    same_bits(yi, yh, "%s igemm fused vs halo fused" % a.name)
    ra = H.oracle_full(a, ta["x"], ta)
    rb = H.oracle_full(b, H.round_like_output(ra[0], "bf16"), tb)
    H.check_chain(yh.float().numpy(), rb[0], rb[1], "%s halo fused vs oracle chain" % a.name)


@pytest.mark.parametrize("first", [1, 4])
def test_halo_fused_yolo640_pairs_full_size(first):
    """L2 -> L3 and L5 -> L6 of the 640x640 stack through the halo kernel."""
    wl = workload("yolo640_bf16")
    a, b = wl.layers[first], wl.layers[first + 1]
    ta = dict(layer_params(wl, first))
    ta["x"] = torch.randn((a.n, a.h, a.w, a.cin), generator=torch.Generator().manual_seed(77)).to(torch.bfloat16)
    tb = layer_params(wl, first + 1)
    print("halo fused full size", a.name, b.name, flush=True)
    ys, yh, yi, d = fused_runs(a, b, ta, tb)
    same_bits(ys, yh, "%s+%s separate vs halo fused [%s]" % (a.name, b.name, d))
    same_bits(yi, yh, "%s+%s igemm fused vs halo fused" % (a.name, b.name))
