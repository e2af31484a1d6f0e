"""A KxK layer and the 1x1 layer after it in one launch (conv_run_fused).

* The fused launch must give the same bytes as the two layers run one after
  the other through conv_run: its first stage rounds the intermediate to bf16
  as a store would and the second stage reduces over the same channels in the
  same order, so the comparison is bit for bit. Cases: both gathers (tap and
  vec16), 64 and 128 intermediate channels, 4 to 64 output channels, every
  activation on either layer, a missing bias, ragged pixel counts, stride 2,
  and the two pairs of the 640x640 stack at full size.
* Against the oracle: the oracle runs the first layer, rounds its output to
  bf16 and runs the 1x1 layer on that (the chain rule of tests/helpers.py,
  which allows for one-ulp rounding differences of the intermediate).
* The fused 640x640 stack, captured and replayed as the benchmark times it,
  must reproduce the unfused stack's written buffers bit for bit.
"""
import numpy as np
import pytest
import torch

from convolution_conv2d_nhwc_amd import _lib
from convolution_conv2d_nhwc_amd.data import Layer, layer_params, random_layer_tensors, workload
from oracle import oracle
from tests import helpers as H

pytestmark = pytest.mark.gpu


def L(name, n, h, w, cin, cout, k, s=1, act="mish"):
    p = k // 2
    ho, wo = oracle.out_hw(h, w, k, k, s, s, p, p)
    return Layer(name, n, h, w, cin, cout, k, k, s, s, p, p, 1, "bf16", "bf16", act, ho, wo)


def pair(name, n, h, w, cin, cmid, cout, k=3, s=1, act1="mish", act2="mish"):
    a = L(name + "_a", n, h, w, cin, cmid, k, s, act1)
    b = L(name + "_b", n, a.ho, a.wo, cmid, cout, 1, 1, act2)
    return a, b


def run_both(a, b, ta, tb, drop_bias=False):
    """(separate, fused, descriptions) on the GPU for layers a then b."""
    c1, c2 = _lib.Conv2d.from_layer(a), _lib.Conv2d.from_layer(b)
    assert _lib.fusable(c1, c2), (a, b)
    d = _lib.describe_fused(c1, c2)
    x = ta["x"].cuda()
    w1, w2 = ta["w"].cuda(), tb["w"].cuda()
    b1 = None if drop_bias else ta["b"].cuda()
    b2 = None if drop_bias else tb["b"].cuda()
    t = c1.empty_output()
    t.fill_(float("nan"))
    c1.run(x, w1, b1, t)
    ys = c2.empty_output()
    ys.fill_(float("nan"))
    c2.run(t, w2, b2, ys)
    yf = c2.empty_output()
    yf.fill_(float("nan"))
    _lib.run_fused(c1, c2, x, w1, b1, w2, b2, yf)
    torch.cuda.synchronize()
    desc = (c1.describe(), c2.describe(), d)
    c1.close()
    c2.close()
    return ys.cpu(), yf.cpu(), desc


def assert_same_bits(ys, yf, what):
    a = ys.view(torch.int16).numpy()
    b = yf.view(torch.int16).numpy()
    bad = np.nonzero(a.reshape(-1) != b.reshape(-1))[0]
    assert bad.size == 0, "%s: %d of %d outputs differ, first at %s: separate %s fused %s" % (
        what, bad.size, a.size, bad[:6], ys.reshape(-1)[bad[:6]].tolist(), yf.reshape(-1)[bad[:6]].tolist())


CASES = [
    pair("tap_c64_64to64", 1, 19, 23, 64, 64, 64),
    pair("tap_c64_128to64_s2", 2, 21, 17, 64, 128, 64, s=2, act1="relu", act2="relu6"),
    pair("vec_c32_64to32", 1, 13, 29, 32, 64, 32, act1="relu6", act2="none"),
    pair("vec_c16_128to4", 1, 11, 9, 16, 128, 4, act1="none", act2="relu"),
    # 9216 pixels: enough workgroups that the 5x5 layer is not split
    pair("tap_c64_64to60_5x5", 1, 96, 96, 64, 64, 60, k=5, act1="mish", act2="relu"),
    pair("vec_c24_64to64_ragged", 3, 7, 5, 24, 64, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0].name[:-2] for c in CASES])
def test_fused_equals_separate_and_oracle(case):
    a, b = case
    print("fused pair", a.name, flush=True)
    ta = random_layer_tensors(a, "bf16", seed=61)
    tb = random_layer_tensors(b, "bf16", seed=62)
    ys, yf, desc = run_both(a, b, ta, tb)
    assert "fused_1x1" in desc[2], desc
    assert_same_bits(ys, yf, "%s %s" % (a.name, desc))
    # the oracle chain: layer a, rounded to bf16, then layer b
    ra = H.oracle_full(a, ta["x"], ta)
    mid = H.round_like_output(ra[0], "bf16")
    rb = H.oracle_full(b, mid, tb)
    H.check_chain(yf.float().numpy(), rb[0], rb[1], "%s fused vs oracle chain" % a.name)


def test_fused_without_bias():
    a, b = pair("nobias", 1, 15, 14, 64, 128, 48, s=2)
    ta = random_layer_tensors(a, "bf16", seed=63)
    tb = random_layer_tensors(b, "bf16", seed=64)
    ys, yf, desc = run_both(a, b, ta, tb, drop_bias=True)
    assert_same_bits(ys, yf, "no bias %s" % (desc,))


@pytest.mark.parametrize("first", [1, 4])
def test_yolo640_pairs_full_size(first):
    """L2 -> L3 (640x640x32 s2 -> 64, then 64 -> 64) and L5 -> L6 (320x320x64
    s2 -> 128, then 128 -> 64) with the stack's own seeded tensors."""
    wl = workload("yolo640_bf16")
    a, b = wl.layers[first], wl.layers[first + 1]
    ta = layer_params(wl, first)
    tb = layer_params(wl, first + 1)
    x = torch.randn((a.n, a.h, a.w, a.cin), generator=torch.Generator().manual_seed(65)).to(torch.bfloat16)
    ta = dict(ta, x=x)
    print("yolo640 pair", a.name, b.name, flush=True)
    ys, yf, desc = run_both(a, b, ta, tb)
    assert_same_bits(ys, yf, "%s+%s %s" % (a.name, b.name, desc))


def test_fused_stack_replay_matches_unfused():
    from convolution_conv2d_nhwc_amd.stack import Stack
    wl = workload("yolo640_bf16")
    ref = Stack(wl)
    ref.capture()
    ref.replay()
    torch.cuda.synchronize()
    want = [b.clone() for b in ref.bufs]
    ref.close()
    st = Stack(wl, fuse=True)
    nodes = st.nodes()
    assert (1, 2) in nodes and (4, 5) in nodes, nodes
    st.capture()
    for rep in range(3):
        for b in st.bufs:
            b.fill_(float("nan"))
        st.replay()
        torch.cuda.synchronize()
        for node in nodes:
            i = node[-1]
            assert torch.equal(st.bufs[i].view(torch.int16), want[i].view(torch.int16)), (rep, node)
    st.close()
