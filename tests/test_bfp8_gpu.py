"""Block-floating-point (bfp8) weights on the GPU, against the oracle.

* conv_pack_bfp8 must reproduce oracle/bfp8.encode byte for byte (integer
  work: bit-exact), from bf16 and fp32 weights, including ties, the exponent
  bump, zero and padded blocks and tiny magnitudes.
* A layer with bfp8 weights computes the bf16 convolution of the decoded
  weights; it is compared with the oracle's fp64 convolution on
  oracle/bfp8.decode(oracle/bfp8.encode(w)) under the bf16 rule, on every
  16-byte loader, every implicit-GEMM tile, a split reduction, the residual
  epilogue, and the 40x40x512 -> 512 3x3 layer of the N=16 YOLO sweep
  (sampled outputs, plus one full image element by element)."""
import numpy as np
import pytest
import torch

from convolution_conv2d_nhwc_amd import _lib
from convolution_conv2d_nhwc_amd.data import Layer, random_layer_tensors
from oracle import bfp8, oracle
from tests import helpers as H

pytestmark = pytest.mark.gpu


def L(name, n, h, w, cin, cout, k, s=1, p=None, act="mish"):
    p = k // 2 if p is None else p
    ho, wo = oracle.out_hw(h, w, k, k, s, s, p, p)
    return Layer(name, n, h, w, cin, cout, k, k, s, s, p, p, 1, "bf16", "bf16", act, ho, wo)


def oracle_encode(w: torch.Tensor):
    w2 = w.float().reshape(w.shape[0], -1).numpy()
    return bfp8.encode(w2)


def decoded_params(t):
    """The layer's tensors with the weights replaced by decode(encode(w))
    (exactly bf16 values)."""
    w = t["w"]
    m, e = oracle_encode(w)
    d = bfp8.decode(m, e, w[0].numel()).reshape(tuple(w.shape))
    out = dict(t)
    out["w"] = torch.from_numpy(d.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(out["w"].double(), torch.from_numpy(d))
    return out


@pytest.mark.parametrize("shape,dt", [((64, 3, 3, 64), "bf16"), ((37, 3, 5, 9), "f32"), ((128, 3, 3, 256), "bf16"),
                                      ((5, 1, 1, 20), "f32")])
def test_pack_bit_exact(shape, dt):
    rng = np.random.default_rng(7)
    k = int(np.prod(shape[1:]))
    w = torch.from_numpy(rng.normal(0, np.sqrt(2.0 / k), shape).astype(np.float32))
    if dt == "bf16":
        w = w.to(torch.bfloat16)
    print("bfp8 pack", shape, dt, flush=True)
    got = _lib.pack_bfp8(w.cuda().contiguous()).cpu().numpy()
    m, e = oracle_encode(w)
    want = bfp8.pack(m, e)
    assert got.size == want.size == _lib.bfp8_bytes(shape[0], k)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "%d bytes differ, first %s: got %s want %s" % (bad.size, bad[:6], got[bad[:6]], want[bad[:6]])


def test_pack_special_blocks_bit_exact():
    # row 0: powers of two; row 1: ties; row 2: the exponent bump; row 3:
    # zeros; row 4: tiny magnitudes (fp32 denormals); K = 20 pads each row
    w = np.zeros((5, 20), dtype=np.float32)
    w[0, :4] = [1.0, 0.5, -0.25, 0.75]
    w[1, :5] = [1.0, 3 / 128, 5 / 128, 7 / 128, -3 / 128]
    w[2, :2] = [1.9921875, 0.03125]
    w[4, :2] = [2.0 ** -130, 2.0 ** -132]
    w[4, 16:18] = [-(2.0 ** -140), 2.0 ** -141]
    wt = torch.from_numpy(w)
    got = _lib.pack_bfp8(wt.cuda()).cpu().numpy()
    m, e = bfp8.encode(w)
    want = bfp8.pack(m, e)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "%d bytes differ, first %s: got %s want %s" % (bad.size, bad[:6], got[bad[:6]], want[bad[:6]])


# every 16-byte loader, ragged pixel and channel counts, strides
LAYERS = [
    L("q_tap_3x3_c64", 1, 19, 23, 64, 96, 3),
    L("q_tap_3x3s2_c128", 2, 17, 15, 128, 64, 3, s=2, act="relu"),
    L("q_vec_3x3_c32", 1, 21, 18, 32, 40, 3, act="relu6"),
    L("q_vec_5x5_c24", 1, 13, 11, 24, 48, 5, act="none"),
    L("q_1x1_c64", 2, 15, 17, 64, 72, 1),
    L("q_1x1_c40", 1, 19, 13, 40, 32, 1, act="relu"),  # K = 40: a padded last block
]


@pytest.mark.parametrize("layer", LAYERS, ids=[l.name for l in LAYERS])
def test_conv_all_tiles(layer):
    t = random_layer_tensors(layer, "bf16", seed=41)
    tq = decoded_params(t)
    ref = H.oracle_full(layer, t["x"], tq)
    xg, wq, b = t["x"].cuda(), _lib.pack_bfp8(t["w"].cuda()), t["b"].cuda()
    for algo in (0, 1, 2, 3, 4):
        conv = _lib.Conv2d.from_layer(layer, algo=algo, w_format="bfp8")
        d = conv.describe()
        assert "w=bfp8" in d and d.startswith("igemm "), d
        y = conv.empty_output()
        y.fill_(float("nan"))
        conv.run(xg, wq, b, y)
        H.check_float(y.cpu().float().numpy(), ref[0], ref[1], "bf16", "%s algo=%d [%s]" % (layer.name, algo, d))
        conv.close()


def test_conv_split_k_and_noalloc():
    layer = L("q_splitk_10x10_512_256", 1, 10, 10, 512, 256, 3)
    t = random_layer_tensors(layer, "bf16", seed=42)
    tq = decoded_params(t)
    conv = _lib.Conv2d.from_layer(layer, w_format="bfp8")
    d = conv.describe()
    assert "ksplit=" in d and "ksplit=1 " not in d, d
    xg, wq, b = t["x"].cuda(), _lib.pack_bfp8(t["w"].cuda()), t["b"].cuda()
    y = conv.run(xg, wq, b)
    H.check_layer_full(layer, t["x"], tq, y, "%s [%s]" % (layer.name, d))
    y2 = conv.empty_output()
    conv.run_noalloc(xg, wq, b, y2)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), y2.cpu())


def test_conv_residual():
    layer = L("q_res_3x3_c64", 1, 14, 13, 64, 64, 3)
    t = random_layer_tensors(layer, "bf16", seed=43)
    tq = decoded_params(t)
    conv = _lib.Conv2d.from_layer(layer, w_format="bfp8")
    r = (0.5 * torch.randn(conv.out_shape, generator=torch.Generator().manual_seed(44))).to(torch.bfloat16)
    y = conv.run(t["x"].cuda(), _lib.pack_bfp8(t["w"].cuda()), t["b"].cuda(), residual=r.cuda())
    rr, a = H.oracle_full(layer, t["x"], tq)
    want, asum = oracle.add_residual_float(rr, a, r.float().numpy().astype(np.float64))
    H.check_float(y.cpu().float().numpy(), want, asum, "bf16", layer.name)


def test_unsupported_layers_refused():
    # the 3-channel stem, int8, depthwise and a forced large-layer tile
    for kw in (dict(c_in=3, c_out=32), dict(c_in=64, c_out=64, dtype="i8", out_dtype="i8"),
               dict(c_in=64, c_out=64, groups=64), dict(c_in=64, c_out=256, algo=5)):
        args = dict(n=1, h=20, w=20, c_in=64, c_out=64, kh=3, kw=3, stride=(1, 1), pad=(1, 1), groups=1,
                    dtype="bf16", out_dtype=None, act="none", algo=0, w_format="bfp8")
        args.update(kw)
        with pytest.raises(_lib.ConvError) as e:
            _lib.Conv2d(**args)
        assert e.value.name == "CONV_E_UNSUPPORTED", kw


C5 = L("q_40sq_3x3_512to512", 16, 40, 40, 512, 512, 3)


def test_c5_layer_sampled_and_one_image_full():
    layer = C5
    t = random_layer_tensors(layer, "bf16", seed=45)
    tq = decoded_params(t)
    conv = _lib.Conv2d.from_layer(layer, w_format="bfp8")
    d = conv.describe()
    print("bfp8 C5 layer:", d, flush=True)
    y = conv.run(t["x"].cuda(), _lib.pack_bfp8(t["w"].cuda()), t["b"].cuda())
    torch.cuda.synchronize()
    H.check_layer_sampled(layer, t["x"], tq, y, count=3000, what="%s [%s]" % (layer.name, d))
    # the last image of the batch, every output
    one = Layer(layer.name + "_img15", 1, 40, 40, 512, 512, 3, 3, 1, 1, 1, 1, 1, "bf16", "bf16", "mish", 40, 40)
    H.check_layer_full(one, t["x"][15:16], tq, y[15:16], one.name)
