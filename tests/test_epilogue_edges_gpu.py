"""GPU regression tests of two epilogue edge cases, on every kernel path:

* int8 residual add at exact ties. The residual epilogue (zerolat.eu YOLOv4
  report, section 9 "Four custom Tensix kernels", K2: no intermediate
  rounding of the activation before the add) rounds the exact sum
  act(v) + r once. With scale 0.5 and odd acc + bias, v is an exact
  half-integer, so half of the outputs with an odd residual sit on a tie that
  a kernel rounding act(v) first and adding r afterwards gets wrong
  (rne(2.5) + 1 = 3, rne(3.5) = 4). Bit-exact against the oracle's
  ``add_residual_i8``.
* Mish at large negative pre-activations (v in [-30, -3]), where
  v - 2v/((1+e^v)^2+1) cancels: every bf16 output must keep its sign and be
  within 2^-7 of the true value relative to itself (not to the absolute-value
  convolution, whose floor would hide the cancellation).
"""
import numpy as np
import pytest
import torch

from convolution_conv2d_nhwc_amd import _lib
from oracle import oracle
from tests import helpers as H
from tests.test_parity_gpu import L, XL_ALGOS, forced_tiles

pytestmark = pytest.mark.gpu

# One int8 layer per kernel path that writes an int8 output, with the
# describe() text that names the path.
TIE_LAYERS = [
    (L("tie_i8_tap", 1, 12, 11, 128, 64, 3, 3, (1, 1), (1, 1), dtype="i8", out="i8", act="none"), "loader=tap"),
    (L("tie_i8_vec_s2", 1, 13, 12, 32, 48, 3, 3, (2, 2), (1, 1), dtype="i8", out="i8", act="relu"), "loader=vec16"),
    (L("tie_i8_1x1", 2, 9, 7, 64, 96, 1, 1, dtype="i8", out="i8", act="none"), "loader=1x1"),
    (L("tie_i8_cout5", 1, 15, 17, 16, 5, 3, 3, (1, 1), (1, 1), dtype="i8", out="i8", act="none"), "igemm"),
    (L("tie_i8_xl", 1, 13, 9, 128, 256, 3, 3, (1, 1), (1, 1), dtype="i8", out="i8", act="none"), "igemm_xl"),
    (L("tie_i8_smallk", 1, 17, 15, 3, 32, 3, 3, (1, 1), (1, 1), dtype="i8", out="i8", act="relu"), "smallk"),
    (L("tie_i8_splitk", 1, 8, 8, 512, 256, 3, 3, (1, 1), (1, 1), dtype="i8", out="i8", act="none"), "ksplit="),
    (L("tie_i8_xl_1x1", 1, 12, 12, 128, 128, 1, 1, dtype="i8", out="i8", act="none"), "igemm_xl"),
    (L("tie_i8_xl_splitk", 1, 8, 8, 512, 256, 3, 3, (1, 1), (1, 1), dtype="i8", out="i8", act="none"), "igemm_xl"),
    (L("tie_dw_i8_rows", 1, 9, 10, 64, 64, 3, 3, (1, 1), (1, 1), groups=64, dtype="i8", out="i8", act="none"),
     "dw3x3_i8_kernel"),
    (L("tie_dw_i8_s2", 1, 12, 12, 32, 32, 3, 3, (2, 2), (1, 1), groups=32, dtype="i8", out="i8", act="relu"),
     "dw3x3_kernel"),
]


def _tie_tensors(layer, seed):
    """Small int8 values (so that sums stay far from saturation), scale 0.5
    on every channel (v = (acc + b) / 2 exactly), residual in [-20, 20]."""
    g = np.random.default_rng(seed)
    x = g.integers(-3, 4, (layer.n, layer.h, layer.w, layer.cin)).astype(np.int8)
    w = g.integers(-3, 4, (layer.cout, layer.kh, layer.kw, layer.cin // layer.groups)).astype(np.int8)
    b = g.integers(-40, 41, layer.cout).astype(np.int32)
    s = np.full(layer.cout, 0.5, np.float32)
    return {"x": torch.from_numpy(x), "w": torch.from_numpy(w), "b": torch.from_numpy(b), "s": torch.from_numpy(s)}


def _forced_algo(layer):
    if layer.name.endswith("_xl"):
        return next(a for a in forced_tiles(layer) if a in XL_ALGOS)
    if "_xl_" in layer.name:
        return next(a for a in forced_tiles(layer) if a in XL_ALGOS)
    return 0


@pytest.mark.parametrize("layer,path", TIE_LAYERS, ids=[l.name for l, _ in TIE_LAYERS])
def test_residual_i8_ties(layer, path):
    t = _tie_tensors(layer, seed=77)
    conv = _lib.Conv2d.from_layer(layer, algo=_forced_algo(layer))
    d = conv.describe()
    assert path in d, (layer.name, d)
    if layer.name.endswith("splitk") and torch.cuda.is_available():
        assert "ksplit=1 " not in d, d
    q_plain, m = H.oracle_full(layer, t["x"], t)
    g = np.random.default_rng(78)
    res = g.integers(-20, 21, conv.out_shape).astype(np.int8)
    q_ref, tsum = oracle.add_residual_i8(m, res)
    # the case this test exists for: an exact half-integer activation and an
    # odd residual (rounding act(v) first would give the other neighbour)
    frac = np.abs(m - np.floor(m) - 0.5) == 0
    hits = int(np.sum(frac & (res % 2 != 0) & (np.abs(tsum) < 126)))
    assert hits >= 50, (layer.name, hits)
    b = _lib.pack_bias_scale(t["b"], t["s"]).cuda()
    y = conv.empty_output()
    y.fill_(-77)
    conv.run(t["x"].cuda(), t["w"].cuda(), b, y, residual=torch.from_numpy(res).cuda())
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    bad = np.nonzero(got.reshape(-1) != q_ref.reshape(-1))[0]
    assert bad.size == 0, "%s [%s]: %d of %d differ (%d tie cases), first %s: got %s want %s (m=%s r=%s)" % (
        layer.name, d, bad.size, got.size, hits, bad[:4], got.reshape(-1)[bad[:4]], q_ref.reshape(-1)[bad[:4]],
        m.reshape(-1)[bad[:4]], res.reshape(-1)[bad[:4]])
    # and the plain epilogue of the same layer is unchanged (ties to even)
    y2 = conv.run(t["x"].cuda(), t["w"].cuda(), b)
    torch.cuda.synchronize()
    assert np.array_equal(y2.cpu().numpy(), q_plain), layer.name
    conv.close()


# Layers whose output channel co at every pixel equals one input value
# (a unit centre tap), so the pre-activation is exactly the input value.
NEG_LAYERS = [
    (L("neg_bf16_tap", 1, 10, 9, 64, 64, 3, 3, (1, 1), (1, 1)), "loader=tap"),
    (L("neg_bf16_1x1", 1, 9, 9, 64, 32, 1, 1), "loader=1x1"),
    (L("neg_bf16_vec_s2", 1, 11, 10, 32, 40, 3, 3, (2, 2), (1, 1)), "loader=vec16"),
    (L("neg_bf16_xl", 1, 11, 9, 128, 256, 3, 3, (1, 1), (1, 1)), "igemm_xl"),
    (L("neg_bf16_smallk", 1, 13, 11, 3, 32, 3, 3, (1, 1), (1, 1)), "smallk"),
    (L("neg_bf16_splitk", 1, 8, 8, 512, 256, 3, 3, (1, 1), (1, 1)), "ksplit="),
    (L("neg_bf16_xl_splitk", 1, 8, 8, 512, 256, 3, 3, (1, 1), (1, 1)), "igemm_xl"),
    (L("neg_dw_bf16_rows", 1, 9, 10, 64, 64, 3, 3, (1, 1), (1, 1), groups=64), "dw3x3_rows_kernel"),
    (L("neg_dw_bf16_s2", 1, 12, 12, 32, 32, 3, 3, (2, 2), (1, 1), groups=32), "dw3x3_kernel"),
    (L("neg_f32", 1, 10, 10, 4, 8, 3, 3, (1, 1), (1, 1), dtype="f32"), "direct_f32"),
    (L("neg_dw_f32", 1, 9, 9, 8, 8, 3, 3, (1, 1), (1, 1), groups=8, dtype="f32"), "dw3x3"),
]


@pytest.mark.parametrize("layer,path", NEG_LAYERS, ids=[l.name for l, _ in NEG_LAYERS])
def test_mish_large_negative(layer, path):
    assert layer.act == "mish"
    g = np.random.default_rng(91)
    xv = -g.uniform(3.0, 30.0, (layer.n, layer.h, layer.w, layer.cin)).astype(np.float32)
    w = np.zeros((layer.cout, layer.kh, layer.kw, layer.cin // layer.groups), np.float32)
    ch, cw = layer.kh // 2, layer.kw // 2
    if layer.groups > 1:
        w[:, ch, cw, 0] = 1.0
    else:
        w[np.arange(layer.cout), ch, cw, np.arange(layer.cout) % layer.cin] = 1.0
    tdt = torch.bfloat16 if layer.dtype == "bf16" else torch.float32
    x = torch.from_numpy(xv).to(tdt)
    wt = torch.from_numpy(w).to(tdt)
    b = torch.zeros(layer.cout, dtype=torch.float32)
    conv = _lib.Conv2d.from_layer(layer, algo=_forced_algo(layer))
    d = conv.describe()
    assert path in d, (layer.name, d)
    y = conv.run(x.cuda(), wt.cuda(), b.cuda())
    torch.cuda.synchronize()
    r, a = oracle.conv_float(x.float().numpy(), wt.float().numpy(), b.numpy(), (layer.sh, layer.sw),
                             (layer.ph, layer.pw), layer.groups, "mish")
    yc = y.cpu().float().numpy().astype(np.float64)
    # every pre-activation is one input value in [-30, -3]: Mish is negative
    # and at least 2.8e-12 in magnitude, far inside the normal float range
    assert np.all(r < 0) and np.all(np.abs(r) > 1e-12)
    rel = np.abs(yc - r) / np.abs(r)
    tol = 2.0 ** -7 if layer.dtype == "bf16" else 1e-5
    i = int(np.argmax(rel))
    assert np.all(yc < 0) and rel.max() <= tol, "%s [%s]: worst rel err %.3g at %d: y=%r r=%r" % (
        layer.name, d, rel.max(), i, yc.reshape(-1)[i], r.reshape(-1)[i])
    conv.close()
