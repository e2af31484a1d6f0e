"""GPU parity on the five workloads at their full sizes, in the launch
configuration the benchmark times (automatic kernel/tile choice).

Every layer of the chained stacks (KWS int8, VWW bf16, the 640x640 YOLO
stack) is first checked on its own at full size with a fresh seeded input,
under the strict per-layer rules. The chains are then run twice:
once on the GPU, each layer consuming the GPU's previous output, and once
through the oracle, each layer consuming the oracle's previous output
rounded to the layer's output type. Every layer of the GPU chain is then
compared with the same layer of the oracle chain (bit-exact for int8; for
bf16 under the chain rule of tests/helpers.py, which bounds the effect of
one-ulp rounding flips between the two chains' inputs). No oracle input
comes from the GPU. The batched N=16 sweeps and the depthwise probe are
compared on sampled outputs (random positions plus every border class), which the
oracle evaluates one by one.
"""
import numpy as np
import pytest
import torch

from convolution_conv2d_nhwc_amd import _lib
from convolution_conv2d_nhwc_amd.data import fresh_input, layer_params, network_input, workload
from oracle import oracle
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _run_chain(wl, x0_gpu):
    outs = []
    x = x0_gpu
    for i, layer in enumerate(wl.layers):
        p = layer_params(wl, i)
        y, conv = H.gpu_run(layer, x, p)
        outs.append((y, conv.describe()))
        conv.close()
        x = y
    torch.cuda.synchronize()
    return outs


def _oracle_chain_check(wl, x0_cpu, gpu_outs, skip=()):
    """Compare gpu_outs[i] with layer i of the oracle chain, except for the
    layers in `skip` (outputs a fused launch never stores)."""
    x = x0_cpu
    stats = []
    for i, layer in enumerate(wl.layers):
        p = layer_params(wl, i)
        ref = H.oracle_full(layer, x, p)
        y, desc = gpu_outs[i]
        what = "%s/%s [%s]" % (wl.name, layer.name, desc)
        if i in skip:
            stats.append(None)
            x = H.round_like_output(ref[0], layer.out)
            continue
        if layer.dtype == "i8":
            stats.append(H.check_int(y.cpu().numpy(), ref, layer, what))
            x = torch.from_numpy(ref[0]) if layer.out == "i8" else torch.from_numpy(ref)
        else:
            stats.append(H.check_chain(y.cpu().float().numpy(), ref[0], ref[1], what))
            x = H.round_like_output(ref[0], layer.out)
    return stats


@pytest.mark.parametrize("name", ["kws_int8", "vww_bf16", "yolo640_bf16"])
def test_stack_layers_fresh_inputs(name):
    """Each layer of a stack on its own, full size, strict rules."""
    wl = workload(name)
    for i, layer in enumerate(wl.layers):
        p = layer_params(wl, i)
        x = fresh_input(wl, i)
        y, conv = H.gpu_run(layer, x, p)
        s = H.check_layer_full(layer, x, p, y, "%s/%s [%s]" % (name, layer.name, conv.describe()))
        print(name, layer.name, conv.describe(), s)
        conv.close()


def test_mnist_f32_full():
    wl = workload("mnist_f32")
    layer = wl.layers[0]
    x = network_input(wl)
    p = layer_params(wl, 0)
    y, conv = H.gpu_run(layer, x, p)
    H.check_layer_full(layer, x, p, y, "mnist_f32")


def test_kws_int8_chain_bit_exact():
    wl = workload("kws_int8")
    x0 = network_input(wl)
    outs = _run_chain(wl, x0.cuda())
    stats = _oracle_chain_check(wl, x0, outs)
    assert all(s["mismatch"] == 0 for s in stats)


def test_vww_bf16_chain():
    wl = workload("vww_bf16")
    x0 = network_input(wl)
    outs = _run_chain(wl, x0.cuda())
    _oracle_chain_check(wl, x0, outs)


def test_yolo640_mosaic_and_chain():
    wl = workload("yolo640_bf16")
    tiles = network_input(wl)
    canvas = _lib.mosaic_pack(tiles.cuda(), out_dtype=torch.bfloat16)
    ref_bits = oracle.mosaic(tiles.numpy(), out="bf16")
    got_bits = canvas.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got_bits, ref_bits), "mosaic not bit-exact"
    x0 = torch.from_numpy(ref_bits.view(np.int16)).view(torch.bfloat16)
    outs = _run_chain(wl, canvas)
    stats = _oracle_chain_check(wl, x0, outs)
    for layer, s in zip(wl.layers, stats):
        print(layer.name, s)


@pytest.mark.parametrize("name", ["yolo640_bf16", "kws_int8", "vww_bf16", "mnist_f32"])
def test_stack_graph_replay_matches_oracle(name):
    """The exact graph bench.py times (the Stack executor: mosaic + every
    layer captured once, replayed, with the fusable 3x3 + 1x1 pairs as one
    launch): after the first replay every stored layer output is checked
    against the oracle chain (int8 bit-exact, bf16 under the chain rule, the
    single fp32 layer under the strict rule); two more replays, with every
    buffer overwritten by eager fills in between, and one eager pass must
    reproduce it bit for bit."""
    from convolution_conv2d_nhwc_amd.stack import Stack
    wl = workload(name)
    st = Stack(wl, fuse=True)
    if name == "yolo640_bf16":
        assert (1, 2) in st.nodes() and (4, 5) in st.nodes(), st.nodes()
    unstored = [n[0] for n in st.nodes() if len(n) == 2]
    st.capture()
    st.replay()
    torch.cuda.synchronize()
    first = [b.clone() for b in st.bufs]
    descs = [c.describe() for c in st.convs]
    for n in st.nodes():
        if len(n) == 2:
            descs[n[1]] = st.node_kernel(n)
    if wl.mosaic is not None:
        bits = oracle.mosaic(network_input(wl).numpy(), out="bf16")
        if st.canvas is not None:
            can = st.canvas.cpu().view(torch.int16).numpy().view(np.uint16)
            c = bits.shape[-1]
            # the canvas may carry zero pad channels for the first layer's kernel
            assert np.array_equal(can[..., :c], bits), "mosaic"
            assert not np.any(can[..., c:]), "mosaic pad channels"
        else:
            assert st.mosaic_fused  # the first layer read the tiles: its output is checked below
        x0 = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    elif wl.chained:
        x0 = network_input(wl)
    else:
        x0 = None
    if x0 is None:
        p = layer_params(wl, 0)
        H.check_layer_full(wl.layers[0], p["x"], p, first[0], "%s graph [%s]" % (name, descs[0]))
    else:
        stats = _oracle_chain_check(wl, x0, list(zip(first, descs)), skip=unstored)
        print(name, stats[-1])
    for rep in range(2):
        for b in st.bufs:
            b.fill_(-77 if b.dtype == torch.int8 else float("nan") if b.dtype.is_floating_point else -(2 ** 30))
        if st.canvas is not None:
            st.canvas.zero_()
        st.replay()
        torch.cuda.synchronize()
        for i, (b, f0) in enumerate(zip(st.bufs, first)):
            if i not in unstored:
                assert torch.equal(b.view(torch.uint8), f0.view(torch.uint8)), (name, "replay", rep, i)
    st.step()
    torch.cuda.synchronize()
    for i, (b, f0) in enumerate(zip(st.bufs, first)):
        if i not in unstored:
            assert torch.equal(b.view(torch.uint8), f0.view(torch.uint8)), (name, "eager", i)
    st.close()


@pytest.mark.parametrize("name", ["yolo_sweep_int8", "yolo_sweep_bf16"])
def test_yolo_sweep_sampled(name):
    wl = workload(name)
    for i, layer in enumerate(wl.layers):
        p = layer_params(wl, i)
        y, conv = H.gpu_run(layer, p["x"], p)
        torch.cuda.synchronize()
        s = H.check_layer_sampled(layer, p["x"], p, y, count=3000, what="%s/%s [%s]" % (name, layer.name, conv.describe()))
        print(name, layer.name, conv.describe(), s)
        conv.close()
        del y


@pytest.mark.parametrize("name", ["yolo_sweep_int8", "yolo_sweep_bf16"])
def test_yolo_sweep_full_elementwise(name):
    """Every output of every N=16 sweep layer (each shipped kernel instance at
    its real shape: the 128x128 implicit-GEMM tile on 160x160x128, the
    large-layer tiles on the 80x80, 40x40 and 20x20 3x3 layers, the 1x1
    loaders) against the oracle under the strict rules."""
    wl = workload(name)
    for i, layer in enumerate(wl.layers):
        p = layer_params(wl, i)
        y, conv = H.gpu_run(layer, p["x"], p)
        torch.cuda.synchronize()
        s = H.check_layer_full(layer, p["x"], p, y, "%s/%s full [%s]" % (name, layer.name, conv.describe()))
        print(name, layer.name, conv.describe(), s, flush=True)
        conv.close()
        del y


def test_yolo_sweep_int32_checkpoint_sampled():
    """The int8 sweep with the int32 checkpoint output: bit-exact."""
    from dataclasses import replace
    wl = workload("yolo_sweep_int8")
    for i, layer0 in enumerate(wl.layers):
        layer = replace(layer0, out="i32", act="none")
        p = layer_params(wl, i)
        y, conv = H.gpu_run(layer, p["x"], p)
        torch.cuda.synchronize()
        H.check_layer_sampled(layer, p["x"], p, y, count=2000, what="i32/%s [%s]" % (layer.name, conv.describe()))
        conv.close()


@pytest.mark.parametrize("name", ["dw_probe_bf16", "dw_probe_int8"])
def test_dw_probe_sampled(name):
    wl = workload(name)
    for i, layer in enumerate(wl.layers):
        p = layer_params(wl, i)
        y, conv = H.gpu_run(layer, p["x"], p)
        torch.cuda.synchronize()
        H.check_layer_sampled(layer, p["x"], p, y, count=3000, what="%s/%s [%s]" % (name, layer.name, conv.describe()))
        conv.close()


@pytest.mark.gpu
def test_residual_resblock_full_size():
    """The residual epilogue at the size bench.py times it: a CSPDarknet
    ResBlock tail of the 640-pixel network (3x3, 64 -> 64, Mish, 320x320,
    N=1, bf16), every output against the oracle's activation plus the
    residual, and in place."""
    from convolution_conv2d_nhwc_amd.data import Layer, random_layer_tensors
    layer = Layer("resblock_3x3_64", 1, 320, 320, 64, 64, 3, 3, 1, 1, 1, 1, 1, "bf16", "bf16", "mish", 320, 320)
    t = random_layer_tensors(layer, "bf16", seed=7)
    ref = H.oracle_full(layer, t["x"], t)
    g = torch.Generator().manual_seed(8)
    res = (torch.randn((1, 320, 320, 64), generator=g) * 0.5).to(torch.bfloat16)
    r, a = oracle.add_residual_float(ref[0], ref[1], res.float().numpy())
    conv = _lib.Conv2d.from_layer(layer)
    x, w, b = t["x"].cuda(), t["w"].cuda(), t["b"].cuda()
    for inplace in (False, True):
        rg = res.cuda()
        y = rg if inplace else conv.empty_output()
        conv.run(x, w, b, y, residual=rg)
        torch.cuda.synchronize()
        H.check_float(y.cpu().float().numpy(), r, a, "bf16", "resblock inplace=%s [%s]" % (inplace, conv.describe()))
    conv.close()
