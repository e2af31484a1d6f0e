"""Pins of the bfp8 oracle (oracle/bfp8.py) against hand-computed blocks and
properties the definition fixes, so that a dropped rounding step, a wrong
exponent or a transposed block fails here before any GPU comparison.

Every expected value below is worked out by hand from the definition:
value = m * 2^(E - 133), e = floor(log2 max|w|), step 2^(e - 6), mantissas
rounded half to even, exponent raised by one if a mantissa would be 128."""
import numpy as np
import pytest
import torch

from oracle import bfp8

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def one_block(vals, k=16):
    w = np.zeros((1, k), dtype=np.float32)
    w[0, : len(vals)] = vals
    return w


def test_hand_block_powers_of_two():
    # max 1.0: e = 0, step 1/64 -> 1.0 = 64, 0.5 = 32, -0.25 = -16, 0.75 = 48
    m, e = bfp8.encode(one_block([1.0, 0.5, -0.25, 0.75]))
    assert list(m[0, :5]) == [64, 32, -16, 48, 0]
    assert e[0, 0] == 127
    assert np.array_equal(bfp8.decode(m, e, 16)[0, :4], [1.0, 0.5, -0.25, 0.75])


def test_hand_block_largest_mantissa_and_truncated_small_values():
    # max 1.984375 = 127/64: e = 0, mantissa 127; 0.01 / (1/64) = 0.64 -> 1;
    # 0.007 / (1/64) = 0.448 -> 0
    m, e = bfp8.encode(one_block([1.984375, 0.01, 0.007, -1.0]))
    assert list(m[0, :4]) == [127, 1, 0, -64]
    assert e[0, 0] == 127


def test_exponent_bump_when_the_maximum_rounds_to_128():
    # max 1.9921875 = 255/128: 127.5 steps of 1/64 -> ties to 128 -> e = 1,
    # step 1/32: 1.9921875 * 32 = 63.75 -> 64; 0.03125 = 1/32 -> 1
    m, e = bfp8.encode(one_block([1.9921875, 0.03125]))
    assert e[0, 0] == 128
    assert list(m[0, :2]) == [64, 1]
    assert bfp8.decode(m, e, 16)[0, 0] == 2.0
    # just below the tie (127.4 steps) keeps e = 0 and mantissa 127
    m2, e2 = bfp8.encode(one_block([127.4 / 64]))
    assert e2[0, 0] == 127 and m2[0, 0] == 127


def test_ties_round_half_to_even():
    # step 1/64 (max 1.0): 3/128 = 1.5 steps -> 2, 5/128 = 2.5 -> 2,
    # 7/128 = 3.5 -> 4, -3/128 -> -2
    m, _ = bfp8.encode(one_block([1.0, 3 / 128, 5 / 128, 7 / 128, -3 / 128]))
    assert list(m[0, 1:5]) == [2, 2, 4, -2]


def test_zero_block_and_padding():
    # K = 20: two blocks, the second holds 4 values and 12 zeros of padding;
    # the first block is all zeros
    w = np.zeros((2, 20), dtype=np.float32)
    w[1, 17] = 0.375  # block 1 of row 1: max 0.375, e = -2, step 2^-8 -> 96
    m, e = bfp8.encode(w)
    assert m.shape == (2, 32) and e.shape == (2, 2)
    assert e[0, 0] == 0 and e[0, 1] == 0 and not m[0].any()
    assert e[1, 0] == 0 and e[1, 1] == 125 and m[1, 17] == 96
    assert not np.delete(m[1], 17).any()
    assert bfp8.packed_bytes(2, 20) == 2 * 32 + 2 * 2


def test_tiny_block_exponent_floor():
    # max 2^-130 (an fp32 subnormal): e is held at -126, step 2^-132 -> 4
    m, e = bfp8.encode(one_block([2.0 ** -130, 2.0 ** -132]))
    assert e[0, 0] == 1 and list(m[0, :2]) == [4, 1]


def test_blocks_run_along_k_within_one_output_channel():
    # two rows, K = 32: each row has its own blocks; scaling row 1 by 8
    # changes only its exponents
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.05, (2, 32)).astype(np.float32)
    w[1] = w[0] * 8
    m, e = bfp8.encode(w)
    assert np.array_equal(m[0], m[1]) and np.array_equal(e[1].astype(int), e[0].astype(int) + 3)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_properties_on_kaiming_weights(seed):
    rng = np.random.default_rng(seed)
    k = 3 * 3 * 37
    w = torch.from_numpy(rng.normal(0, np.sqrt(2 / k), (24, k)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    m, e = bfp8.encode(w)
    d = bfp8.decode(m, e, k)
    kp = bfp8.padded_k(k)
    wb = np.zeros((24, kp))
    wb[:, :k] = w
    step = np.ldexp(1.0, e.astype(int) - 133)  # per block
    err = np.abs(np.pad(d, ((0, 0), (0, kp - k))) - wb).reshape(24, kp // 16, 16)
    # within half a step of the input, every element
    assert np.all(err <= step[:, :, None] / 2)
    # the largest mantissa of a nonzero block uses the top bit
    mx = np.abs(m.astype(int)).reshape(24, kp // 16, 16).max(axis=2)
    assert np.all((mx >= 64) & (mx <= 127))
    # idempotent: the decoded weights encode to the same bytes
    m2, e2 = bfp8.encode(d.astype(np.float32))
    assert np.array_equal(m, m2) and np.array_equal(e, e2)
    # sign symmetric
    m3, e3 = bfp8.encode(-w)
    assert np.array_equal(m3, -m) and np.array_equal(e3, e)
    # every decoded value is a bf16 value (7 significant bits at most)
    dt = torch.from_numpy(d.astype(np.float32))
    assert torch.equal(dt.to(torch.bfloat16).float(), dt)
    assert np.array_equal(dt.double().numpy(), d)


def test_pack_unpack_layout():
    rng = np.random.default_rng(5)
    w = rng.normal(0, 0.1, (3, 40)).astype(np.float32)
    m, e = bfp8.encode(w)
    buf = bfp8.pack(m, e)
    assert buf.dtype == np.uint8 and buf.size == bfp8.packed_bytes(3, 40) == 3 * 48 + 3 * 3
    # mantissas row-major first, then exponents row-major
    assert np.array_equal(buf[:48].view(np.int8), m[0]) and buf[3 * 48] == e[0, 0] and buf[-1] == e[2, 2]
    m2, e2 = bfp8.unpack(buf, 3, 40)
    assert np.array_equal(m, m2) and np.array_equal(e, e2)


def test_rejects_non_finite():
    with pytest.raises(ValueError):
        bfp8.encode(one_block([1.0, np.inf]))
