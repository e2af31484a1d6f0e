"""Block-floating-point (bfp8) weights: encode and decode by the definition.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and ``bench.py``'s CPU leg;
never by the product package, and it shares no code with the HIP library.

The pages name the format and its block: YOLOv4 on Tenstorrent Wormhole, the
table "Precision in the selected m640 graph" (weights in bfp8 block floating
point, groups of 16 values sharing one exponent) and the glossary entry for
bfp8 (a shared exponent per group of values, for compact storage); the
zerolat.eu technology page, "Spend precision selectively" (bfp8 weights with
bf16 activations for most of m640, the first convolution kept in bf16). They
fix neither the mantissa width nor the rounding nor the grouping axis, so
this module takes the plain reading of "bfp8" as 8 bits per value:

* a block is 16 consecutive weights of one output channel along the
  reduction axis K = (kh, kw, ci) of the OHWI tensor; K is padded with zeros
  to Kp = 16 * ceil(K / 16);
* each value is a signed integer mantissa m in [-127, 127] (one byte), and
  the block shares one exponent byte E; the value is m * 2^(E - 133), i.e.
  a 7-bit magnitude below the block scale 2^(E - 127);
* encoding a block with largest magnitude A > 0 takes e = floor(log2 A)
  (at least -126), m_i = round_half_even(w_i / 2^(e - 6)); if a mantissa
  rounds to 128 (A / 2^(e - 6) >= 127.5) the exponent is raised by one and
  the block rounded again, so every value is within half a step of its
  input; E = e + 127. An all-zero block has E = 0 and zero mantissas.

Every decoded value has at most 7 significant bits and is therefore exactly
representable in bf16: a bf16 convolution on the decoded weights is the
computation the format defines.

Storage layout taken by the library (``conv_pack_bfp8``): the mantissas as
int8[c_out][Kp], followed by the exponents as uint8[c_out][Kp / 16].
"""
from __future__ import annotations

import numpy as np

BLOCK = 16
MANT_MAX = 127
EXP_BIAS = 127
FRAC_BITS = 6  # the largest mantissa of a block lies in [64, 127]


def padded_k(k: int) -> int:
    return BLOCK * ((k + BLOCK - 1) // BLOCK)


def packed_bytes(c_out: int, k: int) -> int:
    kp = padded_k(k)
    return c_out * kp + c_out * (kp // BLOCK)


def _blocks(w2d: np.ndarray) -> np.ndarray:
    """[rows][K] -> [rows][Kp/16][16], zero padded, as float64 (exact for
    fp32 and bf16 inputs)."""
    rows, k = w2d.shape
    kp = padded_k(k)
    out = np.zeros((rows, kp), dtype=np.float64)
    out[:, :k] = w2d.astype(np.float64)
    return out.reshape(rows, kp // BLOCK, BLOCK)


def encode(w2d: np.ndarray):
    """Weights [c_out][K] (finite fp32 or bf16 values) -> (mantissas
    int8[c_out][Kp], exponents uint8[c_out][Kp/16])."""
    blk = _blocks(np.asarray(w2d))
    if not np.all(np.isfinite(blk)):
        raise ValueError("bfp8 encodes finite weights only")
    rows, nb, _ = blk.shape
    mant = np.zeros((rows, nb, BLOCK), dtype=np.int64)
    expo = np.zeros((rows, nb), dtype=np.int64)
    for r in range(rows):
        for b in range(nb):
            v = blk[r, b]
            amax = np.max(np.abs(v))
            if amax == 0.0:
                continue  # E = 0, m = 0
            _, x = np.frexp(amax)  # amax = f * 2^x, f in [0.5, 1)
            e = max(int(x) - 1, -126)
            q = np.rint(v / 2.0 ** (e - FRAC_BITS))  # exact quotient, ties to even
            if np.max(np.abs(q)) > MANT_MAX:
                e += 1
                q = np.rint(v / 2.0 ** (e - FRAC_BITS))
            if e + EXP_BIAS > 255:
                raise ValueError("weight magnitude beyond the exponent byte")
            mant[r, b] = q
            expo[r, b] = e + EXP_BIAS
    return mant.reshape(rows, nb * BLOCK).astype(np.int8), expo.astype(np.uint8)


def decode(mant: np.ndarray, expo: np.ndarray, k: int) -> np.ndarray:
    """(mantissas, exponents) -> the weights they stand for, float64
    [c_out][K]: m * 2^(E - 133)."""
    rows, kp = mant.shape
    scale = np.ldexp(1.0, expo.astype(np.int64) - EXP_BIAS - FRAC_BITS)  # [rows][nb]
    vals = mant.astype(np.float64).reshape(rows, kp // BLOCK, BLOCK) * scale[:, :, None]
    return vals.reshape(rows, kp)[:, :k]


def pack(mant: np.ndarray, expo: np.ndarray) -> np.ndarray:
    """The byte image the library takes: mantissas, then exponents."""
    return np.concatenate([mant.reshape(-1).view(np.uint8), expo.reshape(-1)])


def unpack(buf: np.ndarray, c_out: int, k: int):
    kp = padded_k(k)
    buf = np.asarray(buf, dtype=np.uint8).reshape(-1)
    mant = buf[: c_out * kp].view(np.int8).reshape(c_out, kp)
    expo = buf[c_out * kp: c_out * kp + c_out * (kp // BLOCK)].reshape(c_out, kp // BLOCK)
    return mant, expo
