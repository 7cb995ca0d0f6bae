"""MXFP8 (E4M3 elements, E8M0 block scales) quantiser of the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/moe_oracle.py``).

The pages only name the format: the Olmo-core 3 article's "three splits" section
switches the expert GEMMs to MXFP8, and the SonicMoE article's closing section
lists FP8/MXFP8 as future work.  The element and scale rules below are those of
the public OCP Microscaling (MX) v1.0 specification:

* a block is 32 consecutive values along the GEMM's reduction axis;
* shared exponent X = floor(log2(max |v|)) - 8, where 8 is the largest exponent
  of E4M3, clamped to [-127, 127]; an all-zero block takes X = -127;
* scale byte (E8M0) = X + 127;
* element = v / 2^X rounded to nearest-even E4M3 ("FN" variant: bias 7, three
  mantissa bits, largest finite 448, subnormal quantum 2^-9), saturating at
  +-448; the element byte keeps the sign bit of v.

A trailing partial block (fewer than 32 values) takes its maximum over the
values it has; missing values count as zero.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6
E4M3_SUB_QUANTUM = 2.0 ** -9
EMAX_ELEM = 8


def _floor_log2(v):
    """floor(log2(v)) for v > 0, exactly (via frexp: v = m * 2^e, 0.5 <= m < 1)."""
    _, e = np.frexp(v)
    return e - 1


def e4m3_round(s):
    """Round non-negative float64 values to the nearest E4M3 value, ties to even,
    saturating at 448."""
    s = np.asarray(s, np.float64)
    out = np.zeros_like(s)
    nz = s > 0
    v = s[nz]
    ex = _floor_log2(v)
    normal = ex >= E4M3_MIN_NORMAL_EXP
    q = np.where(normal, np.ldexp(1.0, np.maximum(ex, E4M3_MIN_NORMAL_EXP) - 3), E4M3_SUB_QUANTUM)
    r = np.round(v / q) * q
    out[nz] = np.minimum(r, E4M3_MAX)
    return out


def e4m3_encode(sign, mag):
    """Byte of an E4M3 value given its sign bit (0/1) and an exactly representable magnitude."""
    mag = np.asarray(mag, np.float64)
    code = np.zeros(mag.shape, np.int64)
    sub = (mag > 0) & (mag < 2.0 ** E4M3_MIN_NORMAL_EXP)
    code[sub] = np.round(mag[sub] / E4M3_SUB_QUANTUM).astype(np.int64)
    nrm = mag >= 2.0 ** E4M3_MIN_NORMAL_EXP
    ex = _floor_log2(mag[nrm])
    mant = np.round((mag[nrm] / np.ldexp(1.0, ex) - 1.0) * 8).astype(np.int64)
    code[nrm] = ((ex + 7) << 3) | mant
    return (code | (np.asarray(sign, np.int64) << 7)).astype(np.uint8)


def e4m3_decode(code):
    code = np.asarray(code, np.int64)
    sign = np.where(code & 0x80, -1.0, 1.0)
    ef = (code >> 3) & 0xF
    m = code & 7
    val = np.where(ef == 0, m * E4M3_SUB_QUANTUM, np.ldexp(1.0 + m / 8.0, ef - 7))
    return sign * val


def quantize(v, axis=-1):
    """MX-quantise ``v`` along ``axis`` in blocks of 32.

    Returns (codes uint8 same shape as v, scales uint8 with the axis length
    ceil(n/32), dequantised float64 values)."""
    v = np.asarray(v, np.float64)
    vm = np.moveaxis(v, axis, -1)
    n = vm.shape[-1]
    nb = -(-n // BLOCK)
    pad = nb * BLOCK - n
    if pad:
        vm = np.concatenate([vm, np.zeros(vm.shape[:-1] + (pad,))], axis=-1)
    blk = vm.reshape(vm.shape[:-1] + (nb, BLOCK))
    amax = np.abs(blk).max(axis=-1)
    X = np.full(amax.shape, -127, np.int64)
    pos = amax > 0
    X[pos] = np.clip(_floor_log2(amax[pos]) - EMAX_ELEM, -127, 127)
    scale = np.ldexp(1.0, X)[..., None]
    mag = e4m3_round(np.abs(blk) / scale)
    sign = np.signbit(blk).astype(np.int64)
    codes = e4m3_encode(sign, mag)
    deq = np.where(sign == 1, -mag, mag) * scale
    codes = codes.reshape(vm.shape)[..., :n]
    deq = deq.reshape(vm.shape)[..., :n]
    return (np.moveaxis(codes, -1, axis), np.moveaxis((X + 127).astype(np.uint8), -1, axis),
            np.moveaxis(deq, -1, axis))


def mx_roundtrip(v, axis=-1):
    """Dequantised MXFP8 values of ``v`` (blocks along ``axis``)."""
    return quantize(v, axis)[2]


def block_exponent(amax):
    """Shared exponent the amax rule picks for blocks whose largest magnitude is
    ``amax`` (a scalar, or an array of them)."""
    a = np.asarray(amax, np.float64)
    X = np.full(a.shape, -127, np.int64)
    pos = a > 0
    X[pos] = np.clip(_floor_log2(a[pos]) - EMAX_ELEM, -127, 127)
    return int(X) if X.ndim == 0 else X


def roundtrip_at(block, X):
    """Dequantised values of ``block`` quantised with the shared exponent ``X``
    given by the caller instead of the one the amax rule picks (elements still
    rounded to nearest-even E4M3 and saturated at 448).  With X one above or
    below the rule's choice this is the other outcome of a scale decision taken
    on an amax that sits at a power of two."""
    b = np.asarray(block, np.float64)
    scale = np.ldexp(1.0, int(X))
    mag = e4m3_round(np.abs(b) / scale)
    return np.where(np.signbit(b), -mag, mag) * scale
