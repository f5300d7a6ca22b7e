"""fp64 CPU oracle for MXFP8 jagged attention: block quantisation, then the
attention definition on the quantised values.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP path.

"Training GEM at LLM scale" (Meta engineering post), section "Mixed
Ultra-Low-Precision Training", part "Low Precision Flash Attention": the
attention products run as MXFP8 block-scaled matrix products in the forward
and the backward; every tensor is quantised once, with one scale per square
block of 32 x 32 elements, so that a block and its transpose share the scale
(the backward reads Q, K, dO transposed); the kernel converts P (and, in the
backward, dS) to MXFP8 itself, reusing the row maximum softmax already has.

The pages fix neither the element format, the rounding nor the scale rule.
Readings taken here:
  * elements are FP8 E4M3 in the OCP 8-bit floating point format (bias 7,
    three mantissa bits, subnormals, largest finite value 448, no infinity),
    rounded to nearest, ties to even;
  * a scale is a power of two 2^X stored as the E8M0 byte X + 127 (OCP
    Microscaling Formats (MX) specification v1.0, shared-scale type);
  * X is the smallest integer with amax * 2^-X <= 448 (amax = largest
    magnitude in the block), so no element saturates; amax = 0 gives X = -127;
  * a block covers 32 consecutive rows of one sample (the last block of a
    sample may be shorter) and 32 consecutive features of one head;
  * the attention is then the plain definition (oracle.attention) on the
    dequantised Q, K, V (and dO): P and dS are kept exact here; the kernel's
    own conversion of P and dS to MXFP8 is an approximation whose error the
    parity tests bound element by element (DESIGN readings).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6  # 2^-6
E4M3_MANT_BITS = 3
BLOCK = 32
E8M0_BIAS = 127


# ----------------------------------------------------------------------------
# FP8 E4M3 (OCP): rounding, encoding, decoding
# ----------------------------------------------------------------------------
def e4m3_round(y):
    """Round float64 values with |y| <= 448 to the nearest E4M3 value (ties to
    even).  Spacing: 2^(e-3) for |y| in [2^e, 2^(e+1)), e >= -6; 2^-9 below."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(np.abs(y) > E4M3_MAX):
        raise ValueError("value outside the E4M3 range")
    a = np.abs(y)
    _, e = np.frexp(a)  # a = m 2^e, m in [0.5, 1)  ->  floor(log2 a) = e - 1
    e = np.maximum(e - 1, E4M3_MIN_NORMAL_EXP)
    q = np.ldexp(1.0, e - E4M3_MANT_BITS)  # spacing of the grid at a
    r = np.round(a / q) * q  # numpy rounds half to even; a / q is exact
    return np.copysign(r, y)


def e4m3_encode(y):
    """E4M3 byte codes of values already on the grid (e4m3_round output)."""
    y = np.asarray(y, dtype=np.float64)
    sign = (np.signbit(y)).astype(np.uint8) << 7
    a = np.abs(y)
    out = np.zeros(a.shape, dtype=np.uint8)
    sub = a < 2.0 ** E4M3_MIN_NORMAL_EXP
    # subnormals: value = m 2^-9, m in 0..7, exponent field 0
    out[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.uint8)
    nz = ~sub
    if np.any(nz):
        m, e = np.frexp(a[nz])  # a = (2m) 2^(e-1), 2m in [1, 2)
        field = (e - 1 + 7).astype(np.int64)
        mant = np.rint((2.0 * m - 1.0) * 8.0).astype(np.int64)
        out[nz] = ((field << 3) | mant).astype(np.uint8)
    code = out | sign
    if not np.array_equal(e4m3_decode(code), y):
        raise ValueError("value not on the E4M3 grid")
    return code


def e4m3_decode(code):
    """float64 value of E4M3 byte codes (0x7F / 0xFF are NaN)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    f = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(f == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, f - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


# ----------------------------------------------------------------------------
# shared block scale
# ----------------------------------------------------------------------------
def scale_exponent(amax):
    """Smallest integer X in [-127, 127] with amax * 2^-X <= 448 (-127 for 0).

    With amax = m 2^e (m in [0.5, 1)) and 448 = 0.875 2^9: amax 2^-X <= 448
    holds iff e - X <= 9 when m <= 0.875, and iff e - X <= 8 when m > 0.875."""
    a = np.asarray(amax, dtype=np.float64)
    m, e = np.frexp(a)
    x = e - 9 + (m > 0.875)
    x = np.where(a == 0.0, -E8M0_BIAS, x)
    return np.clip(x, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def row_block_starts(offsets):
    """Index of each sample's first 32-row block in the scale array, [B + 1]."""
    n = np.diff(np.asarray(offsets, dtype=np.int64))
    nb = (n + BLOCK - 1) // BLOCK
    out = np.zeros(len(nb) + 1, dtype=np.int64)
    np.cumsum(nb, out=out[1:])
    return out


def quantize(x, offsets):
    """MXFP8 quantisation of a jagged [T, H, D] tensor in 32 x 32 blocks.

    Returns (codes uint8 [T, H, D], scales uint8 [RB, H, D/32] holding X + 127,
    dequantised values float64 [T, H, D]).  Block (b, r, h, c) holds rows
    offsets[b] + 32r .. (cut at the sample end) and features 32c .. 32c + 31 of
    head h; its scale sits at scales[row_block_starts(offsets)[b] + r, h, c]."""
    x = np.asarray(x, dtype=np.float64)
    T, H, D = x.shape
    if D % BLOCK:
        raise ValueError("D must be a multiple of 32")
    off = np.asarray(offsets, dtype=np.int64)
    rbs = row_block_starts(off)
    codes = np.zeros((T, H, D), dtype=np.uint8)
    deq = np.zeros((T, H, D))
    scales = np.zeros((int(rbs[-1]), H, D // BLOCK), dtype=np.uint8)
    for b in range(len(off) - 1):
        for r in range(int(rbs[b + 1] - rbs[b])):
            r0 = int(off[b]) + BLOCK * r
            r1 = min(r0 + BLOCK, int(off[b + 1]))
            blk = x[r0:r1].reshape(r1 - r0, H, D // BLOCK, BLOCK)  # rows, head, col block, col
            amax = np.max(np.abs(blk), axis=(0, 3))  # [H, D/32]
            X = scale_exponent(amax)
            s = np.ldexp(1.0, X)[None, :, :, None]
            q = e4m3_round(blk / s)  # exact division by a power of two
            codes[r0:r1] = e4m3_encode(q).reshape(r1 - r0, H, D)
            deq[r0:r1] = (q * s).reshape(r1 - r0, H, D)
            scales[int(rbs[b]) + r] = (X + E8M0_BIAS).astype(np.uint8)
    return codes, scales, deq


def transposed(codes):
    """The transposed copy of [T, H, D] codes: [H, D, T] (feature-major per
    head), which serves the products whose reduction runs over tokens."""
    return np.ascontiguousarray(np.transpose(np.asarray(codes), (1, 2, 0)))


def dequantize(codes, scales, offsets):
    """Values of MXFP8 codes with their block scales (inverse of quantize)."""
    codes = np.asarray(codes, dtype=np.uint8)
    T, H, D = codes.shape
    off = np.asarray(offsets, dtype=np.int64)
    rbs = row_block_starts(off)
    v = e4m3_decode(codes)
    out = np.zeros((T, H, D))
    for b in range(len(off) - 1):
        for r in range(int(rbs[b + 1] - rbs[b])):
            r0 = int(off[b]) + BLOCK * r
            r1 = min(r0 + BLOCK, int(off[b + 1]))
            X = scales[int(rbs[b]) + r].astype(np.int64) - E8M0_BIAS  # [H, D/32]
            s = np.repeat(np.ldexp(1.0, X), BLOCK, axis=1)  # [H, D]
            out[r0:r1] = v[r0:r1] * s[None]
    return out
