"""Pins of the MXFP8 oracle (oracle/mxfp8.py) against things other than itself.

* E4M3 rounding equals torch's own float8_e4m3fn conversion (a library route
  with the OCP format) on values across the whole range, including ties,
  subnormals and the largest finite value.
* Code points fixed by the OCP 8-bit floating point format: 1.0 = 0x38,
  448 = 0x7E (largest finite), 2^-6 = 0x08 (smallest normal), 2^-9 = 0x01
  (smallest subnormal), -2.0 = 0xC0, 0x7F is NaN; every finite code decodes
  and re-encodes to itself.
* The shared scale is the smallest power of two that keeps the block within
  448 (checked by brute force over neighbouring exponents).
* Quantisation: the block grid is square, so quantising a sample's [l, D]
  slab and transposing equals quantising its transpose ("Training GEM at LLM
  scale", section "Mixed Ultra-Low-Precision Training": a block and its
  transpose share one scale, each tensor is quantised once); values already
  on a block's grid come back exactly; the error of any element is within
  half a grid step; a block's scale depends only on its own elements; zero
  and partial blocks; dequantize inverts quantize.
* A planted mistake (the scale one power too small) fails the range pin.
"""
import numpy as np
import pytest
import torch

from oracle import mxfp8 as mx


def test_e4m3_round_matches_torch_float8():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000),
        # exact ties between neighbouring grid values, normal and subnormal
        (np.arange(1, 200) + 0.5) * 2.0 ** -9,
        (8 + np.arange(8) + 0.5) * 2.0 ** -3,
        np.array([448.0, -448.0, 2.0 ** -6, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 0.0]),
    ])
    vals = vals[np.abs(vals) <= 448.0]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(mx.e4m3_round(vals), ref)


def test_e4m3_code_points():
    table = {1.0: 0x38, 448.0: 0x7E, 2.0 ** -6: 0x08, 2.0 ** -9: 0x01, -2.0: 0xC0, 0.0: 0x00, 0.5: 0x30,
             240.0: 0x77}
    for v, c in table.items():
        assert int(mx.e4m3_encode(np.array([v]))[0]) == c, (v, hex(c))
        assert float(mx.e4m3_decode(np.array([c]))[0]) == v
    assert np.isnan(mx.e4m3_decode(np.array([0x7F, 0xFF]))).all()
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = mx.e4m3_decode(codes)
    back = mx.e4m3_encode(vals)
    # +0 and -0 both decode to 0; every other code comes back itself
    same = back == codes
    assert np.all(same | (codes == 0x80))
    # and the codes enumerate 253 distinct values in order of magnitude
    assert len(np.unique(vals)) == 253


def test_scale_exponent_is_the_smallest_power_that_fits():
    rng = np.random.default_rng(1)
    amax = np.concatenate([np.abs(rng.standard_normal(5000)) * 2.0 ** rng.integers(-30, 30, 5000),
                           [448.0, 449.0, 447.0, 224.0, 896.0, 1.0, 2.0 ** -200]])
    X = mx.scale_exponent(amax)
    assert np.all(amax * np.ldexp(1.0, -X) <= 448.0)
    free = X > -127  # not clamped at the bottom of the E8M0 range
    assert np.all(amax[free] * np.ldexp(1.0, -(X[free] - 1)) > 448.0)
    assert X[-1] == -127  # 2^-200 needs less than the smallest scale
    assert mx.scale_exponent(np.array([448.0]))[0] == 0
    assert mx.scale_exponent(np.array([449.0]))[0] == 1
    assert mx.scale_exponent(np.array([0.0]))[0] == -127


def test_planted_scale_mistake_is_caught():
    """A scale one power of two too small leaves the largest element above 448."""
    amax = np.array([3.7, 100.0, 0.01])
    X = mx.scale_exponent(amax) - 1
    assert np.any(amax * np.ldexp(1.0, -X) > 448.0)


def _slab(l, D, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((l, 1, D)) * np.exp(rng.standard_normal((l, 1, 1)))).astype(np.float32).astype(
        np.float64)


@pytest.mark.parametrize("l", [32, 64, 77, 5])
def test_quantization_is_transpose_invariant(l):
    D = 64 if l != 5 else 32
    x = _slab(l, D, l)
    off = np.array([0, l])
    c, s, deq = mx.quantize(x, off)
    # the transposed slab: D rows, l features (pad the features to a multiple of 32)
    lp = (l + 31) // 32 * 32
    xt = np.zeros((D, 1, lp))
    xt[:, 0, :l] = x[:, 0, :].T
    ct, st, deqt = mx.quantize(xt, np.array([0, D]))
    np.testing.assert_array_equal(deqt[:, 0, :l], deq[:, 0, :].T)
    np.testing.assert_array_equal(ct[:, 0, :l], c[:, 0, :].T)
    # scales: block (r, c) of x is block (c, r) of its transpose
    np.testing.assert_array_equal(st[:, 0, :], s[:, 0, :].T)
    np.testing.assert_array_equal(mx.transposed(c)[0], c[:, 0, :].T)


def test_exact_on_representable_inputs():
    rng = np.random.default_rng(3)
    l, H, D = 70, 2, 64
    off = np.array([0, 40, 70])
    codes = rng.integers(0, 126, (l, H, D)).astype(np.uint8) | (rng.integers(0, 2, (l, H, D)) << 7).astype(np.uint8)
    vals = mx.e4m3_decode(codes)
    # give every block one element at 448 (so its scale is exactly 2^X) and a power-of-two factor
    x = np.zeros_like(vals)
    rbs = mx.row_block_starts(off)
    for b in range(2):
        for r in range(int(rbs[b + 1] - rbs[b])):
            r0 = off[b] + 32 * r
            r1 = min(r0 + 32, off[b + 1])
            for h in range(H):
                for c in range(D // 32):
                    blk = vals[r0:r1, h, 32 * c:32 * c + 32].copy()
                    blk[0, 0] = 448.0
                    x[r0:r1, h, 32 * c:32 * c + 32] = blk * 2.0 ** int(rng.integers(-20, 20))
    _, _, deq = mx.quantize(x, off)
    np.testing.assert_array_equal(deq, x)


def test_error_within_half_a_grid_step_and_dequantize_inverts():
    rng = np.random.default_rng(4)
    lens = [1, 0, 33, 64, 100]
    off = np.concatenate([[0], np.cumsum(lens)])
    H, D = 3, 96
    x = rng.standard_normal((off[-1], H, D)) * np.exp(2 * rng.standard_normal((off[-1], H, 1)))
    x[5] = 0.0  # a zero row inside a block
    c, s, deq = mx.quantize(x, off)
    np.testing.assert_array_equal(mx.dequantize(c, s, off), deq)
    rbs = mx.row_block_starts(off)
    for b in range(len(lens)):
        for r in range(int(rbs[b + 1] - rbs[b])):
            r0 = off[b] + 32 * r
            r1 = min(r0 + 32, off[b + 1])
            X = s[rbs[b] + r].astype(np.int64) - 127  # [H, D/32]
            step = np.repeat(np.ldexp(1.0, X), 32, axis=1)[None]  # 2^X per column
            a = np.abs(x[r0:r1]) / step  # element on the code scale
            _, e = np.frexp(a)
            ulp = np.ldexp(1.0, np.maximum(e - 1, -6) - 3) * step
            assert np.all(np.abs(deq[r0:r1] - x[r0:r1]) <= 0.5 * ulp + 1e-300)
            # the block's largest element maps into (224, 448]
            amax = np.max(np.abs(x[r0:r1]).reshape(r1 - r0, H, D // 32, 32), axis=(0, 3))
            live = amax > 0
            ratio = amax / np.ldexp(1.0, X)
            assert np.all((ratio[live] > 224.0) & (ratio[live] <= 448.0))


def test_block_scale_depends_only_on_its_block():
    x = _slab(64, 64, 9)
    off = np.array([0, 64])
    _, s0, _ = mx.quantize(x, off)
    y = x.copy()
    y[40, 0, 50] = 1e6  # block (row block 1, column block 1)
    _, s1, _ = mx.quantize(y, off)
    changed = s0 != s1
    assert changed[1, 0, 1] and changed.sum() == 1
