"""The dBias comparison of the GPU tests catches a misplaced value that the
2e-2 max-abs bound alone would accept (CPU only; the mistake is planted in
oracle output)."""
import numpy as np
import pytest

from jagged_variable_length_amd import inputs as gen
from oracle import attention as ora

from gpu_util import check_dbias


def _long_sample_dbias():
    # one sample with many keys and flat scores: P is close to 1 / lk, and so
    # is every dBias = P (dP - Di) element
    inp = gen.make_custom([40], [6000], 1, 32, "bf16", seed=3, bias=True)
    g = ora.backward(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("dout"), inp.q_offsets, inp.kv_offsets,
                     scale=0.02, bias=inp.f64("bias"), want_dbias=True)
    return g[3]


def test_dbias_check_accepts_rounding():
    ref = _long_sample_dbias()
    assert np.max(np.abs(ref)) < 2e-2  # the absolute bound alone is vacuous here
    noisy = ref * (1 + 2.0 ** -8 * np.random.default_rng(0).standard_normal(ref.shape))
    check_dbias(noisy, ref)


@pytest.mark.parametrize("shift", [1, 6000])  # next key; next query row
def test_dbias_check_rejects_misplaced_values(shift):
    ref = _long_sample_dbias()
    planted = np.roll(ref, shift)
    assert np.max(np.abs(planted - ref)) < 2e-2  # within the absolute bound
    with pytest.raises(AssertionError):
        check_dbias(planted, ref)
