"""GPU parity of the bias path at every 2-byte alignment of the bias rows.

The kernels move bias rows HBM -> LDS as 16-byte loads at the rows' own
(2-byte) alignment and mask keys past a row's end.  These cases place the
bias tensor at element offsets 0..3 of an allocation, use odd key counts (so
consecutive rows alternate in alignment), and end the tensor with a sample
whose key count is odd: its last element then shares a dword with the two
bytes past the tensor end, which the kernels reload on their own.  Every
tile shape of the three kernels meets these rows (short-query forward/dQ,
64-key forward/dQ steps, 32/64/128-key dK/dV units)."""
import numpy as np
import pytest
import torch

from jagged_variable_length_amd import attention as A
from jagged_variable_length_amd import inputs as gen

pytestmark = pytest.mark.gpu

from gpu_util import check, check_dbias, check_lse, device_inputs, make_op, oracle_bwd, oracle_fwd, say, sync  # noqa: E402

CASES = {
    # long rows, several query tiles, odd lk everywhere, odd last lk
    "long": ([3, 130, 67, 1, 200], [7, 65, 129, 33, 131]),
    # short keys (32/64-key dK/dV units), odd last lk
    "short_keys": ([40, 300, 9, 77], [17, 31, 1, 45]),
    # short queries (key-split forward/dQ shape), odd last lk
    "short_queries": ([32, 32, 17, 32], [301, 63, 5, 257]),
}


def _shifted(t: torch.Tensor, offset: int) -> torch.Tensor:
    """Copy of t starting `offset` elements into a fresh allocation."""
    base = torch.full((t.numel() + offset + 8,), float("nan"), dtype=t.dtype, device=t.device)
    view = base[offset:offset + t.numel()]
    view.copy_(t)
    return view


@pytest.mark.parametrize("offset", [0, 1, 2, 3])
@pytest.mark.parametrize("case", sorted(CASES))
def test_bias_alignment_fwd_bwd(case, offset):
    lq, lk = CASES[case]
    say(f"case: bias layout {case} offset={offset} lq={lq} lk={lk}")
    inp = gen.make_custom(lq, lk, 2, 128, "bf16", seed=17 + offset, bias=True)
    # O in fp32: with few keys P is nearly one-hot and dBias = P (dP - Di)
    # inherits the bf16 rounding of a stored O through Di undamped; this
    # test is about where bias values land, not about that rounding
    op = make_op(inp, bias=True, want_dbias=True, out_dtype="f32", grad_dtype="f32", dbias_dtype="f32")
    d = device_inputs(inp)
    bias = _shifted(d["bias"], offset)
    assert bias.data_ptr() % 16 == (d["bias"].data_ptr() + 2 * offset) % 16
    o, lse = op.forward(d["q"], d["k"], d["v"], bias=bias)
    dq, dk, dv, db = op.backward(d["q"], d["k"], d["v"], d["dout"], o=o, lse=lse, bias=bias)
    sync()
    ro, rl = oracle_fwd(inp, op)
    check(A.to_f64(o), ro, "O")
    check_lse(A.to_f64(lse), rl)
    ref = oracle_bwd(inp, op)
    for name, g, r in zip(["dQ", "dK", "dV", "dBias"], (dq, dk, dv, db), ref):
        (check_dbias if name == "dBias" else check)(A.to_f64(g), r, name)


def test_bias_last_element_matters():
    """The final bias element alone decides a visible difference: with a large
    value on the last key of the last query row, that row's softmax is close
    to one-hot, so O of the row is the last V row and dV of the last key gets
    that row's dO in full.  Reading the element as zero would miss both."""
    lq, lk = [5, 3], [9, 7]
    inp = gen.make_custom(lq, lk, 1, 64, "bf16", seed=3, bias=True)
    inp.bias[-1] = gen.f32_to_bf16_bits(np.array([30.0], dtype=np.float32))[0]
    op = make_op(inp, bias=True, want_dbias=True, out_dtype="f32", grad_dtype="f32", dbias_dtype="f32")
    d = device_inputs(inp)
    ro, _ = oracle_fwd(inp, op)
    ref = oracle_bwd(inp, op)
    assert np.max(np.abs(ro[-1] - gen.to_f64(inp.v[-1], "bf16"))) < 1e-3  # the pin: one-hot row
    for offset in (0, 1):
        say(f"  offset {offset}")
        b = _shifted(d["bias"], offset)
        o, lse = op.forward(d["q"], d["k"], d["v"], bias=b)
        dq, dk, dv, db = op.backward(d["q"], d["k"], d["v"], d["dout"], o=o, lse=lse, bias=b)
        sync()
        check(A.to_f64(o), ro, "O")
        for name, g, r in zip(["dQ", "dK", "dV", "dBias"], (dq, dk, dv, db), ref):
            (check_dbias if name == "dBias" else check)(A.to_f64(g), r, name)
