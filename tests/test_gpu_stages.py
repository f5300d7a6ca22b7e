"""The backward's stage contract through jattn_bwd_stages (softmax, bf16 inputs).

Where dQ forms Di and LSE * log2(e) itself (bf16 O; fp32 O below D = 128):
the stages called one at a time in the library's own order (DQ, then DKDV)
reproduce jattn_bwd bit for bit, DQ alone needs no Di pass, and a Di pass
followed by DKDV and DQ (three calls) stays within the parity bound against
the fp64 oracle.  Where Di keeps a pass of its own (D = 128 with fp32 O):
PREP, DKDV, DQ in three calls reproduce jattn_bwd bit for bit, and match the
oracle.  Every output starts as NaN, so a stage that skips its writes fails.

The lengths include a one-key sample (P = 1, so dS = dP - Di takes Di's
error undamped); with bf16 O at D = 128 the rounding of the stored O alone
moves Di by about 2^-9 sqrt(D) |O| |dO| against the oracle's exact O, which
puts that sample's dBias error near 1.9e-2, inside the bound.
"""
import numpy as np
import pytest
import torch

from jagged_variable_length_amd import attention as A
from jagged_variable_length_amd import binding as B
from jagged_variable_length_amd import inputs as gen

pytestmark = pytest.mark.gpu

from gpu_util import check, check_dbias, device_inputs, make_op, oracle_bwd, say, sync  # noqa: E402

LQ = [1, 0, 130, 64, 257, 33, 7, 500]
LK = [5, 9, 0, 64, 300, 1, 129, 70]


def _nan_like(op, rows, dtype):
    return torch.full((rows, op.H, op.D), float("nan"), dtype=dtype, device="cuda")


def _backward(op, d, o, lse, stages):
    """Run the backward as the given sequence of stage masks, into NaN-filled outputs."""
    gdt = A._TORCH_DT[op.grad_dtype]
    dq, dk, dv = _nan_like(op, op.Tq, gdt), _nan_like(op, op.Tk, gdt), _nan_like(op, op.Tk, gdt)
    db = None
    if op.want_dbias:
        db = torch.full((int(op.info.bias_elems),), float("nan"), dtype=A._TORCH_DT[op.dbias_dtype], device="cuda")
    for st in stages:
        op.backward(d["q"], d["k"], d["v"], d["dout"], o=o, lse=lse, bias=d["bias"], dq=dq, dk=dk, dv=dv,
                    dbias=db, stages=st)
    sync()
    return dq, dk, dv, db


def _setup(D, out_dtype, bias, seed):
    inp = gen.make_custom(LQ, LK, 3, D, "bf16", seed=seed, bias=bias)
    op = make_op(inp, bias=bias, want_dbias=bias, out_dtype=out_dtype, grad_dtype="f32", dbias_dtype="f32")
    d = device_inputs(inp)
    o, lse = op.forward(d["q"], d["k"], d["v"], bias=d["bias"])
    sync()
    return inp, op, d, o, lse


def _same(a, b, name):
    if a is None:
        return
    assert not torch.isnan(a).any(), f"{name}: unwritten (NaN) elements"
    assert torch.equal(a, b), f"{name}: differs from jattn_bwd"


def _vs_oracle(inp, op, got):
    ref = oracle_bwd(inp, op)
    for name, g, r in zip(["dQ", "dK", "dV", "dBias"], got, ref):
        if r is None:
            continue
        (check_dbias if name == "dBias" else check)(A.to_f64(g), r, name)


@pytest.mark.parametrize("D,out_dtype,bias", [(128, "bf16", True), (64, "f32", False), (64, "bf16", True)])
def test_stages_with_rowstats_in_dq(D, out_dtype, bias):
    say(f"case: stages, Di formed in dQ, D={D} O={out_dtype} bias={bias}")
    inp, op, d, o, lse = _setup(D, out_dtype, bias, seed=D + bias)
    whole = _backward(op, d, o, lse, [B.JATTN_BWD_ALL])
    for name, a, b in zip(["dQ", "dK", "dV", "dBias"], _backward(op, d, o, lse, [B.JATTN_BWD_DQ, B.JATTN_BWD_DKDV]),
                          whole):
        _same(a, b, name + " (DQ then DKDV)")
    # DQ alone forms its own row statistics
    dq_alone = _backward(op, d, o, lse, [B.JATTN_BWD_DQ])[0]
    _same(dq_alone, whole[0], "dQ (DQ alone)")
    # a Di pass, then DKDV and DQ in separate calls
    three = _backward(op, d, o, lse, [B.JATTN_BWD_PREP, B.JATTN_BWD_DKDV, B.JATTN_BWD_DQ])
    _same(three[0], whole[0], "dQ (PREP, DKDV, DQ)")
    _vs_oracle(inp, op, three)


def test_stages_with_a_di_pass():
    """D = 128 with fp32 O keeps the separate Di pass."""
    say("case: stages, separate Di pass, D=128 O=f32 bias=True")
    inp, op, d, o, lse = _setup(128, "f32", True, seed=7)
    whole = _backward(op, d, o, lse, [B.JATTN_BWD_ALL])
    three = _backward(op, d, o, lse, [B.JATTN_BWD_PREP, B.JATTN_BWD_DKDV, B.JATTN_BWD_DQ])
    for name, a, b in zip(["dQ", "dK", "dV", "dBias"], three, whole):
        _same(a, b, name + " (PREP, DKDV, DQ)")
    _vs_oracle(inp, op, whole)
