"""GPU parity of the forward kernels against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

from jagged_variable_length_amd import attention as A
from jagged_variable_length_amd import inputs as gen

pytestmark = pytest.mark.gpu

from gpu_util import check, check_dbias, check_lse, device_inputs, make_op, oracle_bwd, oracle_fwd, say, sync  # noqa: E402
from oracle import attention as ora  # noqa: E402


def _run_fwd(inp, **kw):
    op = make_op(inp, **kw)
    d = device_inputs(inp)
    o, lse = op.forward(d["q"], d["k"], d["v"], bias=d["bias"])
    sync()
    return op, A.to_f64(o), (A.to_f64(lse) if lse is not None else None)


def _compare(inp, op, o, lse):
    ro, rl = oracle_fwd(inp, op)
    check(o, ro, "O")
    if rl is not None and lse is not None:
        check_lse(lse, rl)


def test_fwd_config0_f32():
    say("case: config 0 (fp32, D=32, zero-length sample)")
    inp = gen.make_inputs(0, 0)
    op, o, lse = _run_fwd(inp, out_dtype="f32", grad_dtype="f32")
    _compare(inp, op, o, lse)


@pytest.mark.parametrize("D", [128, 64, 32])
@pytest.mark.parametrize("bias", [False, True])
def test_fwd_softmax_ragged(D, bias):
    say(f"case: softmax ragged D={D} bias={bias}")
    lq = [1, 0, 130, 64, 257, 33, 7, 500]
    lk = [5, 9, 0, 64, 300, 1, 129, 70]
    inp = gen.make_custom(lq, lk, 3, D, "bf16", seed=D + bias, bias=bias)
    op, o, lse = _run_fwd(inp, bias=bias)
    _compare(inp, op, o, lse)


@pytest.mark.parametrize("act", ["gelu", "silu"])
@pytest.mark.parametrize("split", [False, True])
def test_fwd_gdpa(act, split):
    say(f"case: gdpa {act} split={split}")
    lq = [32, 32, 0, 32, 32]
    lk = [64, 300, 50, 0, 1000]
    inp = gen.make_custom(lq, lk, 2, 128, "bf16", seed=5)
    op, o, _ = _run_fwd(inp, act=act, split=split, out_dtype="f32")
    assert op.info.fwd.tile_rows == 32  # short-query shape: key tiles split over waves
    if split:
        _compare(inp, op, o, None)
        return
    # Without the hi/lo split, P enters the PV product rounded to bf16: the
    # error is bounded by u * (|P| |V|) with u = 2^-8 (bf16 unit roundoff).
    ro, _ = oracle_fwd(inp, op)
    q, k, v = inp.f64("q"), inp.f64("k"), inp.f64("v")
    act_fn = {"gelu": ora.gelu, "silu": ora.silu}[act]
    for b in range(inp.B):
        sq = slice(inp.q_offsets[b], inp.q_offsets[b + 1])
        sk = slice(inp.kv_offsets[b], inp.kv_offsets[b + 1])
        for h in range(inp.H):
            P = act_fn(op.scale * q[sq, h] @ k[sk, h].T)
            bound = 2.0 ** -8 * (np.abs(P) @ np.abs(v[sk, h])) + 1e-3
            assert np.all(np.abs(o[sq, h] - ro[sq, h]) <= bound), (b, h)


@pytest.mark.parametrize("D,bias", [(64, True), (128, False)])
def test_fwd_short_query_softmax_split_keys(D, bias):
    """32-row queries: the key tiles are split over the waves and combined."""
    say(f"case: softmax with 32-row queries (key-split combine) D={D} bias={bias}")
    lq = [32, 20, 1, 32]
    lk = [700, 0, 129, 64]
    inp = gen.make_custom(lq, lk, 2, D, "bf16", seed=6, bias=bias)
    op, o, lse = _run_fwd(inp, bias=bias)
    assert op.info.fwd.tile_rows == 32
    _compare(inp, op, o, lse)


def test_fwd_short_query_bias_d128_uses_regular_shape():
    say("case: 32-row queries with bias at D=128 (regular shape)")
    inp = gen.make_custom([32, 20, 32], [700, 9, 64], 2, 128, "bf16", seed=7, bias=True)
    op, o, lse = _run_fwd(inp, bias=True)
    assert op.info.fwd.tile_rows == 256
    _compare(inp, op, o, lse)


def test_fwd_outputs_overwrite_garbage():
    """Zero-length samples are written by the library, not assumed zero."""
    say("case: garbage-filled outputs")
    lq, lk = [3, 10, 0], [0, 4, 5]
    inp = gen.make_custom(lq, lk, 2, 64, "bf16", seed=8)
    op = make_op(inp)
    d = device_inputs(inp)
    o = torch.full((op.Tq, 2, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((op.Tq, 2), 7.0, dtype=torch.float32, device="cuda")
    op.forward(d["q"], d["k"], d["v"], o=o, lse=lse)
    sync()
    _compare(inp, op, A.to_f64(o), A.to_f64(lse))


def test_fwd_deterministic():
    say("case: run-to-run bitwise identical")
    inp = gen.make_custom([300, 17, 900], [250, 1000, 3], 4, 128, "bf16", seed=9, bias=True)
    op = make_op(inp, bias=True)
    d = device_inputs(inp)
    o1, l1 = op.forward(d["q"], d["k"], d["v"], bias=d["bias"])
    o2, l2 = op.forward(d["q"], d["k"], d["v"], bias=d["bias"])
    sync()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("order", ["heavy_first", "lpt"])
def test_fwd_orders_agree(order):
    say(f"case: order {order}")
    inp = gen.make_custom([300, 17, 900, 45], [250, 1000, 3, 64], 2, 64, "bf16", seed=10)
    op1 = make_op(inp)
    op2 = make_op(inp, order=order, num_workers=13)
    d = device_inputs(inp)
    o1, l1 = op1.forward(d["q"], d["k"], d["v"])
    o2, l2 = op2.forward(d["q"], d["k"], d["v"])
    sync()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("lq", [[5, 40, 70], [300, 260, 1]])
def test_fwd_bwd_adversarial_negative_bias(lq):
    """Subtraction scheme near its documented limit: every valid score sits
    around -5.5 (bias -5.5, Q K^T nearly zero) while the zero-filled tail
    keys score 0, so the row sum is n_pad + sum(e^s) - n_pad in fp32.  With at
    most 127 padded keys the cancellation leaves a relative error of about
    ulp(128) / e^-5.5 ~ 2e-3 in P, which dBias (up to ~10 here) carries
    inside the bound; far below that it would not (the limit is stated with
    the scheme's readings).  P and dS enter the
    dV / dK products as hi + lo pairs: with 260 queries on 2 keys, bf16 P
    alone would move dV by ~0.05 (the long-query, few-key shape of the
    cross-attention workload, which runs with split operands too)."""
    say(f"case: adversarial negative bias lq={lq}")
    lk = [1, 2, 31]
    inp = gen.make_custom(lq, lk, 2, 64, "bf16", seed=13, bias=True)
    rng = np.random.default_rng(13)
    inp.q = gen.f32_to_bf16_bits(0.01 * rng.standard_normal(inp.q.shape).astype(np.float32))
    inp.bias = gen.f32_to_bf16_bits((-5.5 + 0.1 * rng.standard_normal(inp.bias.shape)).astype(np.float32))
    op = make_op(inp, bias=True, want_dbias=True, out_dtype="f32", grad_dtype="f32", split=True)
    d = device_inputs(inp)
    o, lse = op.forward(d["q"], d["k"], d["v"], bias=d["bias"])
    dq, dk, dv, db = op.backward(d["q"], d["k"], d["v"], d["dout"], o=o, lse=lse, bias=d["bias"])
    sync()
    ro, rl = oracle_fwd(inp, op)
    check(A.to_f64(o), ro, "O")
    check_lse(A.to_f64(lse), rl)
    rg = oracle_bwd(inp, op)
    for name, g, r in zip(["dQ", "dK", "dV", "dBias"], (dq, dk, dv, db), rg):
        (check_dbias if name == "dBias" else check)(A.to_f64(g), r, name)


@pytest.mark.parametrize("level", [-20.0, -1.0e3, -1.0e4])
@pytest.mark.parametrize("D,lq,dt", [(64, [3, 40, 17, 1, 33, 8], "bf16"), (128, [300, 64, 1, 129, 40, 200], "bf16"),
                                     (64, [300, 64, 1, 129, 40, 200], "bf16"), (64, [3, 40, 17, 1, 33, 8], "f32"),
                                     (32, [300, 64, 1, 129, 40, 200], "f32")])
def test_fwd_bwd_very_negative_bias(level, D, lq, dt):
    """Rows whose every valid score lies far below zero, on samples whose key
    count is not a multiple of 32 (so the last key step holds zero-filled
    keys scoring 0).  Softmax is shift-invariant, so the oracle's result is
    an ordinary attention; the forward must not let the padded keys' exp
    terms swamp the row sum (at -20 the subtraction alone would cancel to a
    wrong sum, at -1e3 the valid terms underflow and it would give NaN): such
    rows drop the padded keys in that step instead of subtracting them.
    At -1e4 only the forward is compared: scores near 1.44e4 (log2 units)
    carry fp32 rounding of about 2^-10 absolute, so the backward's
    P = 2^(x - LSE2) errs by about 7e-4 relative, which dV sums over up to
    300 queries to about 0.03 (the precision of fp32 scores at that
    magnitude, not of the tail handling)."""
    say(f"case: very negative bias {level} D={D} lq={lq} {dt}")
    lk = [1, 45, 31, 100, 33, 70]
    inp = gen.make_custom(lq, lk, 2, D, dt, seed=29, bias=True)
    rng = np.random.default_rng(29)
    b = (level + 0.25 * rng.standard_normal(inp.bias.shape)).astype(np.float32)
    inp.bias = gen.f32_to_bf16_bits(b) if dt == "bf16" else b
    op = make_op(inp, bias=True, want_dbias=True, out_dtype="f32", grad_dtype="f32", split=True)
    d = device_inputs(inp)
    o, lse = op.forward(d["q"], d["k"], d["v"], bias=d["bias"])
    dq, dk, dv, db = op.backward(d["q"], d["k"], d["v"], d["dout"], o=o, lse=lse, bias=d["bias"])
    sync()
    ro, rl = oracle_fwd(inp, op)
    check(A.to_f64(o), ro, "O")
    check_lse(A.to_f64(lse), rl)
    for x in (dq, dk, dv, db):
        assert torch.isfinite(x).all()
    if level < -5e3:
        return
    rg = oracle_bwd(inp, op)
    for name, g, r in zip(["dQ", "dK", "dV", "dBias"], (dq, dk, dv, db), rg):
        (check_dbias if name == "dBias" else check)(A.to_f64(g), r, name)
