"""GPU parity of sliding-window attention (forward, dQ, dK/dV) against the
fp64 oracle.

"Training GEM at LLM scale", section "BlockAttention": the sliding-window
kernel visits only the tiles that meet the window.  Query i of a sample sees
keys i - left .. i + right.  Lengths below span several 128-row tiles with
ragged tails; windows cover the degenerate cases (each token alone, causal,
anti-causal, wider than every sample) and windows that end inside a tile.
"""
import numpy as np
import pytest
import torch

from jagged_variable_length_amd import attention as A
from jagged_variable_length_amd import inputs as gen
from oracle import attention as ora
from oracle import batched as bat

pytestmark = pytest.mark.gpu

from gpu_util import check, check_full, check_lse, device_inputs, make_op, oracle_bwd, oracle_fwd, say, sync  # noqa: E402

BIG = 1 << 30
LENGTHS = [1, 0, 130, 64, 257, 33, 500, 129, 2]
WINDOWS = [(0, 0), (5, 130), (200, 0), (63, 64), (0, BIG), (BIG, BIG), (31, 1)]


def _run(inp, **kw):
    op = make_op(inp, **kw)
    d = device_inputs(inp)
    o, lse = op.forward(d["q"], d["k"], d["v"], bias=d["bias"])
    dq, dk, dv, _ = op.backward(d["q"], d["k"], d["v"], d["dout"], o=o, lse=lse, bias=d["bias"])
    sync()
    return op, A.to_f64(o), (A.to_f64(lse) if lse is not None else None), [A.to_f64(x) for x in (dq, dk, dv)]


def _compare(inp, op, o, lse, grads):
    ro, rl = oracle_fwd(inp, op)
    check(o, ro, "O")
    if rl is not None:
        check_lse(lse, rl)
    rg = oracle_bwd(inp, op)
    for name, g, r in zip(["dQ", "dK", "dV"], grads, rg[:3]):
        check(g, r, name)


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("D", [128, 64, 32])
def test_window_softmax(D, window):
    bias = window[0] % 2 == 1  # the odd-left windows also carry a bias
    say(f"case: window softmax D={D} window={window} bias={bias}")
    inp = gen.make_custom(LENGTHS, LENGTHS, 2, D, "bf16", seed=D + window[0] % 97, bias=bias)
    op, o, lse, grads = _run(inp, bias=bias, window=window, grad_dtype="f32")
    assert op.info.fwd.tile_rows == 128 and op.info.dkdv.tile_rows == 128
    _compare(inp, op, o, lse, grads)


@pytest.mark.parametrize("window", [(0, 0), (63, 64), (200, 0), (BIG, BIG)])
@pytest.mark.parametrize("act", ["gelu", "silu"])
@pytest.mark.parametrize("bias", [False, True])
def test_window_gdpa(act, window, bias):
    say(f"case: window {act} window={window} bias={bias}")
    inp = gen.make_custom(LENGTHS, LENGTHS, 2, 128, "bf16", seed=7 + window[0] % 89, bias=bias)
    op, o, lse, grads = _run(inp, act=act, bias=bias, window=window, split=True, out_dtype="f32",
                             grad_dtype="f32")
    assert lse is None
    _compare(inp, op, o, lse, grads)


def test_window_bf16_outputs_and_run_to_run():
    say("case: window bf16 outputs, run-to-run identical")
    inp = gen.make_custom(LENGTHS, LENGTHS, 3, 128, "bf16", seed=3)
    op = make_op(inp, window=(100, 27))
    d = device_inputs(inp)
    outs = []
    for _ in range(2):
        o, lse = op.forward(d["q"], d["k"], d["v"])
        outs.append((o, lse) + op.backward(d["q"], d["k"], d["v"], d["dout"], o=o, lse=lse)[:3])
    sync()
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    o, lse, dq, dk, dv = [A.to_f64(x) for x in outs[0]]
    _compare(inp, op, o, lse, [dq, dk, dv])


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_window_workload_full_size():
    """Long-sequence sliding-window workload at full size, in the launch
    configuration the benchmark times: every element against the oracle,
    evaluated in chunks of 64 query rows with the keys their windows reach
    (oracle.batched; pinned against the per-sample oracle on the CPU)."""
    cfg = 5
    w = gen.WORKLOADS[cfg]
    say(f"case: workload {cfg} ({w.name}) full size, every element")
    inp = gen.make_inputs(cfg, cfg)
    op = A.JaggedAttention(inp.q_offsets, inp.kv_offsets, w.H, w.D, act=w.act, in_dtype=w.dtype,
                           out_dtype=w.out_dtype, grad_dtype=w.grad_dtype, window=w.window).upload()
    d = {n: A.to_device(getattr(inp, n), w.dtype) for n in ("q", "k", "v", "dout")}
    o, lse = op.forward(d["q"], d["k"], d["v"])
    dq, dk, dv, _ = op.backward(d["q"], d["k"], d["v"], d["dout"], o=o, lse=lse)
    sync()
    got = [A.to_f64(x) for x in (o, lse, dq, dk, dv)]
    del d, o, lse, dq, dk, dv
    q, k, v, do = inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("dout")
    kw = dict(scale=op.scale, window=w.window)
    ro, rl = bat.forward(q, k, v, inp.q_offsets, inp.kv_offsets, **kw)
    check_full(got[0], ro, "O", inp.q_offsets)
    check_full(got[1], rl, "lse", inp.q_offsets)
    del ro, rl
    rg = bat.backward(q, k, v, do, inp.q_offsets, inp.kv_offsets, **kw)
    for name, g, r in zip(("dQ", "dK", "dV"), got[2:], rg):
        check_full(g, r, name, inp.q_offsets)
