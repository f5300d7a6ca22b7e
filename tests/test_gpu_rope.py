"""GPU parity of BlockAttention with the fused rotary embedding against the
fp64 oracle (RoPE of Q and K, block-diagonal attention, transposed rotation
of dQ and dK).

"Training GEM at LLM scale", section "BlockAttention": the RoPE backward is
fused into the block-attention epilogue.  Positions are token indices inside
each sample, so long samples reach large angles (the kernels reduce them in
fp64)."""
import numpy as np
import pytest
import torch

from jagged_variable_length_amd import attention as A
from jagged_variable_length_amd import inputs as gen
from oracle import attention as ora
from oracle import batched as bat
from oracle import rope

pytestmark = pytest.mark.gpu

from gpu_util import check, check_full, device_inputs, say, sync  # noqa: E402


def _run(inp, D, out, grad, base=0.0):
    op = A.JaggedAttention(inp.q_offsets, inp.kv_offsets, inp.H, D, block_diagonal=True, out_dtype=out,
                           grad_dtype=grad, rope=True, rope_base=base).upload()
    d = device_inputs(inp)
    o, _ = op.forward(d["q"], d["k"], d["v"])
    dq, dk, dv, _ = op.backward(d["q"], d["k"], d["v"], d["dout"])
    sync()
    return op, [A.to_f64(t) for t in (o, dq, dk, dv)]


def _oracle(inp, op, base):
    off = inp.q_offsets
    b = base if base > 0 else rope.BASE
    qr, kr = rope.forward(inp.f64("q"), off, b), rope.forward(inp.f64("k"), off, b)
    o, _ = ora.forward(qr, kr, inp.f64("v"), off, off, scale=op.scale, block_diagonal=True)
    dqr, dkr, dv, _ = ora.backward(qr, kr, inp.f64("v"), inp.f64("dout"), off, off, scale=op.scale,
                                   block_diagonal=True)
    return o, rope.backward(dqr, off, b), rope.backward(dkr, off, b), dv


@pytest.mark.parametrize("D", [128, 64, 32])
@pytest.mark.parametrize("out,grad", [("bf16", "bf16"), ("f32", "f32")])
def test_block_rope(D, out, grad):
    say(f"case: block + RoPE D={D} out={out} grad={grad}")
    L = [200, 0, 64, 3, 1, 130, 1000]
    inp = gen.make_custom(L, L, 2, D, "bf16", seed=D)
    op, got = _run(inp, D, out, grad)
    for name, g, r in zip(("O", "dQ", "dK", "dV"), got, _oracle(inp, op, 0.0)):
        check(g, r, name)


def _block_oracle(inp, b, t, D, scale, base=rope.BASE):
    """Oracle for block t of sample b as its own 64-row problem at its true
    positions (block-diagonal attention equals its blocks run alone)."""
    L = int(inp.lq[b])
    r0 = int(inp.q_offsets[b]) + 64 * t
    r1 = int(inp.q_offsets[b]) + min(L, 64 * t + 64)
    q, k, v, do = [gen.to_f64(x[r0:r1], "bf16") for x in (inp.q, inp.k, inp.v, inp.dout)]
    ang = rope.angles(np.arange(64 * t, 64 * t + (r1 - r0)), D, base)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    h = D // 2

    def rot(x):
        return np.concatenate([x[..., :h] * c - x[..., h:] * s, x[..., h:] * c + x[..., :h] * s], -1)

    def rot_t(x):
        return np.concatenate([x[..., :h] * c + x[..., h:] * s, x[..., h:] * c - x[..., :h] * s], -1)

    off = np.array([0, r1 - r0])
    ro, _ = ora.forward(rot(q), rot(k), v, off, off, scale=scale)
    rg = ora.backward(rot(q), rot(k), v, do, off, off, scale=scale)
    return slice(r0, r1), (ro, rot_t(rg[0]), rot_t(rg[1]), rg[2])


def test_block_rope_base_and_long_positions():
    """A small base (fast-turning pairs) and a sample long enough for
    positions beyond 16k; its first and last blocks are checked."""
    say("case: block + RoPE, base 500, a 17000-token sample")
    L = [17000, 65]
    inp = gen.make_custom(L, L, 1, 64, "bf16", seed=11)
    op, got = _run(inp, 64, "f32", "f32", base=500.0)
    for b, t in ((0, 0), (0, 17000 // 64 - 1), (0, 17000 // 64), (1, 1)):
        rows, ref = _block_oracle(inp, b, t, 64, op.scale, 500.0)
        for name, g, r in zip(("O", "dQ", "dK", "dV"), got, ref):
            check(g[rows], r, name)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_block_rope_workload_full_size():
    """Full-size workload in the benchmark's configuration, every element:
    the oracle rotates Q and K at their true positions, runs every 64-token
    block as its own problem (oracle.batched, pinned on the CPU) and rotates
    dQ and dK back."""
    cfg = 7
    w = gen.WORKLOADS[cfg]
    say(f"case: workload {cfg} ({w.name}) full size, every element")
    inp = gen.make_inputs(cfg, cfg)
    op = A.JaggedAttention(inp.q_offsets, inp.kv_offsets, w.H, w.D, block_diagonal=True, out_dtype=w.out_dtype,
                           grad_dtype=w.grad_dtype, rope=True).upload()
    d = {n: A.to_device(getattr(inp, n), w.dtype) for n in ("q", "k", "v", "dout")}
    outs = []
    for _ in range(2):
        o, _ = op.forward(d["q"], d["k"], d["v"])
        outs.append((o,) + op.backward(d["q"], d["k"], d["v"], d["dout"])[:3])
    sync()
    for a_, b_ in zip(*outs):
        assert torch.isfinite(a_).all()
        assert torch.equal(a_, b_)
    got = [A.to_f64(t) for t in outs[0]]
    del outs, d
    off = inp.q_offsets
    qr, kr = rope.forward(inp.f64("q"), off), rope.forward(inp.f64("k"), off)
    v, do = inp.f64("v"), inp.f64("dout")
    ro, _ = bat.forward(qr, kr, v, off, off, scale=op.scale, block_diagonal=True)
    check_full(got[0], ro, "O", off)
    del ro
    dqr, dkr, dv, _ = bat.backward(qr, kr, v, do, off, off, scale=op.scale, block_diagonal=True)
    check_full(got[1], rope.backward(dqr, off), "dQ", off)
    check_full(got[2], rope.backward(dkr, off), "dK", off)
    check_full(got[3], dv, "dV", off)
