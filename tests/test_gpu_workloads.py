"""Full-size workloads, in the launch configuration bench.py times (default
plan and workers): every element of every output and gradient against the
fp64 oracle, plus properties that hold at any size (finite everywhere,
bitwise run-to-run identical).  The oracle side is oracle.batched, the
stacked evaluation of the same definition, pinned against the per-sample
oracle on the CPU (tests/test_oracle_batched.py)."""
import numpy as np
import pytest
import torch

from jagged_variable_length_amd import attention as A
from jagged_variable_length_amd import inputs as gen
from oracle import attention as ora
from oracle import batched as bat

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]

from gpu_util import TOL, check, check_dbias, check_full, say  # noqa: E402


def _setup(cfg):
    w = gen.WORKLOADS[cfg]
    inp = gen.make_inputs(cfg)  # canonical seed of the workload
    op = A.JaggedAttention(inp.q_offsets, inp.kv_offsets, w.H, w.D, act=w.act, block_diagonal=w.block_diagonal,
                           has_bias=w.bias, want_dbias=w.want_dbias, in_dtype=w.dtype, out_dtype=w.out_dtype,
                           grad_dtype=w.grad_dtype, split_operands=w.split_operands,
                           dbias_dtype=w.dbias_dtype).upload()
    d = {n: A.to_device(getattr(inp, n), w.dtype) for n in ("q", "k", "v", "dout")}
    d["bias"] = A.to_device(inp.bias, w.dtype) if inp.bias is not None else None
    return w, inp, op, d


def _run(op, d):
    o, lse = op.forward(d["q"], d["k"], d["v"], bias=d["bias"])
    dq, dk, dv, db = op.backward(d["q"], d["k"], d["v"], d["dout"], o=o, lse=lse, bias=d["bias"])
    return o, lse, dq, dk, dv, db


def _run_twice(op, d):
    outs = _run(op, d)
    outs2 = _run(op, d)
    torch.cuda.synchronize()
    for a, b in zip(outs, outs2):
        if a is not None:
            assert torch.isfinite(a).all()
            assert torch.equal(a, b), "not run-to-run identical"
    return [A.to_f64(x) if x is not None else None for x in outs]


@pytest.mark.parametrize("cfg", [1, 2, 3, 8, 4])
def test_workload_full_size_every_element(cfg):
    w, inp, op, d = _setup(cfg)
    say(f"case: workload {cfg} ({w.name}) full size, every element")
    o, lse, dq, dk, dv, db = _run_twice(op, d)
    del d
    q, k, v, do, bias = inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("dout"), inp.f64("bias")
    kw = dict(scale=op.scale, activation=w.act, block_diagonal=w.block_diagonal, bias=bias)
    ro, rl = bat.forward(q, k, v, inp.q_offsets, inp.kv_offsets, **kw)
    check_full(o, ro, "O", inp.q_offsets)
    if rl is not None and lse is not None:
        check_full(lse, rl, "lse", inp.q_offsets)
    del ro, rl
    rg = bat.backward(q, k, v, do, inp.q_offsets, inp.kv_offsets, want_dbias=w.want_dbias, **kw)
    check_full(dq, rg[0], "dQ", inp.q_offsets)
    check_full(dk, rg[1], "dK", inp.kv_offsets)
    check_full(dv, rg[2], "dV", inp.kv_offsets)
    if w.want_dbias:
        st = ora.bias_starts(inp.lq, inp.lk, w.H)
        check_full(db, rg[3], "dBias", st, unit="element")
        # dBias against its own scale, sample by sample (elements shrink with
        # the number of keys, where the absolute bound alone is loose)
        ratio = []
        for b in range(inp.B):
            g, r = db[st[b]:st[b + 1]], rg[3][st[b]:st[b + 1]]
            ratio.append(float(np.max(np.abs(g - r)) / (np.max(np.abs(r)) + 1e-30)) if r.size else 0.0)
        worst = int(np.argmax(ratio))
        say(f"  dBias relative to its sample's own scale: worst sample {worst} ({ratio[worst]:.3e})")
        check_dbias(db[st[worst]:st[worst + 1]], rg[3][st[worst]:st[worst + 1]])


def test_tiny_workload_full():
    say("case: workload 0 (all of it)")
    w, inp, op, d = _setup(0)
    o, lse, dq, dk, dv, _ = [A.to_f64(x) if x is not None else None for x in _run(op, d)]
    torch.cuda.synchronize()
    kw = dict(scale=op.scale)
    ro, rl = ora.forward(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.q_offsets, inp.kv_offsets, **kw)
    rg = ora.backward(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("dout"), inp.q_offsets, inp.kv_offsets, **kw)
    check(o, ro, "O", TOL)
    check(lse[np.isfinite(rl)], rl[np.isfinite(rl)], "lse")
    assert np.all(np.isneginf(lse[~np.isfinite(rl)]))
    for name, g, r in zip(["dQ", "dK", "dV"], (dq, dk, dv), rg):
        check(g, r, name)
