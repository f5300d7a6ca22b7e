"""Full-size workloads, in the launch configuration bench.py times (default
plan and workers): sampled outputs against the fp64 oracle, plus properties
that hold at any size (finite everywhere, bitwise run-to-run identical)."""
import numpy as np
import pytest
import torch

from jagged_variable_length_amd import attention as A
from jagged_variable_length_amd import inputs as gen
from oracle import attention as ora

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

from gpu_util import TOL, check, check_dbias, say  # noqa: E402


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


def _pick_samples(inp, rng):
    lq = inp.lq
    nz = np.nonzero(lq > 0)[0]
    picks = {int(nz[np.argmin(lq[nz])]), int(np.argmax(lq)), 0, int(rng.integers(0, inp.B))}
    return sorted(picks)


@pytest.mark.parametrize("cfg", [1, 2, 3, 8])
def test_dense_workload_full_size(cfg):
    say(f"case: workload {cfg} full size")
    w, inp, op, d = _setup(cfg)
    outs = _run(op, d)
    outs2 = _run(op, d)
    torch.cuda.synchronize()
    for a, b in zip(outs, outs2):
        if a is not None:
            assert torch.isfinite(a).all()
            assert torch.equal(a, b), "not run-to-run identical"
    o, lse, dq, dk, dv, db = [A.to_f64(x) if x is not None else None for x in outs]
    q, k, v, do, bias = inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("dout"), inp.f64("bias")
    bst = ora.bias_starts(inp.lq, inp.lk, w.H)
    for b in _pick_samples(inp, np.random.default_rng(cfg)):
        say(f"  sample {b}: lq={inp.lq[b]} lk={inp.lk[b]}")
        sq = slice(inp.q_offsets[b], inp.q_offsets[b + 1])
        sk = slice(inp.kv_offsets[b], inp.kv_offsets[b + 1])
        kw = dict(scale=op.scale, activation=w.act, bias=bias)
        ro, rl = ora.forward_sample(q, k, v, inp.q_offsets, inp.kv_offsets, b, **kw)
        rg = ora.backward_sample(q, k, v, do, inp.q_offsets, inp.kv_offsets, b, want_dbias=w.want_dbias, **kw)
        check(o[sq], ro, "O")
        if rl is not None:
            check(lse[sq], rl, "lse")
        check(dq[sq], rg[0], "dQ")
        check(dk[sk], rg[1], "dK")
        check(dv[sk], rg[2], "dV")
        if w.want_dbias:
            check_dbias(db[bst[b]:bst[b + 1]], rg[3])


def test_block_workload_full_size():
    """BlockAttention workload: sampled 64-token blocks, each checked as an
    independent 64-row problem (block-diagonal attention equals the blocks run
    on their own; pinned in test_oracle)."""
    say("case: workload 4 full size")
    w, inp, op, d = _setup(4)
    outs = _run(op, d)
    outs2 = _run(op, d)
    torch.cuda.synchronize()
    for a, b in zip(outs, outs2):
        if a is not None:
            assert torch.isfinite(a).all()
            assert torch.equal(a, b)
    o, _, dq, dk, dv, _ = outs
    rng = np.random.default_rng(4)
    q, k, v, do = inp.q, inp.k, inp.v, inp.dout
    for b in _pick_samples(inp, rng):
        L = int(inp.lq[b])
        nblk = (L + 63) // 64
        for t in sorted({0, nblk - 1, int(rng.integers(0, nblk))}):
            r0 = int(inp.q_offsets[b]) + 64 * t
            r1 = int(inp.q_offsets[b]) + min(L, 64 * t + 64)
            say(f"  sample {b} block {t}: rows {r1 - r0}")
            sub = [gen.to_f64(x[r0:r1], "bf16") for x in (q, k, v, do)]
            off = np.array([0, r1 - r0])
            ro, _ = ora.forward(sub[0], sub[1], sub[2], off, off, scale=op.scale)
            rg = ora.backward(sub[0], sub[1], sub[2], sub[3], off, off, scale=op.scale)
            check(A.to_f64(o[r0:r1]), ro, "O")
            check(A.to_f64(dq[r0:r1]), rg[0], "dQ")
            check(A.to_f64(dk[r0:r1]), rg[1], "dK")
            check(A.to_f64(dv[r0:r1]), rg[2], "dV")


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
