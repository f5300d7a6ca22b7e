"""GPU parity of QK-norm (row-wise L2 normalisation) and of GDPA with the
ALU-only polynomial GELU, against the fp64 oracle.

"Training GEM at LLM scale", section "Generalized Dot-Product Attention
(GDPA)", item on the ALU-only activation: the polynomial GELU is meant for
the bounded scores that QK-norm gives, so the attention cases below run on
normalised Q and K (scores are scale x cosine)."""
import numpy as np
import pytest
import torch

from jagged_variable_length_amd import attention as A
from jagged_variable_length_amd import inputs as gen
from oracle import attention as ora
from oracle import batched as bat
from oracle import qknorm as qn

pytestmark = pytest.mark.gpu

from gpu_util import check, check_full, say, sync  # noqa: E402

_TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _rows(n, D, seed, dtype):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 3, D)).astype(np.float32) * rng.uniform(1e-3, 50, (n, 3, 1)).astype(np.float32)
    x[min(5, n - 1), 1] = 0.0  # a zero row stays zero
    if dtype == "bf16":
        bits = gen.f32_to_bf16_bits(x)
        return A.to_device(bits, "bf16"), gen.bf16_bits_to_f32(bits).astype(np.float64)
    return A.to_device(x, "f32"), x.astype(np.float64)


@pytest.mark.parametrize("D", [128, 64, 32])
@pytest.mark.parametrize("xt,yt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"), ("f32", "bf16")])
def test_l2norm_forward_backward(D, xt, yt):
    say(f"case: l2norm D={D} x={xt} y={yt}")
    n = 1001  # not a multiple of the rows one workgroup pass covers
    x, x64 = _rows(n, D, seed=D, dtype=xt)
    y, r = A.qk_norm(x, out_dtype=yt)
    dy64 = np.random.default_rng(D + 1).standard_normal(x64.shape)
    dy = torch.from_numpy(dy64.astype(np.float32)).to("cuda").to(_TDT[yt])
    dy64 = A.to_f64(dy)
    dx = A.qk_norm_backward(x, dy, out_dtype="f32")
    sync()
    ry, rr = qn.forward(x64)
    check(A.to_f64(y), ry, "y", 8e-3 if yt == "bf16" else 1e-5)
    live = np.isfinite(rr) & (np.linalg.norm(x64, axis=-1) > 0)
    rel = np.max(np.abs(A.to_f64(r)[live] / rr[live] - 1.0))
    assert rel < 1e-5, rel
    ref_dx = qn.backward(x64, dy64)
    # relative to the row's scale 1/||x|| (rows span five orders of magnitude);
    # the zero row (dx = dy / eps by definition) is left out
    got = A.to_f64(dx)[live]
    err = np.max(np.abs(got - ref_dx[live]) / rr[live][:, None])
    say(f"  dx max|err| / r = {err:.3e}")
    assert err < 1e-4


def test_l2norm_in_place():
    say("case: l2norm in place")
    x, x64 = _rows(300, 64, seed=9, dtype="bf16")
    A.qk_norm(x, out=x)
    sync()
    check(A.to_f64(x), qn.forward(x64)[0], "y", 8e-3)


def _gdpa_case(lq, lk, H, D, seed, scale, bias=False, window=None):
    inp = gen.make_custom(lq, lk, H, D, "bf16", seed=seed, bias=bias)
    dev = {n: A.to_device(getattr(inp, n), "bf16") for n in ("q", "k", "v", "dout")}
    qh, _ = A.qk_norm(dev["q"])
    kh, _ = A.qk_norm(dev["k"])
    op = A.JaggedAttention(inp.q_offsets, inp.kv_offsets, H, D, act="gelu_poly", has_bias=bias,
                           out_dtype="f32", grad_dtype="f32", split_operands=True, scale=scale,
                           window=window).upload()
    b = A.to_device(inp.bias, "bf16") if bias else None
    o, _ = op.forward(qh, kh, dev["v"], bias=b)
    dqh, dkh, dv, _ = op.backward(qh, kh, dev["v"], dev["dout"], bias=b)
    dq = A.qk_norm_backward(dev["q"], dqh)
    dk = A.qk_norm_backward(dev["k"], dkh)
    sync()
    return inp, op, qh, kh, [A.to_f64(t) for t in (o, dq, dk, dv, dqh, dkh)]


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("scale", [1.0, 3.0])
def test_gdpa_gelu_poly_on_normalised_inputs(D, scale):
    """Attention on the kernel's own normalised Q and K (rounded to bf16):
    the oracle takes those same bf16 values."""
    say(f"case: gelu_poly GDPA D={D} scale={scale}")
    lq = [1, 0, 130, 64, 257, 33, 32, 500]
    lk = [5, 9, 0, 64, 300, 1, 1500, 70]
    inp, op, qh, kh, (o, _, _, dv, dqh, dkh) = _gdpa_case(lq, lk, 2, D, seed=D, scale=scale)
    q64, k64 = A.to_f64(qh), A.to_f64(kh)
    kw = dict(scale=scale, activation="gelu_poly")
    ro, _ = ora.forward(q64, k64, inp.f64("v"), inp.q_offsets, inp.kv_offsets, **kw)
    rg = ora.backward(q64, k64, inp.f64("v"), inp.f64("dout"), inp.q_offsets, inp.kv_offsets, **kw)
    check(o, ro, "O")
    check(dqh, rg[0], "dQhat")
    check(dkh, rg[1], "dKhat")
    check(dv, rg[2], "dV")


@pytest.mark.parametrize("window", [None, (40, 7)])
def test_qknorm_gelu_poly_chain(window):
    """Raw Q, K -> QK-norm -> polynomial-GELU attention -> backward -> QK-norm
    backward, against the two oracles chained in fp64 from the raw inputs."""
    say(f"case: qknorm + gelu_poly chain, window={window}")
    L = [70, 1, 200, 0, 129]
    lq, lk = (L, L) if window else ([70, 1, 32, 0, 129], [9, 300, 64, 5, 129])
    inp, op, _, _, (o, dq, dk, dv, _, _) = _gdpa_case(lq, lk, 2, 128, seed=3, scale=2.0, bias=True,
                                                      window=window)
    q, k = inp.f64("q"), inp.f64("k")
    qh, kh = qn.forward(q)[0], qn.forward(k)[0]
    kw = dict(scale=2.0, activation="gelu_poly", bias=inp.f64("bias"), window=window)
    ro, _ = ora.forward(qh, kh, inp.f64("v"), inp.q_offsets, inp.kv_offsets, **kw)
    rg = ora.backward(qh, kh, inp.f64("v"), inp.f64("dout"), inp.q_offsets, inp.kv_offsets, **kw)
    check(o, ro, "O")
    check(dq, qn.backward(q, rg[0]), "dQ")
    check(dk, qn.backward(k, rg[1]), "dK")
    check(dv, rg[2], "dV")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_qknorm_gelu_poly_workload_full_size():
    """Full-size workload in the benchmark's configuration, checked stage by
    stage on each stage's actual inputs: the QK-norm outputs against the
    oracle's normalised rows (bf16 rounding), the attention against the
    oracle run on the kernel's bf16 Q-hat and K-hat, and the QK-norm backward
    against the oracle's on the raw rows and the oracle's dQ-hat / dK-hat.
    (Chained from the raw inputs in fp64, the bf16 storage of Q-hat and K-hat
    alone moves O by up to ~0.03 on a 4000-key sample, more than the bound.)
    Every element is compared; results are also run-to-run identical."""
    cfg = 6
    w = gen.WORKLOADS[cfg]
    say(f"case: workload {cfg} ({w.name}) full size")
    inp = gen.make_inputs(cfg, cfg)
    dev = {n: A.to_device(getattr(inp, n), w.dtype) for n in ("q", "k", "v", "dout")}
    op = A.JaggedAttention(inp.q_offsets, inp.kv_offsets, w.H, w.D, act=w.act, out_dtype=w.out_dtype,
                           grad_dtype=w.grad_dtype, split_operands=w.split_operands, scale=w.scale).upload()

    def run():
        qh, _ = A.qk_norm(dev["q"])
        kh, _ = A.qk_norm(dev["k"])
        o, _ = op.forward(qh, kh, dev["v"])
        dqh, dkh, dv, _ = op.backward(qh, kh, dev["v"], dev["dout"])
        return (qh, kh, o, A.qk_norm_backward(dev["q"], dqh), A.qk_norm_backward(dev["k"], dkh), dv)

    outs, outs2 = run(), run()
    sync()
    for a_, b_ in zip(outs, outs2):
        assert torch.isfinite(a_).all()
        assert torch.equal(a_, b_)
    qh, kh, o, dq, dk, dv = [A.to_f64(t) for t in outs]
    del outs, outs2, dev
    q, k, v, do = inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("dout")
    check_full(qh, qn.forward(q)[0], "Qhat", inp.q_offsets, 8e-3)
    check_full(kh, qn.forward(k)[0], "Khat", inp.kv_offsets, 8e-3)
    kw = dict(scale=w.scale, activation=w.act)
    ro, _ = bat.forward(qh, kh, v, inp.q_offsets, inp.kv_offsets, **kw)
    check_full(o, ro, "O", inp.q_offsets)
    del ro
    rg = bat.backward(qh, kh, v, do, inp.q_offsets, inp.kv_offsets, **kw)
    check_full(dq, qn.backward(q, rg[0]), "dQ", inp.q_offsets)
    check_full(dk, qn.backward(k, rg[1]), "dK", inp.kv_offsets)
    check_full(dv, rg[2], "dV", inp.kv_offsets)
