"""GPU parity of the backward kernels (Di, dK/dV, dQ) against the fp64 oracle."""
import numpy as np
import pytest
import torch

from jagged_variable_length_amd import attention as A
from jagged_variable_length_amd import inputs as gen

pytestmark = pytest.mark.gpu

from gpu_util import check, check_dbias, check_lse, device_inputs, make_op, oracle_bwd, oracle_fwd, say, sync  # noqa: E402


def _run(inp, **kw):
    op = make_op(inp, **kw)
    d = device_inputs(inp)
    o, lse = op.forward(d["q"], d["k"], d["v"], bias=d["bias"])
    dq, dk, dv, db = op.backward(d["q"], d["k"], d["v"], d["dout"], o=o, lse=lse, bias=d["bias"])
    sync()
    out = [A.to_f64(x) for x in (dq, dk, dv)] + [A.to_f64(db) if db is not None else None]
    return op, out, (o, lse, d)


def _compare(inp, op, got):
    ref = oracle_bwd(inp, op)
    for name, g, r in zip(["dQ", "dK", "dV", "dBias"], got, ref):
        if r is None:
            continue
        (check_dbias if name == "dBias" else check)(g, r, name)


def test_bwd_config0_f32():
    say("case: bwd config 0 (fp32, D=32, zero-length sample)")
    inp = gen.make_inputs(0, 0)
    op, got, _ = _run(inp, out_dtype="f32", grad_dtype="f32")
    _compare(inp, op, got)


@pytest.mark.parametrize("D", [128, 64, 32])
@pytest.mark.parametrize("bias", [False, True])
def test_bwd_softmax_ragged(D, bias):
    say(f"case: bwd softmax ragged D={D} bias={bias}")
    lq = [1, 0, 130, 64, 257, 33, 7, 500]
    lk = [5, 9, 0, 64, 300, 1, 129, 70]
    inp = gen.make_custom(lq, lk, 3, D, "bf16", seed=D + bias, bias=bias)
    op, got, _ = _run(inp, bias=bias, want_dbias=bias, grad_dtype="f32")
    _compare(inp, op, got)


@pytest.mark.parametrize("lk_scale,wkv", [(20, 1), (50, 2), (300, 4)])
def test_bwd_key_tile_shapes(lk_scale, wkv):
    """Each dK/dV unit shape (32, 64, 128 keys; 4, 2, 1 query splits).

    Samples with one to a few keys make P close to 1, so any error in
    Di = rowsum(dO * O) reaches dS undamped; O is kept in fp32 here (with bf16
    O the rounding of O alone gives |dDi| ~ 2^-9 sqrt(D) |O| |dO|)."""
    say(f"case: bwd dkdv shape wkv={wkv}")
    rng = np.random.default_rng(wkv)
    lk = np.clip(rng.integers(1, 2 * lk_scale, 9), 1, None)
    lq = rng.integers(0, 300, 9)
    inp = gen.make_custom(lq, lk, 2, 64, "bf16", seed=wkv, bias=True)
    op, got, _ = _run(inp, bias=True, want_dbias=True, out_dtype="f32", grad_dtype="f32", split=True)
    assert op.info.dkdv.tile_rows == 32 * wkv
    _compare(inp, op, got)


@pytest.mark.parametrize("act", ["gelu", "silu"])
def test_bwd_gdpa(act):
    say(f"case: bwd gdpa {act}")
    lq = [32, 32, 0, 32, 32]
    lk = [64, 300, 50, 0, 1000]
    inp = gen.make_custom(lq, lk, 2, 128, "bf16", seed=5)
    op, got, _ = _run(inp, act=act, split=True, out_dtype="f32", grad_dtype="f32")
    _compare(inp, op, got)


@pytest.mark.parametrize("act", ["gelu", "silu"])
def test_bwd_gdpa_bias_long_queries(act):
    say(f"case: bwd gdpa {act} with bias, long queries")
    lq = [200, 0, 77, 130]
    lk = [90, 40, 3, 257]
    inp = gen.make_custom(lq, lk, 2, 64, "bf16", seed=15, bias=True)
    op, got, _ = _run(inp, act=act, bias=True, want_dbias=True, split=True, out_dtype="f32", grad_dtype="f32")
    _compare(inp, op, got)


@pytest.mark.parametrize("D", [64, 32])
@pytest.mark.parametrize("act", ["softmax", "silu", "gelu"])
def test_bwd_two_workgroups_per_cu(D, act):
    """dK/dV at D <= 64 without a bias on 64-key units runs two workgroups per
    CU over twice the workers; erf-GELU keeps one (its registers do not fit
    two waves per SIMD).  The plan's dK/dV worker count shows which ran."""
    say(f"case: bwd two dK/dV workgroups per CU D={D} act={act}")
    rng = np.random.default_rng(D + len(act))
    lk = rng.integers(33, 65, 12)  # mean key count in (32, 64]: 64-key units
    lq = rng.integers(0, 400, 12)
    inp = gen.make_custom(lq, lk, 2, D, "bf16", seed=D + len(act))
    gdpa = act != "softmax"
    op, got, _ = _run(inp, act=act, split=gdpa, out_dtype="f32" if gdpa else None, grad_dtype="f32",
                      num_workers=64)
    assert op.info.dkdv.tile_rows == 64
    assert op.info.dkdv.num_workers == (64 if act == "gelu" else 128)
    _compare(inp, op, got)


@pytest.mark.parametrize("D,act,split,out,W", [
    (64, "softmax", False, "bf16", 64), (32, "softmax", False, "f32", 64),
    (64, "softmax", True, "f32", 64),
    (64, "gelu", True, "f32", 64), (32, "silu", True, "f32", 64), (64, "gelu_poly", True, "f32", 64),
    (32, "gelu_poly", True, "bf16", 64),
    (64, "softmax", False, "bf16", 7)])  # 21 forward workers: not a multiple of the 8 XCDs
def test_fwd_three_workgroups_per_cu(D, act, split, out, W):
    """The bf16 forward at D <= 64 without a bias or window on long queries
    takes 128-row tiles with 32-key steps, three workgroups per CU, over three
    times the workers (softmax dQ the same tiles, two per CU; GDPA dQ keeps 256 rows);
    the plan's tile shapes and worker counts show which ran.  The whole backward is checked after it."""
    say(f"case: fwd three workgroups per CU D={D} act={act} split={split} out={out} W={W}")
    rng = np.random.default_rng(D + 7 * len(act) + split)
    lq = rng.integers(60, 400, 10)
    lq[3] = 0
    # at least 33 keys a sample (one full step and a ragged one); a one-key
    # sample (P = 1, where the rounding of O in Di reaches dS undamped and adds
    # up over a key's queries) only with fp32 O
    lk = rng.integers(33, 120, 10)
    lk[6] = 0
    if out == "f32":
        lk[8] = 1
    inp = gen.make_custom(lq, lk, 2, D, "bf16", seed=D + len(act) + split)
    if act == "gelu_poly":
        # its polynomial tanh is meant for small scores (QK-normalised rows):
        # Q / 4, exact in bf16, keeps |s| near 1
        inp.q = gen.f32_to_bf16_bits((inp.f64("q") * 0.25).astype(np.float32))
    op, got, (o, lse, _) = _run(inp, act=act, split=split, out_dtype=out, grad_dtype="f32", num_workers=W)
    assert (op.info.fwd.tile_rows, op.info.fwd.step_rows, op.info.fwd.num_workers) == (128, 32, 3 * W)
    # softmax dQ takes the same shape, two workgroups per CU; the GDPA
    # activations keep 256-row tiles
    if act == "softmax":
        assert (op.info.dq.tile_rows, op.info.dq.step_rows, op.info.dq.num_workers) == (128, 32, 2 * W)
    else:
        assert (op.info.dq.tile_rows, op.info.dq.step_rows, op.info.dq.num_workers) == (256, 32, W)
    ref_o, ref_lse = oracle_fwd(inp, op)
    check(A.to_f64(o), ref_o, "O")
    if act == "softmax":
        check_lse(A.to_f64(lse), ref_lse)
    _compare(inp, op, got)


@pytest.mark.parametrize("W,out", [(64, "bf16"), (7, "f32")])
def test_fwd_two_workgroups_per_cu_d128(W, out):
    """The bf16 softmax forward and dQ at D = 128 without a bias or window
    take 128-row tiles with 32-key steps, two workgroups per CU, over twice the
    workers (7 asked for: 14, not a multiple of the 8 XCDs); the whole
    backward is checked after it."""
    say(f"case: fwd two workgroups per CU D=128 W={W} out={out}")
    rng = np.random.default_rng(128 + W)
    lq = rng.integers(60, 500, 10)
    lq[2] = 0
    lk = rng.integers(33, 400, 10)
    lk[5] = 0
    inp = gen.make_custom(lq, lk, 2, 128, "bf16", seed=128 + W)
    op, got, (o, lse, _) = _run(inp, out_dtype=out, grad_dtype="f32", num_workers=W)
    assert (op.info.fwd.tile_rows, op.info.fwd.step_rows, op.info.fwd.num_workers) == (128, 32, 2 * W)
    # dQ takes the same tile shape, also two workgroups per CU
    assert (op.info.dq.tile_rows, op.info.dq.step_rows, op.info.dq.num_workers) == (128, 32, 2 * W)
    ref_o, ref_lse = oracle_fwd(inp, op)
    check(A.to_f64(o), ref_o, "O")
    check_lse(A.to_f64(lse), ref_lse)
    _compare(inp, op, got)


@pytest.mark.parametrize("D,bias,tile", [(64, True, 32), (128, False, 32), (128, True, 256)])
def test_bwd_short_query_softmax(D, bias, tile):
    """Short query tiles: the dQ kernel splits each 32-row group's keys over
    4 waves; at D = 128 a bias tile does not fit that shape and the plan keeps
    128-row query tiles."""
    say(f"case: bwd softmax 32-row queries (dQ key-split) D={D} bias={bias}")
    lq = [32, 20, 1, 32]
    lk = [700, 0, 129, 64]
    inp = gen.make_custom(lq, lk, 2, D, "bf16", seed=6, bias=bias)
    op, got, _ = _run(inp, bias=bias, want_dbias=bias, grad_dtype="f32")
    assert op.info.dq.tile_rows == tile
    _compare(inp, op, got)


def test_bwd_bf16_gradients_balanced():
    """bf16 gradients on self-attention lengths like the JFA workload."""
    say("case: bwd bf16 grads, lengths 8..1000")
    rng = np.random.default_rng(3)
    lens = np.clip(np.rint(np.exp(np.log(300) + rng.standard_normal(12))), 8, 1000).astype(int)
    inp = gen.make_custom(lens, lens, 4, 128, "bf16", seed=3, bias=True)
    op, got, _ = _run(inp, bias=True, want_dbias=True, dbias_dtype="bf16")
    _compare(inp, op, got)


def test_bwd_overwrites_garbage_and_is_deterministic():
    say("case: bwd garbage-filled outputs + determinism")
    lq, lk = [0, 10, 6, 0], [4, 0, 9, 0]
    inp = gen.make_custom(lq, lk, 2, 64, "bf16", seed=8, bias=True)
    op = make_op(inp, bias=True, want_dbias=True, grad_dtype="f32")
    d = device_inputs(inp)
    o, lse = op.forward(d["q"], d["k"], d["v"], bias=d["bias"])
    res = []
    for _ in range(2):
        dq = torch.full((op.Tq, 2, 64), 5.0, device="cuda")
        dk = torch.full((op.Tk, 2, 64), 5.0, device="cuda")
        dv = torch.full((op.Tk, 2, 64), 5.0, device="cuda")
        db = torch.full((int(op.info.bias_elems),), 5.0, device="cuda")
        op.backward(d["q"], d["k"], d["v"], d["dout"], o=o, lse=lse, bias=d["bias"], dq=dq, dk=dk, dv=dv,
                    dbias=db)
        res.append((dq, dk, dv, db))
    sync()
    for a, b in zip(*res):
        assert torch.equal(a, b)
    _compare(inp, op, [A.to_f64(x) for x in res[0]])
