"""GPU parity at the largest per-sample size the library accepts with a bias
and an fp32 dBias: one sample of 16383 x 16383 (a head's dBias block is
16383^2 * 4 = 1 073 610 756 bytes, just under the 2^30-byte limit that keeps
every per-(sample, head) byte offset inside a buffer descriptor's 32-bit
range; 16383 also leaves a ragged tail in every tile size), checked whole
against the fp64 oracle: O, LSE, dQ, dK, dV and every dBias element."""
import numpy as np
import pytest

from jagged_variable_length_amd import attention as A
from jagged_variable_length_amd import inputs as gen
from oracle import attention as ora

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

from gpu_util import check, check_dbias, check_lse, say, sync  # noqa: E402

L = 16383


def test_largest_sample_with_fp32_dbias():
    assert L * L * 4 < (1 << 30) <= (L + 1) * (L + 1) * 4
    say(f"case: one sample {L} x {L}, H=1, D=128, bias + fp32 dBias")
    inp = gen.make_custom([L], [L], 1, 128, "bf16", seed=11, bias=True)
    op = A.JaggedAttention(inp.q_offsets, inp.kv_offsets, 1, 128, has_bias=True, want_dbias=True,
                           dbias_dtype="f32").upload()
    d = {n: A.to_device(getattr(inp, n), "bf16") for n in ("q", "k", "v", "dout")}
    bias = A.to_device(inp.bias, "bf16")
    o, lse = op.forward(d["q"], d["k"], d["v"], bias=bias)
    dq, dk, dv, db = op.backward(d["q"], d["k"], d["v"], d["dout"], o=o, lse=lse, bias=bias)
    sync()
    got = [A.to_f64(t) for t in (o, lse, dq, dk, dv)]
    gdb = A.to_f64(db)
    del o, lse, dq, dk, dv, db, d, bias
    say("  oracle (fp64, one dense 16383 x 16383 head)")
    q, k, v, do, b = inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("dout"), inp.f64("bias")
    ro, rl = ora.forward(q, k, v, inp.q_offsets, inp.kv_offsets, scale=op.scale, bias=b)
    check(got[0], ro, "O")
    check_lse(got[1], rl)
    del ro, rl
    rdq, rdk, rdv, rdb = ora.backward(q, k, v, do, inp.q_offsets, inp.kv_offsets, scale=op.scale, bias=b,
                                      want_dbias=True)
    check(got[2], rdq, "dQ")
    check(got[3], rdk, "dK")
    check(got[4], rdv, "dV")
    assert gdb.shape == rdb.shape
    check_dbias(gdb, rdb)
    # the last element of the dBias block sits at byte offset ~2^30 - 4
    assert np.isfinite(gdb[-1]) and abs(gdb[-1] - rdb[-1]) <= 2e-2
