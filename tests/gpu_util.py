"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
the fp64 oracle on the same seeded inputs, and compare element by element."""
from __future__ import annotations

import sys

import numpy as np
import torch

from jagged_variable_length_amd import attention as A
from jagged_variable_length_amd import inputs as gen
from oracle import attention as ora

TOL = 2e-2  # max-abs bound on every output and gradient element


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_op(inp: gen.JaggedInputs, *, act="softmax", block=False, bias=False, want_dbias=False,
            out_dtype=None, grad_dtype=None, split=False, order="zigzag", num_workers=0, dbias_dtype=None,
            window=None):
    op = A.JaggedAttention(inp.q_offsets, inp.kv_offsets, inp.H, inp.D, act=act, block_diagonal=block,
                           has_bias=bias, want_dbias=want_dbias, in_dtype=inp.dtype, out_dtype=out_dtype,
                           grad_dtype=grad_dtype, split_operands=split, order=order,
                           num_workers=num_workers, dbias_dtype=dbias_dtype, window=window)
    return op.upload()


def device_inputs(inp: gen.JaggedInputs):
    d = {n: A.to_device(getattr(inp, n), inp.dtype) for n in ("q", "k", "v")}
    d["bias"] = A.to_device(inp.bias, inp.dtype) if inp.bias is not None else None
    d["dout"] = A.to_device(inp.dout, inp.dtype) if inp.dout is not None else None
    return d


def oracle_fwd(inp, op):
    return ora.forward(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.q_offsets, inp.kv_offsets,
                       scale=op.scale, activation=op.act, block_diagonal=op.block_diagonal,
                       bias=inp.f64("bias"), window=op.window)


def oracle_bwd(inp, op):
    return ora.backward(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("dout"), inp.q_offsets,
                        inp.kv_offsets, scale=op.scale, activation=op.act,
                        block_diagonal=op.block_diagonal, bias=inp.f64("bias"),
                        want_dbias=op.want_dbias, window=op.window)


def max_err(got: np.ndarray, ref: np.ndarray, name: str):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    return err, rms


def check(got, ref, name, tol=TOL):
    err, rms = max_err(got, ref, name)
    say(f"  {name:6s} max|err| = {err:.3e}  (rms ref {rms:.3e}, tol {tol})")
    assert err <= tol, f"{name}: max abs error {err} > {tol}"
    return err


def check_full(got, ref, name, starts, tol=TOL, unit="row"):
    """Every element of a full-size tensor against the oracle; prints the
    worst error and the sample it sits in.  ``starts``: the sample offsets
    along the first axis (rows of [T, H, D] or [T, H], or flat elements of
    dBias).  -inf (LSE of a row without keys) must match exactly."""
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    inf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf), f"{name}: -inf pattern differs"
    with np.errstate(invalid="ignore"):
        diff = np.where(inf, 0.0, np.abs(got - ref))
    assert np.all(np.isfinite(diff)), f"{name}: non-finite values"
    if diff.size == 0:
        say(f"  {name:6s} (empty)")
        return 0.0
    flat = int(np.argmax(diff))
    err = float(diff.reshape(-1)[flat])
    pos = int(np.unravel_index(flat, ref.shape)[0])
    sample = int(np.searchsorted(np.asarray(starts), pos, side="right") - 1)
    rms = float(np.sqrt(np.mean(np.where(inf, 0.0, ref) ** 2)))
    say(f"  {name:6s} max|err| = {err:.3e} at sample {sample} ({unit} {pos - int(starts[sample])}), "
        f"{diff.size} elements (rms ref {rms:.3e}, tol {tol})")
    assert err <= tol, f"{name}: max abs error {err} > {tol} (sample {sample})"
    return err


def check_dbias(got, ref, name="dBias", tol=TOL):
    """dBias against the 2e-2 bound and also against its own scale: dBias
    elements shrink with the number of keys (about 1e-3 on long samples), so
    the absolute bound alone would not see a value written to the wrong
    place; a misplaced value errs by the order of max|ref|, a correct one by
    well under 1 % of it here."""
    err = check(got, ref, name, tol)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    assert err <= 0.1 * scale + 1e-4, f"{name}: max abs error {err} against max|ref| {scale}"
    return err


def check_lse(got, ref, tol=TOL):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "LSE -inf pattern differs"
    return check(got[fin], ref[fin], "lse", tol)


def sync():
    torch.cuda.synchronize()
