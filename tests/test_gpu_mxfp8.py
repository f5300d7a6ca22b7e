"""GPU parity of MXFP8 attention ("Training GEM at LLM scale", section "Mixed
Ultra-Low-Precision Training", part "Low Precision Flash Attention").

* The quantiser is integer/byte work: its codes, transposed codes and scales
  must equal the oracle's (oracle/mxfp8.py) bit for bit.
* The forward is compared with the exact attention of the dequantised inputs
  (oracle.attention on oracle.mxfp8's values).  The kernel rounds P to E4M3
  with a shared exponent, so each P value carries a relative error of at
  most 2^-4 (half a step of three mantissa bits) or, below the smallest
  normal of its block, an absolute error of at most 2^-17 of the block's
  reference value; O then differs from the exact attention by at most
      2^-4 sum_j |Phat_ij| |V_jd| + 2^-17 sum_j ref_ij |V_jd|
  (Phat = P / rowsum for softmax, P for GDPA; ref_ij = the row's largest |P|
  in j's 32-key block for GDPA, 1 for normalised softmax), plus what the
  fp32 accumulation of the products (S, dP, Di) moves: EPS = 1e-4 of the
  sum of the magnitudes of each one's terms (fp32 accumulation of D terms
  stays within D 2^-24 <= 7.6e-6 of it; the kernels' measured errors are
  around 1e-5).  Every element is checked against that bound; LSE (from
  the unrounded row sum) to 2e-3.  The backward is bounded the same way
  (see _bwd_bounds), including where softmax's dS = P (dP - Di) cancels.
"""
import numpy as np
import pytest
import torch

from jagged_variable_length_amd import attention as A
from jagged_variable_length_amd import inputs as gen
from oracle import attention as ora
from oracle import mxfp8 as mx

pytestmark = pytest.mark.gpu

from gpu_util import say, sync  # noqa: E402


def _op(inp, act="softmax", out="f32", **kw):
    return A.JaggedAttention(inp.q_offsets, inp.kv_offsets, inp.H, inp.D, act=act, in_dtype="mxfp8", out_dtype=out,
                             grad_dtype="f32", **kw).upload()


def _oracle_codes_t(codes, offsets):
    """Expected codes_t: per 32-row block r, [H, D, 32] with tokens past the sample zero."""
    T, H, D = codes.shape
    rbs = mx.row_block_starts(offsets)
    out = np.zeros((int(rbs[-1]), H, D, 32), dtype=np.uint8)
    for b in range(len(offsets) - 1):
        for r in range(int(rbs[b + 1] - rbs[b])):
            r0 = int(offsets[b]) + 32 * r
            r1 = min(r0 + 32, int(offsets[b + 1]))
            out[rbs[b] + r, :, :, :r1 - r0] = np.transpose(codes[r0:r1], (1, 2, 0))
    return out


def _u8(t, n):
    return t[:n].cpu().numpy()


def _scaled_inputs(inp, seed):
    """Row magnitudes spread over several binades, and a zero row, so that
    blocks get different scales."""
    rng = np.random.default_rng(seed)
    for name in ("q", "k", "v"):
        x = gen.bf16_bits_to_f32(getattr(inp, name))
        x = x * np.exp(1.5 * rng.standard_normal((x.shape[0], x.shape[1], 1))).astype(np.float32)
        if x.shape[0] > 3:
            x[3] = 0.0
        setattr(inp, name, gen.f32_to_bf16_bits(x))
    return inp


@pytest.mark.parametrize("D", [128, 64])
def test_mx_quantize_bit_exact(D):
    lq = [33, 0, 1, 64, 100, 31, 32, 7]
    lk = [5, 9, 70, 0, 200, 32, 33, 1]
    inp = _scaled_inputs(gen.make_custom(lq, lk, 3, D, "bf16", seed=D), seed=D)
    op = _op(inp)
    for rows, name, off in (("q", "q", inp.q_offsets), ("kv", "k", inp.kv_offsets), ("kv", "v", inp.kv_offsets)):
        say(f"case: MXFP8 quantise {name} D={D}")
        x = A.to_device(getattr(inp, name), "bf16")
        m = op.mx_quantize(x, rows)
        sync()
        codes, scales, _ = mx.quantize(inp.f64(name), off)
        T = codes.shape[0]
        got_c = _u8(m.codes, codes.size).reshape(codes.shape)
        got_s = _u8(m.scales, scales.size).reshape(scales.shape)
        ref_t = _oracle_codes_t(codes, off)
        got_t = _u8(m.codes_t, ref_t.size).reshape(ref_t.shape)
        assert np.array_equal(got_s, scales), f"{name}: scales differ at {np.argwhere(got_s != scales)[:5]}"
        bad = np.argwhere(got_c != codes)
        assert bad.size == 0, f"{name}: codes differ at {bad[:5]} got {got_c[tuple(bad[0])]} want {codes[tuple(bad[0])]}"
        assert np.array_equal(got_t, ref_t), f"{name}: transposed codes differ"
        say(f"  {T} rows, {scales.size} blocks: bit-exact")


EPS = 1e-4  # accumulation error of S, dP, Di: this fraction of the sum of |products|


def _fwd_bound(qd, kd, vd, qo, ko, act, scale):
    """Element bound |O_mx - O_exact| for P rounded to E4M3 (see the module
    doc), plus the fp32 accumulation of S (EPS of the sum of the magnitudes of
    its products), which moves P by a relative 2 scale * S_err for softmax
    (exponent and row sum) and by |act'| scale * S_err for GDPA."""
    Tq, H, D = qd.shape
    bound = np.full((Tq, H, D), 1e-5)  # rows without keys: O = 0 exactly
    for b in range(len(qo) - 1):
        rq, rk = slice(qo[b], qo[b + 1]), slice(ko[b], ko[b + 1])
        nq, nk = qo[b + 1] - qo[b], ko[b + 1] - ko[b]
        if nq == 0 or nk == 0:
            continue
        for h in range(H):
            S = scale * (qd[rq, h] @ kd[rk, h].T)
            eS = EPS * scale * (np.abs(qd[rq, h]) @ np.abs(kd[rk, h]).T)
            av = np.abs(vd[rk, h])
            if act == "softmax":
                E = np.exp(S - S.max(axis=1, keepdims=True))
                P = E / E.sum(axis=1, keepdims=True)
                ref = np.ones_like(P)
                eP = 2.0 * P * eS
            else:
                f, fg = ora._ACTS[act]
                P = f(S)
                nb = (nk + 31) // 32
                Pp = np.zeros((nq, nb * 32))
                Pp[:, :nk] = np.abs(P)
                ref = np.repeat(Pp.reshape(nq, nb, 32).max(axis=2), 32, axis=1)[:, :nk]
                eP = np.abs(fg(S)) * eS
            bound[rq, h] = (2.0 ** -4 * np.abs(P) + eP) @ av + 2.0 ** -17 * (ref @ av) + 1e-5
    return bound


def _bound_ratio(got, ref, bound, name):
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    r = err / bound
    ratio = float(np.max(r)) if err.size else 0.0
    where = np.unravel_index(int(np.argmax(r)), r.shape) if err.size else ()
    say(f"  {name:6s} max|err| = {float(err.max()) if err.size else 0.0:.3e}, worst err/bound = {ratio:.3f} at {where}")
    return ratio


def _check_bound(got, ref, bound, name):
    ratio = _bound_ratio(got, ref, bound, name)
    assert ratio <= 1.0, f"{name}: error above the E4M3 rounding bound (ratio {ratio})"


@pytest.mark.parametrize("act", ["softmax", "gelu", "silu"])
@pytest.mark.parametrize("D", [128, 64])
def test_mx_forward(act, D):
    say(f"case: MXFP8 forward act={act} D={D}")
    lq = [130, 0, 1, 64, 300, 31, 129, 5]
    lk = [70, 9, 200, 0, 300, 64, 1, 129]
    inp = gen.make_custom(lq, lk, 2, D, "bf16", seed=7 + D)
    op = _op(inp, act=act)
    dq, dk, dv = (A.to_device(getattr(inp, n), "bf16") for n in ("q", "k", "v"))
    qm, km, vm = op.mx_quantize(dq, "q"), op.mx_quantize(dk, "kv"), op.mx_quantize(dv, "kv")
    o, lse = op.mx_forward(qm, km, vm)
    sync()
    _, _, qd = mx.quantize(inp.f64("q"), inp.q_offsets)
    _, _, kd = mx.quantize(inp.f64("k"), inp.kv_offsets)
    _, _, vd = mx.quantize(inp.f64("v"), inp.kv_offsets)
    ro, rl = ora.forward(qd, kd, vd, inp.q_offsets, inp.kv_offsets, scale=op.scale, activation=act)
    bound = _fwd_bound(qd, kd, vd, inp.q_offsets, inp.kv_offsets, act, op.scale)
    if act == "softmax":
        got = A.to_f64(lse)
        assert np.array_equal(np.isneginf(got), np.isneginf(rl))
        fin = np.isfinite(rl)
        err = float(np.max(np.abs(got[fin] - rl[fin])))
        say(f"  lse    max|err| = {err:.3e}")
    _check_bound(A.to_f64(o), ro, bound, "O")
    if act == "softmax":
        assert err <= 2e-3


def test_mx_forward_rejects_bf16_entry_points():
    inp = gen.make_custom([5], [7], 1, 64, "bf16", seed=1)
    op = _op(inp)
    d = {n: A.to_device(getattr(inp, n), "bf16") for n in ("q", "k", "v")}
    from jagged_variable_length_amd import binding as B
    with pytest.raises(B.JattnError) as e:
        B.jattn_fwd(op.plan, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), None,
                    d["q"].data_ptr(), None, op.workspace.data_ptr(), None)
    assert e.value.code == B.JATTN_E_UNSUPPORTED


def _block_amax(M, nq, nk):
    """Each element replaced by the largest |M| of its 32 x 32 block (blocks
    aligned to the sample's first query and key)."""
    bq, bk = (nq + 31) // 32, (nk + 31) // 32
    P = np.zeros((bq * 32, bk * 32))
    P[:nq, :nk] = np.abs(M)
    a = P.reshape(bq, 32, bk, 32).max(axis=(1, 3))
    return np.repeat(np.repeat(a, 32, axis=0), 32, axis=1)[:nq, :nk]


def _bwd_bounds(qd, kd, vd, dod, qo, ko, act, scale, ro, o_err=None, lse_err=None):
    """Element bounds of dQ, dK, dV.  Two sources:
    * rounding of P and dS to E4M3 with one exponent per 32 x 32 block (P of
      softmax: the fixed exponent -8, P <= 1): each element errs by at most
      2^-4 of itself or 2^-17 of its block's largest magnitude (2^-18 for
      softmax P);
    * the fp32 accumulation of S = Q K^T, dP = dO V^T (exact products of E4M3
      values) and Di = rowsum(dO O): each errs by at most EPS times the sum of
      the magnitudes of its products (fp32 accumulation of D terms is within
      D 2^-24 <= 7.6e-6 of it; EPS keeps a margin).  They reach dS through
      P (relative error scale * dS_err) and through dP - Di, where softmax
      cancels: a key that takes a row's whole weight has dS = 0 exactly, but
      its computed dP - Di is the difference of two separately rounded sums.
    With o_err / lse_err (bounds of the O and LSE the backward was given, when
    they come from the MXFP8 forward rather than the exact definition), Di
    moves by at most sum_d |dO| o_err and P by a relative 2 lse_err."""
    bq = np.full(qd.shape, 1e-5)
    bk = np.full(kd.shape, 1e-5)
    bv = np.full(vd.shape, 1e-5)
    for b in range(len(qo) - 1):
        rq, rk = slice(qo[b], qo[b + 1]), slice(ko[b], ko[b + 1])
        nq, nk = qo[b + 1] - qo[b], ko[b + 1] - ko[b]
        if nq == 0 or nk == 0:
            continue
        for h in range(qd.shape[1]):
            Q, K, V, dO = qd[rq, h], kd[rk, h], vd[rk, h], dod[rq, h]
            S = scale * (Q @ K.T)
            dP = dO @ V.T
            eS = EPS * scale * (np.abs(Q) @ np.abs(K).T)  # |error of scale * S|
            edP = EPS * (np.abs(dO) @ np.abs(V).T)
            if act == "softmax":
                E = np.exp(S - S.max(axis=1, keepdims=True))
                P = E / E.sum(axis=1, keepdims=True)
                Di = np.sum(dO * ro[rq, h], axis=1, keepdims=True)
                eDi = EPS * np.sum(np.abs(dO) * np.abs(ro[rq, h]), axis=1, keepdims=True)
                if o_err is not None:
                    eDi = eDi + np.sum(np.abs(dO) * o_err[rq, h], axis=1, keepdims=True)
                dS = P * (dP - Di)
                eP = P * 2.0 * eS  # exp of a shifted score: relative error ~ the score's (row sum too)
                if lse_err is not None:
                    eP = eP + P * 2.0 * lse_err[rq, h][:, None]
                edS = P * (edP + eDi) + np.abs(dP - Di) * eP
                pref = np.full_like(P, 2.0 ** -1)  # 2^-18 = 2^-17 * 2^-1 of P's unit scale
            else:
                f, fg = ora._ACTS[act]
                P, dS = f(S), fg(S) * dP
                eP = np.abs(fg(S)) * eS
                edS = np.abs(fg(S)) * edP + np.abs(dP) * eS  # |act''| <= 1 for erf-GELU and SiLU
                pref = _block_amax(P, nq, nk)
            sref = _block_amax(dS, nq, nk)
            aP, adS = np.abs(P), np.abs(dS)
            bv[rk, h] += (2.0 ** -4 * aP + eP).T @ np.abs(dO) + 2.0 ** -17 * (pref.T @ np.abs(dO))
            bk[rk, h] += scale * ((2.0 ** -4 * adS + edS).T @ np.abs(Q) + 2.0 ** -17 * (sref.T @ np.abs(Q)))
            bq[rq, h] += scale * ((2.0 ** -4 * adS + edS) @ np.abs(K) + 2.0 ** -17 * (sref @ np.abs(K)))
    return bq, bk, bv


@pytest.mark.parametrize("act", ["softmax", "gelu", "silu"])
@pytest.mark.parametrize("D", [128, 64])
def test_mx_backward(act, D):
    """The backward is given the exact O and LSE of the quantised inputs (so
    only its own rounding of P and dS is measured) and compared with the
    exact gradients of the dequantised inputs, element by element against
    the rounding bound."""
    say(f"case: MXFP8 backward act={act} D={D}")
    lq = [130, 0, 1, 64, 300, 31, 129, 5]
    lk = [70, 9, 200, 0, 300, 64, 1, 129]
    inp = gen.make_custom(lq, lk, 2, D, "bf16", seed=11 + D)
    op = _op(inp, act=act)
    dev = {n: A.to_device(getattr(inp, n), "bf16") for n in ("q", "k", "v", "dout")}
    qm, km, vm = op.mx_quantize(dev["q"], "q"), op.mx_quantize(dev["k"], "kv"), op.mx_quantize(dev["v"], "kv")
    dom = op.mx_quantize(dev["dout"], "q")
    _, _, qd = mx.quantize(inp.f64("q"), inp.q_offsets)
    _, _, kd = mx.quantize(inp.f64("k"), inp.kv_offsets)
    _, _, vd = mx.quantize(inp.f64("v"), inp.kv_offsets)
    _, _, dod = mx.quantize(inp.f64("dout"), inp.q_offsets)
    kw = dict(scale=op.scale, activation=act)
    ro, rl = ora.forward(qd, kd, vd, inp.q_offsets, inp.kv_offsets, **kw)
    o = torch.from_numpy(ro.astype(np.float32)).cuda()
    lse = torch.from_numpy(rl.astype(np.float32)).cuda() if rl is not None else None
    dq, dk, dv = op.mx_backward(qm, km, vm, dom, o=o, lse=lse)
    sync()
    rg = ora.backward(qd, kd, vd, dod, inp.q_offsets, inp.kv_offsets, **kw)
    if act == "softmax":
        # the row statistics the Di pass left in the workspace's scratch region
        # (its last 2 * align256(4 Tq H) bytes: Di, then LSE * log2 e)
        n = op.Tq * op.H
        a256 = (4 * n + 255) // 256 * 256
        ws = op.workspace[-2 * a256:].cpu().numpy()
        di = ws[:4 * n].view(np.float32).reshape(op.Tq, op.H)
        l2 = ws[a256:a256 + 4 * n].view(np.float32).reshape(op.Tq, op.H)
        rdi = np.sum(dod * ro, axis=2)
        fin = np.isfinite(rl)
        say(f"  Di     max|err| = {float(np.max(np.abs(di - rdi))):.3e}, "
            f"LSE2 max|err| = {float(np.max(np.abs(l2[fin] - rl[fin] * np.log2(np.e)))):.3e}")
        assert np.max(np.abs(di - rdi)) <= 1e-4 * (1 + np.max(np.abs(rdi)))
    bq, bk, bv = _bwd_bounds(qd, kd, vd, dod, inp.q_offsets, inp.kv_offsets, act, op.scale, ro)
    ratios = [_bound_ratio(A.to_f64(g), r, b, name) for g, r, b, name in
              ((dq, rg[0], bq, "dQ"), (dk, rg[1], bk, "dK"), (dv, rg[2], bv, "dV"))]
    assert max(ratios) <= 1.0, f"error above the E4M3 rounding bound: {ratios}"


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_mx_workload_full_size():
    """Full-size MXFP8 workload in the benchmark's launch configuration:
    quantisation bit-exact, the forward against its bound, and the backward
    run on the forward's own O and LSE (as the benchmark chains them) against
    its bound extended by those inputs' own error bounds; every element."""
    cfg = 9
    w = gen.WORKLOADS[cfg]
    say(f"case: workload {cfg} ({w.name}) full size, every element")
    inp = gen.make_inputs(cfg)
    op = A.JaggedAttention(inp.q_offsets, inp.kv_offsets, w.H, w.D, act=w.act, in_dtype="mxfp8",
                           out_dtype=w.out_dtype, grad_dtype=w.grad_dtype).upload()
    dev = {n: A.to_device(getattr(inp, n), "bf16") for n in ("q", "k", "v", "dout")}
    qm, km, vm = op.mx_quantize(dev["q"], "q"), op.mx_quantize(dev["k"], "kv"), op.mx_quantize(dev["v"], "kv")
    dom = op.mx_quantize(dev["dout"], "q")
    o, lse = op.mx_forward(qm, km, vm)
    dq, dk, dv = op.mx_backward(qm, km, vm, dom, o=o, lse=lse)
    o2, _ = op.mx_forward(qm, km, vm)
    dq2, _, _ = op.mx_backward(qm, km, vm, dom, o=o, lse=lse)
    sync()
    assert torch.equal(o, o2) and torch.equal(dq, dq2), "not run-to-run identical"
    codes, scales, qd = mx.quantize(inp.f64("q"), inp.q_offsets)
    assert np.array_equal(_u8(qm.codes, codes.size).reshape(codes.shape), codes)
    assert np.array_equal(_u8(qm.scales, scales.size).reshape(scales.shape), scales)
    _, _, kd = mx.quantize(inp.f64("k"), inp.kv_offsets)
    _, _, vd = mx.quantize(inp.f64("v"), inp.kv_offsets)
    _, _, dod = mx.quantize(inp.f64("dout"), inp.q_offsets)
    kw = dict(scale=op.scale, activation=w.act)
    ro, rl = ora.forward(qd, kd, vd, inp.q_offsets, inp.kv_offsets, **kw)
    bo = _fwd_bound(qd, kd, vd, inp.q_offsets, inp.kv_offsets, w.act, op.scale)
    _check_bound(A.to_f64(o), ro, bo, "O")
    got_l = A.to_f64(lse)
    lerr = np.abs(got_l - rl)
    # LSE is 1-Lipschitz in the scores: its error is within the largest score error of the row
    lse_bound = np.zeros_like(rl)
    for b in range(inp.B):
        rq, rk = slice(inp.q_offsets[b], inp.q_offsets[b + 1]), slice(inp.kv_offsets[b], inp.kv_offsets[b + 1])
        for h in range(w.H):
            lse_bound[rq, h] = (EPS * op.scale * (np.abs(qd[rq, h]) @ np.abs(kd[rk, h]).T)).max(axis=1) + 1e-5
    say(f"  lse    max|err| = {float(lerr.max()):.3e}, worst err/bound = {float(np.max(lerr / lse_bound)):.3f}")
    assert np.all(lerr <= lse_bound)
    rg = ora.backward(qd, kd, vd, dod, inp.q_offsets, inp.kv_offsets, **kw)
    bq, bk, bv = _bwd_bounds(qd, kd, vd, dod, inp.q_offsets, inp.kv_offsets, w.act, op.scale, ro, o_err=bo,
                             lse_err=lse_bound)
    ratios = [_bound_ratio(A.to_f64(g), r, b_, name) for g, r, b_, name in
              ((dq, rg[0], bq, "dQ"), (dk, rg[1], bk, "dK"), (dv, rg[2], bv, "dV"))]
    assert max(ratios) <= 1.0, f"error above the E4M3 rounding bound: {ratios}"
