"""fp64 CPU oracle for jagged attention, forward and backward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library
never calls it and it shares no code with the HIP path.

What it computes is the plain definition of attention on each sample of a
jagged batch, one (sample, head) at a time, in float64:

* "Training GEM at LLM scale" (Meta engineering post), section "Jagged
  Sequence Flash Attention": attention over unpadded variable-length
  tensors, with custom additive biases, Q and K/V of different lengths, and
  a backward pass.  The subtraction scheme described there is stated to give
  results numerically equivalent to masked attention, so the oracle is the
  masked definition itself, not the scheme.
* same post, section "Generalized Dot-Product Attention (GDPA)": two matrix
  products with an element-wise activation (GELU or SiLU) where softmax
  would be; no normalisation.
* same post, section "BlockAttention": fixed 64-token blocks; query block i
  sees only key/value block i.
* same post, section "BlockAttention" (its account of the sliding-window
  kernel that came before block attention): each token attends only to
  nearby events of its own sequence.  The pages give no window size and no
  direction, so the window is two parameters (left, right): query i of a
  sample sees key j iff  i - left <= j <= i + right  (self-attention only,
  lq == lk per sample).  (left, right) = (inf, 0) is causal attention.

Conventions (readings where the pages are silent):
  S = scale * Q K^T + bias   (bias added after scaling, shape [H, lq, lk])
  no causal mask; zero-length samples give O = 0, LSE = -inf, zero grads.
Matrix products use numpy (BLAS) in float64; erf is scipy's float64 erf.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
from scipy.special import erf

BLOCK = 64  # BlockAttention block length, "BlockAttention" section


# ----------------------------------------------------------------------------
# pointwise activations used by GDPA ("Generalized Dot-Product Attention")
# ----------------------------------------------------------------------------
def gelu(x):
    """Exact (erf) GELU: x * Phi(x)."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def gelu_grad(x):
    """d/dx [x Phi(x)] = Phi(x) + x phi(x)."""
    cdf = 0.5 * (1.0 + erf(x / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
    return cdf + x * pdf


def silu(x):
    """x * sigmoid(x)."""
    return x / (1.0 + np.exp(-x))


def silu_grad(x):
    """sigmoid(x) * (1 + x (1 - sigmoid(x)))."""
    s = 1.0 / (1.0 + np.exp(-x))
    return s * (1.0 + x * (1.0 - s))


# ALU-only GELU ("Generalized Dot-Product Attention (GDPA)", item on the
# ALU-only activation approximation): GELU in its tanh form,
#   0.5 x (1 + tanh(c (x + a x^3))),  c = sqrt(2/pi), a = 0.044715
# (Hendrycks and Gimpel's approximation), with tanh replaced by its Taylor
# polynomial about 0 through order 6.  tanh is odd, so its even coefficients
# vanish: t(u) = u - u^3/3 + 2 u^5/15.  Accurate only for bounded inputs,
# which QK-norm provides (see qk_norm below).
GELU_TANH_C = math.sqrt(2.0 / math.pi)
GELU_TANH_A = 0.044715


def tanh_taylor6(u):
    return u - u ** 3 / 3.0 + 2.0 * u ** 5 / 15.0


def tanh_taylor6_grad(u):
    return 1.0 - u ** 2 + 2.0 * u ** 4 / 3.0


def gelu_poly(x):
    u = GELU_TANH_C * (x + GELU_TANH_A * x ** 3)
    return 0.5 * x * (1.0 + tanh_taylor6(u))


def gelu_poly_grad(x):
    u = GELU_TANH_C * (x + GELU_TANH_A * x ** 3)
    du = GELU_TANH_C * (1.0 + 3.0 * GELU_TANH_A * x ** 2)
    return 0.5 * (1.0 + tanh_taylor6(u)) + 0.5 * x * tanh_taylor6_grad(u) * du


def identity(x):
    return x


def identity_grad(x):
    return np.ones_like(x)


_ACTS = {
    "gelu": (gelu, gelu_grad),
    "silu": (silu, silu_grad),
    "gelu_poly": (gelu_poly, gelu_poly_grad),
    "identity": (identity, identity_grad),
}


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def _lengths(offsets):
    off = np.asarray(offsets, dtype=np.int64)
    return off[:-1], np.diff(off)


def bias_starts(lq, lk, H):
    """Element offset of each sample's [H, lq, lk] bias block."""
    sizes = H * np.asarray(lq, np.int64) * np.asarray(lk, np.int64)
    start = np.zeros(len(sizes) + 1, dtype=np.int64)
    np.cumsum(sizes, out=start[1:])
    return start


def allowed_mask(lq, lk, block_diagonal, window=None):
    """Allowed (i, j) pairs: all of them, floor(i/64) == floor(j/64), or
    (sliding window (left, right)) i - left <= j <= i + right."""
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    if window is not None:
        left, right = window
        return (j >= i - left) & (j <= i + right)
    if not block_diagonal:
        return np.ones((lq, lk), dtype=bool)
    return (i // BLOCK) == (j // BLOCK)


def _check_mask_args(lq, lk, block_diagonal, window):
    if block_diagonal and window is not None:
        raise ValueError("block-diagonal and sliding-window masks are exclusive")
    if (block_diagonal or window is not None) and np.any(lq != lk):
        raise ValueError("block-diagonal / sliding-window attention needs lq == lk per sample")
    if window is not None and (window[0] < 0 or window[1] < 0):
        raise ValueError("window sides must be >= 0")


def _scores(Qb, Kb, scale, bias_bh):
    S = scale * (Qb @ Kb.T)
    if bias_bh is not None:
        S = S + bias_bh
    return S


def _probabilities(S, allowed, activation):
    """P (and LSE for softmax) for one (sample, head)."""
    lq = S.shape[0]
    if activation == "softmax":
        P = np.zeros_like(S)
        lse = np.full(lq, -np.inf)
        rows = allowed.any(axis=1)
        if rows.any():
            Sm = np.where(allowed, S, -np.inf)[rows]
            m = Sm.max(axis=1, keepdims=True)
            E = np.where(allowed[rows], np.exp(Sm - m), 0.0)
            l = E.sum(axis=1, keepdims=True)
            P[rows] = E / l
            lse[rows] = (m + np.log(l))[:, 0]
        return P, lse
    act, _ = _ACTS[activation]
    return np.where(allowed, act(S), 0.0), None


# ----------------------------------------------------------------------------
# forward
# ----------------------------------------------------------------------------
def forward(q, k, v, q_offsets, kv_offsets, *, scale=None, activation="softmax",
            block_diagonal=False, bias=None, window=None):
    """O [Tq,H,D] and LSE [Tq,H] (None for GDPA activations), all fp64.

    q, k, v: float64 [T, H, D]; bias: float64 flat per-sample [H, lq, lk].
    """
    Tq, H, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q0, lq = _lengths(q_offsets)
    k0, lk = _lengths(kv_offsets)
    _check_mask_args(lq, lk, block_diagonal, window)
    bstart = bias_starts(lq, lk, H)
    o = np.zeros((Tq, H, D))
    lse = np.full((Tq, H), -np.inf) if activation == "softmax" else None
    for b in range(len(lq)):
        nq, nk = int(lq[b]), int(lk[b])
        if nq == 0:
            continue
        rq = slice(int(q0[b]), int(q0[b]) + nq)
        if nk == 0:
            continue  # O = 0, LSE = -inf
        rk = slice(int(k0[b]), int(k0[b]) + nk)
        allowed = allowed_mask(nq, nk, block_diagonal, window)
        for h in range(H):
            bias_bh = None
            if bias is not None:
                s0 = int(bstart[b]) + h * nq * nk
                bias_bh = bias[s0:s0 + nq * nk].reshape(nq, nk)
            S = _scores(q[rq, h], k[rk, h], scale, bias_bh)
            P, l = _probabilities(S, allowed, activation)
            o[rq, h] = P @ v[rk, h]
            if lse is not None:
                lse[rq, h] = l
    return o, lse


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------
def backward(q, k, v, dout, q_offsets, kv_offsets, *, scale=None, activation="softmax",
             block_diagonal=False, bias=None, want_dbias=False, window=None):
    """dQ, dK, dV (fp64, [T,H,D]) and dBias (flat, or None).

    For one (sample, head), with P the forward probabilities/activations:
      dV = P^T dO;  dP = dO V^T
      softmax: dS = P * (dP - Di), Di = rowsum(dO * O), O = P V
      GDPA   : dS = act'(S) * dP (0 where not allowed)
      dQ = scale dS K;  dK = scale dS^T Q;  dBias = dS
    """
    Tq, H, D = q.shape
    Tk = k.shape[0]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q0, lq = _lengths(q_offsets)
    k0, lk = _lengths(kv_offsets)
    _check_mask_args(lq, lk, block_diagonal, window)
    bstart = bias_starts(lq, lk, H)
    dq = np.zeros((Tq, H, D))
    dk = np.zeros((Tk, H, D))
    dv = np.zeros((Tk, H, D))
    dbias = np.zeros(int(bstart[-1])) if want_dbias else None
    for b in range(len(lq)):
        nq, nk = int(lq[b]), int(lk[b])
        if nq == 0 or nk == 0:
            continue
        rq = slice(int(q0[b]), int(q0[b]) + nq)
        rk = slice(int(k0[b]), int(k0[b]) + nk)
        allowed = allowed_mask(nq, nk, block_diagonal, window)
        for h in range(H):
            s0 = int(bstart[b]) + h * nq * nk
            bias_bh = None
            if bias is not None:
                bias_bh = bias[s0:s0 + nq * nk].reshape(nq, nk)
            Qb, Kb, Vb, dOb = q[rq, h], k[rk, h], v[rk, h], dout[rq, h]
            S = _scores(Qb, Kb, scale, bias_bh)
            P, _ = _probabilities(S, allowed, activation)
            dV = P.T @ dOb
            dP = dOb @ Vb.T
            if activation == "softmax":
                Ob = P @ Vb
                Di = np.sum(dOb * Ob, axis=1, keepdims=True)
                dS = P * (dP - Di)
            else:
                _, act_grad = _ACTS[activation]
                dS = np.where(allowed, act_grad(S) * dP, 0.0)
            dq[rq, h] = scale * (dS @ Kb)
            dk[rk, h] = scale * (dS.T @ Qb)
            dv[rk, h] = dV
            if dbias is not None:
                dbias[s0:s0 + nq * nk] = dS.reshape(-1)
    return dq, dk, dv, dbias


# ----------------------------------------------------------------------------
# convenience: one sample / head at a time (used for sampled checks at
# full workload sizes, where the whole batch would be slow)
# ----------------------------------------------------------------------------
def forward_sample(q, k, v, q_offsets, kv_offsets, b, *, scale=None, activation="softmax",
                   block_diagonal=False, bias=None, window=None):
    """Forward restricted to sample ``b``: returns (O_b [lq,H,D], LSE_b or None)."""
    sub = _sub_batch(q, k, v, None, q_offsets, kv_offsets, b, bias)
    o, lse = forward(sub["q"], sub["k"], sub["v"], sub["qo"], sub["ko"], scale=scale,
                     activation=activation, block_diagonal=block_diagonal, bias=sub["bias"],
                     window=window)
    return o, lse


def backward_sample(q, k, v, dout, q_offsets, kv_offsets, b, *, scale=None, activation="softmax",
                    block_diagonal=False, bias=None, want_dbias=False, window=None):
    """Backward restricted to sample ``b``: dQ_b, dK_b, dV_b, dBias_b."""
    sub = _sub_batch(q, k, v, dout, q_offsets, kv_offsets, b, bias)
    return backward(sub["q"], sub["k"], sub["v"], sub["do"], sub["qo"], sub["ko"], scale=scale,
                    activation=activation, block_diagonal=block_diagonal, bias=sub["bias"],
                    want_dbias=want_dbias, window=window)


def _sub_batch(q, k, v, dout, q_offsets, kv_offsets, b, bias):
    q_offsets = np.asarray(q_offsets, np.int64)
    kv_offsets = np.asarray(kv_offsets, np.int64)
    H = q.shape[1]
    qa, qb = int(q_offsets[b]), int(q_offsets[b + 1])
    ka, kb = int(kv_offsets[b]), int(kv_offsets[b + 1])
    sub = {
        "q": q[qa:qb], "k": k[ka:kb], "v": v[ka:kb],
        "do": None if dout is None else dout[qa:qb],
        "qo": np.array([0, qb - qa], np.int64), "ko": np.array([0, kb - ka], np.int64),
        "bias": None,
    }
    if bias is not None:
        lq = np.diff(q_offsets)
        lk = np.diff(kv_offsets)
        st = bias_starts(lq, lk, H)
        sub["bias"] = bias[int(st[b]):int(st[b + 1])]
    return sub
