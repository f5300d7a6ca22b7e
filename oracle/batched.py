"""Whole-workload evaluation of the fp64 attention oracle, many problems at once.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP path.

The arithmetic is the definition in ``oracle.attention`` ("Training GEM at
LLM scale", sections "Jagged Sequence Flash Attention", "Generalized
Dot-Product Attention (GDPA)" and "BlockAttention"), for one problem (a set
of query rows against a set of key/value rows, every head):

    S = scale Q K^T + bias,  over the allowed pairs only
    softmax: P = exp(S - m) / sum exp(S - m), LSE = m + ln sum exp(S - m)
    GDPA:    P = act(S)
    O = P V
    dV = P^T dO,  dP = dO V^T,
    dS = P (dP - Di), Di = rowsum(dO O)   (softmax)   or   act'(S) dP  (GDPA)
    dQ = scale dS K,  dK = scale dS^T Q,  dBias = dS

Here it is evaluated for a stack of independent problems of one shape at a
time, with float64 torch products on the CPU, so that full-size workloads
(tens of thousands of 64-token blocks) can be compared element by element in
seconds.  Nothing is blocked or reordered inside a problem; the stack only
replaces a Python loop over problems.  Three ways of cutting a workload into
such problems, each pinned against ``oracle.attention`` on the CPU
(``tests/test_oracle_batched.py``):

* no mask: every sample is one problem; samples of equal (lq, lk) share a
  stack;
* block-diagonal mask: every 64-token block of every sample is a problem of
  its own (section "BlockAttention": query block i sees only key block i,
  so the blocks are independent attention problems);
* sliding window (left, right), self-attention: chunks of C query rows
  [a, a + C) with the keys [a - left, a + C + right) clipped to the sample,
  which hold every key any of those rows sees.  O, LSE and dQ of the chunk's
  rows are exact; a key's dK and dV are the sum of the contributions of the
  chunks that see it (the sum over query rows grouped by chunk).
"""
from __future__ import annotations

import math
from collections import defaultdict

import numpy as np
import torch

from . import attention as _att

BLOCK = _att.BLOCK
_STACK_BYTES = 1 << 28  # bound on one stacked [n, H, nq, nk] float64 array


def _act(activation):
    f, g = _att._ACTS[activation]
    return (lambda x: torch.from_numpy(f(x.numpy()))), (lambda x: torch.from_numpy(g(x.numpy())))


def _probs(S, allowed, activation):
    """P and LSE of a stack S [n, H, nq, nk]; allowed [nq, nk] bool tensor or None."""
    if activation == "softmax":
        if allowed is not None:
            S = S.masked_fill(~allowed, -math.inf)
        m = S.amax(dim=-1, keepdim=True)
        live = torch.isfinite(m)  # rows with at least one allowed key
        m = torch.where(live, m, torch.zeros_like(m))
        E = torch.exp(S - m)  # exp(-inf) = 0 off the mask
        l = E.sum(dim=-1, keepdim=True)
        P = torch.where(live, E / torch.where(live, l, torch.ones_like(l)), torch.zeros_like(E))
        lse = torch.where(live, m + torch.log(l), torch.full_like(m, -math.inf))[..., 0]
        return P, lse
    act, _ = _act(activation)
    P = act(S)
    if allowed is not None:
        P = P.masked_fill(~allowed, 0.0)
    return P, None


def stack_forward(Q, K, V, bias, allowed, scale, activation):
    """O [n, H, nq, D] and LSE [n, H, nq] (or None) of a stack of problems;
    Q [n, H, nq, D], K, V [n, H, nk, D], bias [n, H, nq, nk] or None."""
    S = scale * (Q @ K.transpose(-1, -2))
    if bias is not None:
        S = S + bias
    P, lse = _probs(S, allowed, activation)
    return P @ V, lse


def stack_backward(Q, K, V, dO, bias, allowed, scale, activation):
    """dQ, dK, dV, dS (= dBias) of a stack of problems (shapes as stack_forward)."""
    S = scale * (Q @ K.transpose(-1, -2))
    if bias is not None:
        S = S + bias
    P, _ = _probs(S, allowed, activation)
    dV = P.transpose(-1, -2) @ dO
    dP = dO @ V.transpose(-1, -2)
    if activation == "softmax":
        O = P @ V
        Di = (dO * O).sum(dim=-1, keepdim=True)
        dS = P * (dP - Di)
    else:
        _, grad = _act(activation)
        dS = grad(S) * dP
        if allowed is not None:
            dS = dS.masked_fill(~allowed, 0.0)
    return scale * (dS @ K), scale * (dS.transpose(-1, -2) @ Q), dV, dS


# ----------------------------------------------------------------------------
# problem sets: (query rows, key rows, bias element indices, shared mask)
# ----------------------------------------------------------------------------
class _Group:
    """Problems of one shape: q_rows [n, nq], k_rows [n, nk] absolute row
    indices; bias0 [n] first bias element of each problem's head-0 block (or
    None) with row pitch ``bias_pitch`` and per-head stride ``bias_hstride``
    [n]; allowed [nq, nk] (or None)."""

    def __init__(self, q_rows, k_rows, allowed=None, bias0=None, bias_pitch=None, bias_hstride=None):
        self.q_rows, self.k_rows, self.allowed = q_rows, k_rows, allowed
        self.bias0, self.bias_pitch, self.bias_hstride = bias0, bias_pitch, bias_hstride


def _gather_rows(x, rows):
    """x [T, H, D] tensor, rows [n, r] -> [n, H, r, D]."""
    return x[torch.from_numpy(rows)].permute(0, 2, 1, 3)


def _bias_index(g, sel, H, nq, nk):
    """Flat bias element index [n, H, nq, nk] of the problems ``sel`` of g."""
    b0 = g.bias0[sel][:, None, None, None]
    hs = g.bias_hstride[sel][:, None, None, None]
    h = np.arange(H)[None, :, None, None]
    i = np.arange(nq)[None, None, :, None]
    j = np.arange(nk)[None, None, None, :]
    return b0 + h * hs + i * g.bias_pitch[sel][:, None, None, None] + j


def _chunks(n, H, nq, nk, D):
    per = H * nq * max(nk, D) * 8
    step = max(1, _STACK_BYTES // max(per, 1))
    return [np.arange(s, min(n, s + step)) for s in range(0, n, step)]


def _run(groups, q, k, v, dout, bias, *, scale, activation, want_fwd, want_bwd, want_dbias,
         add_kv=False):
    """Evaluate every group; scatter the results into full-size arrays."""
    Tq, H, D = q.shape
    Tk = k.shape[0]
    qt, kt, vt = torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)
    dot = torch.from_numpy(dout) if want_bwd else None
    bt = torch.from_numpy(bias) if bias is not None else None
    o = np.zeros((Tq, H, D)) if want_fwd else None
    lse = np.full((Tq, H), -np.inf) if (want_fwd and activation == "softmax") else None
    dq = np.zeros((Tq, H, D)) if want_bwd else None
    dk = np.zeros((Tk, H, D)) if want_bwd else None
    dv = np.zeros((Tk, H, D)) if want_bwd else None
    db = np.zeros(bias.shape[0]) if (want_bwd and want_dbias) else None
    for g in groups:
        n, nq = g.q_rows.shape
        nk = g.k_rows.shape[1]
        allowed = torch.from_numpy(g.allowed) if g.allowed is not None else None
        for sel in _chunks(n, H, nq, nk, D):
            Q = _gather_rows(qt, g.q_rows[sel])
            K = _gather_rows(kt, g.k_rows[sel])
            V = _gather_rows(vt, g.k_rows[sel])
            bidx = _bias_index(g, sel, H, nq, nk) if bt is not None else None
            Bs = bt[torch.from_numpy(bidx)] if bidx is not None else None
            qr = g.q_rows[sel].reshape(-1)
            if want_fwd:
                O, L = stack_forward(Q, K, V, Bs, allowed, scale, activation)
                o[qr] = O.permute(0, 2, 1, 3).reshape(-1, H, D).numpy()
                if lse is not None:
                    lse[qr] = L.permute(0, 2, 1).reshape(-1, H).numpy()
            if want_bwd:
                dO = _gather_rows(dot, g.q_rows[sel])
                gq, gk, gv, gs = stack_backward(Q, K, V, dO, Bs, allowed, scale, activation)
                dq[qr] = gq.permute(0, 2, 1, 3).reshape(-1, H, D).numpy()
                kr = g.k_rows[sel].reshape(-1)
                gk = gk.permute(0, 2, 1, 3).reshape(-1, H, D).numpy()
                gv = gv.permute(0, 2, 1, 3).reshape(-1, H, D).numpy()
                if add_kv:
                    ki = torch.from_numpy(kr)
                    torch.from_numpy(dk).index_add_(0, ki, torch.from_numpy(gk))
                    torch.from_numpy(dv).index_add_(0, ki, torch.from_numpy(gv))
                else:
                    dk[kr] = gk
                    dv[kr] = gv
                if db is not None:
                    db[bidx.reshape(-1)] = gs.reshape(-1).numpy()
    return o, lse, (dq, dk, dv, db)


def _lengths(offsets):
    off = np.asarray(offsets, dtype=np.int64)
    return off[:-1], np.diff(off)


def dense_groups(q_offsets, kv_offsets, H, with_bias):
    """One problem per sample with lq > 0 and lk > 0; equal shapes share a group."""
    q0, lq = _lengths(q_offsets)
    k0, lk = _lengths(kv_offsets)
    bst = _att.bias_starts(lq, lk, H)
    by_shape = defaultdict(list)
    for b in range(len(lq)):
        if lq[b] > 0 and lk[b] > 0:
            by_shape[(int(lq[b]), int(lk[b]))].append(b)
    groups = []
    for (nq, nk), bs in sorted(by_shape.items()):
        bs = np.asarray(bs, np.int64)
        qr = q0[bs][:, None] + np.arange(nq)[None, :]
        kr = k0[bs][:, None] + np.arange(nk)[None, :]
        if with_bias:
            groups.append(_Group(qr, kr, None, bst[bs], np.full(len(bs), nk, np.int64),
                                 np.full(len(bs), nq * nk, np.int64)))
        else:
            groups.append(_Group(qr, kr))
    return groups


def block_groups(offsets):
    """One problem per 64-token block (query block = key block); lq == lk."""
    s0, ln = _lengths(offsets)
    by_len = defaultdict(list)
    for b in range(len(ln)):
        for a in range(0, int(ln[b]), BLOCK):
            by_len[min(BLOCK, int(ln[b]) - a)].append(int(s0[b]) + a)
    groups = []
    for r, starts in sorted(by_len.items()):
        rows = np.asarray(starts, np.int64)[:, None] + np.arange(r)[None, :]
        groups.append(_Group(rows, rows))
    return groups


def window_groups(offsets, window, chunk=64):
    """Chunks of ``chunk`` query rows with the keys their window can reach."""
    left, right = window
    s0, ln = _lengths(offsets)
    by_shape = defaultdict(list)
    for b in range(len(ln)):
        L = int(ln[b])
        for a in range(0, L, chunk):
            nq = min(chunk, L - a)
            ks = max(0, a - left)
            ke = min(L, a + nq + right)
            by_shape[(nq, ke - ks, a - ks)].append((int(s0[b]) + a, int(s0[b]) + ks))
    groups = []
    for (nq, nk, shift), lst in sorted(by_shape.items()):
        arr = np.asarray(lst, np.int64)
        qr = arr[:, 0:1] + np.arange(nq)[None, :]
        kr = arr[:, 1:2] + np.arange(nk)[None, :]
        i = np.arange(nq)[:, None] + shift  # query position relative to the first key
        j = np.arange(nk)[None, :]
        allowed = (j >= i - left) & (j <= i + right)
        groups.append(_Group(qr, kr, allowed))
    return groups


# ----------------------------------------------------------------------------
# whole workloads (same arguments and results as oracle.attention)
# ----------------------------------------------------------------------------
def forward(q, k, v, q_offsets, kv_offsets, *, scale=None, activation="softmax", block_diagonal=False,
            bias=None, window=None):
    """Same result as oracle.attention.forward, problems evaluated in stacks."""
    H, D = q.shape[1], q.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    groups = _groups(q_offsets, kv_offsets, H, bias is not None, block_diagonal, window)
    o, lse, _ = _run(groups, q, k, v, None, bias, scale=scale, activation=activation, want_fwd=True,
                     want_bwd=False, want_dbias=False)
    return o, lse


def backward(q, k, v, dout, q_offsets, kv_offsets, *, scale=None, activation="softmax",
             block_diagonal=False, bias=None, want_dbias=False, window=None):
    """Same result as oracle.attention.backward, problems evaluated in stacks."""
    H, D = q.shape[1], q.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    groups = _groups(q_offsets, kv_offsets, H, bias is not None, block_diagonal, window)
    _, _, grads = _run(groups, q, k, v, dout, bias, scale=scale, activation=activation, want_fwd=False,
                       want_bwd=True, want_dbias=want_dbias and bias is not None,
                       add_kv=window is not None)
    return grads


def _groups(q_offsets, kv_offsets, H, with_bias, block_diagonal, window):
    _, lq = _lengths(q_offsets)
    _, lk = _lengths(kv_offsets)
    if (block_diagonal or window is not None) and np.any(lq != lk):
        raise ValueError("block-diagonal / sliding-window attention needs lq == lk per sample")
    if (block_diagonal or window is not None) and with_bias:
        raise ValueError("stacked evaluation of masked attention takes no bias")
    if block_diagonal:
        return block_groups(q_offsets)
    if window is not None:
        return window_groups(q_offsets, window)
    return dense_groups(q_offsets, kv_offsets, H, with_bias)
