"""fp64 CPU oracle for rotary position embedding (RoPE), forward and backward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP path.

"Training GEM at LLM scale" (Meta engineering post), section
"BlockAttention": the RoPE backward is fused into the block-attention
epilogue, so the gradients never leave fp32 registers before the inverse
rotation.  The pages fix no RoPE convention; the reading here is the common
rotate-half form: for a row x of D elements at position m (its token index
inside its own sample), pair element j with element j + D/2 (j < D/2) and
rotate the pair by the angle m * theta_j, theta_j = base^(-2j/D), base =
10000 unless given:
    y_j       = x_j cos(m theta_j) - x_{j+D/2} sin(m theta_j)
    y_{j+D/2} = x_{j+D/2} cos(m theta_j) + x_j sin(m theta_j)
The map is a rotation, so its backward is the transposed rotation.
"""
from __future__ import annotations

import numpy as np

BASE = 10000.0


def positions(offsets):
    """Token index inside its own sample, for every row of a jagged tensor."""
    off = np.asarray(offsets, dtype=np.int64)
    return np.concatenate([np.arange(off[b + 1] - off[b]) for b in range(len(off) - 1)] + [np.zeros(0, np.int64)])


def angles(pos, D, base=BASE):
    theta = base ** (-2.0 * np.arange(D // 2) / D)
    return np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]


def forward(x, offsets, base=BASE):
    """x [T, H, D] float64 -> rotated rows."""
    D = x.shape[-1]
    a = angles(positions(offsets), D, base)[:, None, :]
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., :D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def backward(dy, offsets, base=BASE):
    """Gradient with respect to x of sum(forward(x) * dy): the inverse rotation."""
    D = dy.shape[-1]
    a = angles(positions(offsets), D, base)[:, None, :]
    c, s = np.cos(a), np.sin(a)
    d1, d2 = dy[..., :D // 2], dy[..., D // 2:]
    return np.concatenate([d1 * c + d2 * s, d2 * c - d1 * s], axis=-1)
