"""fp64 CPU oracle for QK-norm (row-wise L2 normalisation), forward and backward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP path.

"Training GEM at LLM scale" (Meta engineering post), section "Generalized
Dot-Product Attention (GDPA)", item on the ALU-only activation: the
polynomial GELU is accurate on the bounded input range that QK-norm (query
and key normalisation) enforces.  The pages do not define QK-norm further;
the reading here is the L2 form: every query row and every key row of every
head is scaled to unit length,
    y = x / max(||x||_2, eps),   eps = 1e-12,
so that |q.k| <= 1 and an attention score scale * q.k lies in [-scale, scale].
Backward (||x|| > eps):  dx = (dy - y (y . dy)) / ||x||;  else dx = dy / eps.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-12


def forward(x):
    """x [..., D] float64 -> (y [..., D], rnorm [...]) with rnorm = 1 / max(||x||, eps)."""
    n = np.sqrt(np.sum(x * x, axis=-1))
    r = 1.0 / np.maximum(n, EPS)
    return x * r[..., None], r


def backward(x, dy):
    """Gradient of sum(forward(x)[0] * dy) with respect to x."""
    n = np.sqrt(np.sum(x * x, axis=-1))
    r = 1.0 / np.maximum(n, EPS)
    y = x * r[..., None]
    along = np.sum(y * dy, axis=-1, keepdims=True)
    live = (n > EPS)[..., None]
    return r[..., None] * (dy - np.where(live, y * along, 0.0))
