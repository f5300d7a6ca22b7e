"""Seeded synthetic inputs for jagged attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the fp64 oracle (through the tests and the bench)
and the HIP path consume exactly the arrays produced here.

Jagged layout ("Training GEM at LLM scale", section "Jagged Sequence Flash
Attention": attention runs directly on unpadded variable-length tensors):
  * values  : [T, H, D] row-major, samples concatenated along T
  * offsets : int64 [B+1], offsets[0] = 0, non-decreasing, offsets[B] = T
  * bias    : one flat array, sample b contributes [H, lq_b, lk_b] row-major
              at element offset sum_{j<b} H*lq_j*lk_j

Recipe (one numpy Generator per call, seed = config index by default):
  draw order = lengths (Q, then K/V when they differ) -> Q -> K -> V -> bias
  -> dO.  Values are float32 standard normals; bf16 configs round them to
  bf16 with round-to-nearest-even and keep the 16-bit patterns.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

ACT_SOFTMAX = "softmax"
ACT_GELU = "gelu"
ACT_SILU = "silu"
ACT_GELU_POLY = "gelu_poly"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One of the five synthetic workloads (shapes, dtype, mode)."""

    name: str
    B: int
    H: int
    D: int
    dtype: str  # "f32" or "bf16"
    act: str
    block_diagonal: bool
    bias: bool
    want_dbias: bool
    # output dtypes chosen so that the 2e-2 max-abs bound is reachable
    out_dtype: str
    grad_dtype: str
    split_operands: bool
    dbias_dtype: str = "f32"
    window: Optional[tuple] = None  # sliding window (left, right), self-attention only
    qk_norm: bool = False  # Q and K rows L2-normalised before attention (and in the backward)
    scale: Optional[float] = None  # score scale; None = 1/sqrt(D)
    rope: bool = False  # block mode: rotary embedding of Q and K fused into the kernels
    seed: Optional[int] = None  # canonical seed; None = the workload index
    mxfp8: bool = False  # inputs quantised to MXFP8 (32 x 32 blocks) and MXFP8 products


WORKLOADS = {
    0: Workload("tiny_self_f32", 4, 2, 32, "f32", ACT_SOFTMAX, False, False, False, "f32", "f32", False),
    1: Workload("jfa_self_bias", 256, 4, 128, "bf16", ACT_SOFTMAX, False, True, True, "bf16", "bf16", False),
    2: Workload("cross_longq_shortkv", 512, 8, 64, "bf16", ACT_SOFTMAX, False, False, False, "bf16", "f32", True),
    3: Workload("gdpa_pma_gelu", 256, 8, 128, "bf16", ACT_GELU, False, False, False, "f32", "f32", True),
    4: Workload("block_attention_64", 64, 4, 128, "bf16", ACT_SOFTMAX, True, False, False, "bf16", "bf16", False),
    # sliding-window self-attention over long sequences (lengths as workload 4)
    5: Workload("swa_long_w256", 64, 4, 128, "bf16", ACT_SOFTMAX, False, False, False, "bf16", "bf16", False,
                window=(256, 256)),
    # pooled multi-head attention shapes (as workload 3) with QK-norm and the
    # ALU-only polynomial GELU; scale 1, so every score is a cosine in [-1, 1]
    6: Workload("gdpa_qknorm_gelu_poly", 256, 8, 128, "bf16", ACT_GELU_POLY, False, False, False, "f32", "f32",
                True, qk_norm=True, scale=1.0),
    # BlockAttention (workload 4's shapes) with the rotary embedding fused in
    7: Workload("block_attention_64_rope", 64, 4, 128, "bf16", ACT_SOFTMAX, True, False, False, "bf16", "bf16",
                False, rope=True),
    # workload 1 without the bias (and dBias): the forward is no longer
    # bound by the bias stream
    8: Workload("jfa_self_nobias", 256, 4, 128, "bf16", ACT_SOFTMAX, False, False, False, "bf16", "bf16", False,
                seed=1),
    # workload 8 in MXFP8: Q, K, V, dO quantised in 32 x 32 blocks, MXFP8
    # products forward and backward, fp32 outputs and gradients
    9: Workload("jfa_self_mxfp8", 256, 4, 128, "bf16", ACT_SOFTMAX, False, False, False, "f32", "f32", False,
                seed=1, mxfp8=True),
}


# ----------------------------------------------------------------------------
# bf16 <-> fp32 bit conversions (data format only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 view of a generated array (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# lengths
# ----------------------------------------------------------------------------
def _lognormal_lengths(rng, n, median, lo, hi):
    x = np.exp(np.log(float(median)) + rng.standard_normal(n))
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def make_lengths(cfg: int, seed: int):
    """Per-sample (lq, lk) for workload ``cfg`` drawn from ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    return _lengths_from(rng, cfg)


def _lengths_from(rng, cfg):
    w = WORKLOADS[cfg]
    if cfg == 0:
        lq = rng.integers(1, 65, w.B).astype(np.int64)
        lq[1] = 0  # one zero-length sample
        return lq, lq.copy()
    if cfg in (1, 8, 9):
        lq = _lognormal_lengths(rng, w.B, 300, 8, 1000)
        return lq, lq.copy()
    if cfg == 2:
        lq = _lognormal_lengths(rng, w.B, 500, 16, 2000)
        lk = rng.integers(16, 65, w.B).astype(np.int64)
        return lq, lk
    if cfg in (3, 6):
        lq = np.full(w.B, 32, dtype=np.int64)
        lk = _lognormal_lengths(rng, w.B, 1500, 64, 4000)
        return lq, lk
    if cfg in (4, 5, 7):
        lq = rng.integers(2048, 16385, w.B).astype(np.int64)
        return lq, lq.copy()
    raise ValueError(f"unknown workload {cfg}")


def offsets_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(lengths.shape[0] + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    return off


# ----------------------------------------------------------------------------
# values
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class JaggedInputs:
    """Generated inputs; value arrays are uint16 bf16 bits or float32."""

    B: int
    H: int
    D: int
    dtype: str
    q_offsets: np.ndarray
    kv_offsets: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    bias: Optional[np.ndarray]
    dout: Optional[np.ndarray]

    @property
    def lq(self):
        return np.diff(self.q_offsets)

    @property
    def lk(self):
        return np.diff(self.kv_offsets)

    def f64(self, name: str) -> Optional[np.ndarray]:
        a = getattr(self, name)
        return None if a is None else to_f64(a, self.dtype)


def _values(rng, shape, dtype, std=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def bias_elements(lq, lk, H) -> int:
    return int(H * np.sum(np.asarray(lq, np.int64) * np.asarray(lk, np.int64)))


def generate(lq, lk, H, D, dtype, *, rng, bias=False, bias_std=0.1, dout=True) -> JaggedInputs:
    """Draw Q, K, V (then bias, then dO) for the given per-sample lengths."""
    lq = np.asarray(lq, dtype=np.int64)
    lk = np.asarray(lk, dtype=np.int64)
    q_off = offsets_from_lengths(lq)
    kv_off = offsets_from_lengths(lk)
    Tq, Tk = int(q_off[-1]), int(kv_off[-1])
    q = _values(rng, (Tq, H, D), dtype)
    k = _values(rng, (Tk, H, D), dtype)
    v = _values(rng, (Tk, H, D), dtype)
    b = _values(rng, (bias_elements(lq, lk, H),), dtype, bias_std) if bias else None
    do = _values(rng, (Tq, H, D), dtype) if dout else None
    return JaggedInputs(len(lq), H, D, dtype, q_off, kv_off, q, k, v, b, do)


def make_inputs(cfg: int, seed: Optional[int] = None, dout: bool = True) -> JaggedInputs:
    """Inputs of workload ``cfg``; the canonical seed is the config index."""
    w = WORKLOADS[cfg]
    if seed is None:
        seed = cfg if w.seed is None else w.seed
    rng = np.random.default_rng(seed)
    lq, lk = _lengths_from(rng, cfg)
    return generate(lq, lk, w.H, w.D, w.dtype, rng=rng, bias=w.bias, dout=dout)


def make_custom(lq, lk, H, D, dtype="bf16", *, seed=0, bias=False, dout=True) -> JaggedInputs:
    """Inputs for explicit lengths (edge cases), same value distributions."""
    rng = np.random.default_rng(seed)
    return generate(lq, lk, H, D, dtype, rng=rng, bias=bias, dout=dout)
