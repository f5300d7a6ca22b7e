"""Torch-facing helper around the C ABI: owns a plan and its device workspace,
allocates outputs, and passes raw pointers plus the current HIP stream.
PyTorch supplies memory and streams only; all computation is in libjattn.so.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

from . import binding as _b

_ACT = {"softmax": _b.JATTN_SOFTMAX, "gelu": _b.JATTN_GELU_ERF, "silu": _b.JATTN_SILU,
        "gelu_poly": _b.JATTN_GELU_POLY}
_DT = {"bf16": _b.JATTN_BF16, "f32": _b.JATTN_F32, "mxfp8": _b.JATTN_MXFP8}
_TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
_ORDER = {"heavy_first": _b.JATTN_HEAVY_FIRST, "zigzag": _b.JATTN_ZIGZAG, "lpt": _b.JATTN_LPT}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _args(*specs):
    """Pointers of the tensors the library reads or writes, each spec being
    (tensor or None, name, dtype, elements the call touches).  The C ABI takes
    bare pointers, so a tensor of the wrong type or with too few elements is
    refused here (a kernel would read or write past its end): types and sizes
    of all tensors first, then that each is a contiguous device tensor."""
    for t, name, dtype, numel in specs:
        if t is None:
            continue
        if t.dtype != _TORCH_DT[dtype]:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {_TORCH_DT[dtype]}")
        if t.numel() < numel:
            raise ValueError(f"{name}: {t.numel()} elements, the plan needs {numel}")
    for t, name, _, _ in specs:
        if t is not None and t.device.type != "cuda":
            raise ValueError(f"{name}: must be a device tensor")
    return [_ptr(t) for t, _, _, _ in specs]


class MxTensor:
    """An MXFP8 tensor (include/jattn.h): E4M3 codes [T, H, D], the same codes
    per 32-token block feature-major [RB, H, D, 32] (or None), and the E8M0
    block scales [RB, H, D/32], all uint8 device tensors."""

    def __init__(self, codes, codes_t, scales):
        self.codes, self.codes_t, self.scales = codes, codes_t, scales

    def c(self) -> "_b.jattn_mx_tensor":
        return _b.jattn_mx_tensor(self.codes.data_ptr(), self.codes_t.data_ptr() if self.codes_t is not None else None,
                                  self.scales.data_ptr())


class JaggedAttention:
    """One jagged batch layout (offsets + options) bound to a plan.

    Values are [T, H, D] tensors with samples concatenated along T; the
    offsets are host int64 arrays [B + 1].  Options map one to one onto the
    C descriptor (include/jattn.h):
      act            "softmax", "gelu" (erf GELU), "silu", or "gelu_poly" (the
                     ALU-only polynomial GELU, meant for QK-normed inputs)
      block_diagonal fixed 64-token blocks (BlockAttention); with rope=True the
                     rotary embedding of Q and K is fused into the block kernels
                     (rope_base <= 0 selects 10000)
      window         (left, right): sliding window, query i sees keys
                     i - left .. i + right of its own sample (lq == lk)
      has_bias / want_dbias, dtypes, order and num_workers of the plan.
      split_operands hi + lo bf16 operands for the P / dS products.  Default
                     (None): on for the GDPA activations, whose unnormalised
                     P V over long key sets errs by up to 2^-8 sum|P||V| with
                     plain bf16 P (about 0.15 at 4000 keys), off for softmax.
    forward() returns (O, LSE); backward() returns (dQ, dK, dV, dBias).  QK-norm
    itself is qk_norm() / qk_norm_backward() below.
    """

    def __init__(self, q_offsets, kv_offsets, H: int, D: int, *, act: str = "softmax",
                 block_diagonal: bool = False, has_bias: bool = False, want_dbias: bool = False,
                 in_dtype: str = "bf16", out_dtype: Optional[str] = None,
                 grad_dtype: Optional[str] = None, split_operands: Optional[bool] = None,
                 order: str = "zigzag", num_workers: int = 0, scale: Optional[float] = None,
                 dbias_dtype: Optional[str] = None, window: Optional[tuple] = None, rope: bool = False,
                 rope_base: float = 0.0, device="cuda"):
        q_offsets = np.asarray(q_offsets, dtype=np.int64)
        kv_offsets = np.asarray(kv_offsets, dtype=np.int64)
        self.B = len(q_offsets) - 1
        self.H, self.D = H, D
        self.act = act
        self.in_dtype = in_dtype
        self.out_dtype = out_dtype or ("bf16" if in_dtype == "mxfp8" else in_dtype)
        self.grad_dtype = grad_dtype or ("bf16" if in_dtype == "mxfp8" else in_dtype)
        self.dbias_dtype = dbias_dtype or self.grad_dtype
        self.has_bias, self.want_dbias = has_bias, want_dbias
        self.block_diagonal = block_diagonal
        self.window = None if window is None else (int(window[0]), int(window[1]))
        self.scale = (1.0 / math.sqrt(D)) if scale is None else scale
        self.device = torch.device(device)
        d = _b.jattn_desc()
        d.B, d.H, d.D, d.scale = self.B, H, D, self.scale
        d.act = _ACT[act]
        d.mask = _b.JATTN_MASK_BLOCKDIAG64 if block_diagonal else _b.JATTN_MASK_NONE
        if self.window is not None:
            d.mask = _b.JATTN_MASK_WINDOW
            d.window_left, d.window_right = self.window
        self.rope = bool(rope)
        d.rope, d.rope_base = int(rope), float(rope_base)
        d.has_bias, d.want_dbias = int(has_bias), int(want_dbias)
        d.in_dtype, d.out_dtype, d.grad_dtype = _DT[in_dtype], _DT[self.out_dtype], _DT[self.grad_dtype]
        if split_operands is None:
            split_operands = act != "softmax"
        self.split_operands = bool(split_operands)
        d.split_operands = int(split_operands)
        d.order = _ORDER[order]
        d.num_workers = num_workers
        d.dbias_dtype = _DT[self.dbias_dtype]
        self.desc = d
        self.plan = _b.jattn_plan_create(d, q_offsets, kv_offsets)
        self.info = _b.jattn_plan_info(self.plan)
        self.Tq, self.Tk = int(self.info.Tq), int(self.info.Tk)
        self.workspace = None

    def upload(self, stream=None):
        """Allocate the workspace on the device and copy the plan into it."""
        nbytes = int(self.info.workspace_bytes)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        st = stream if stream is not None else torch.cuda.current_stream(self.device).cuda_stream
        _b.jattn_plan_upload(self.plan, self.workspace.data_ptr(), self.workspace.numel(), st)
        return self

    def _stream(self):
        """The current stream, on which the call is enqueued.  The workspace
        was allocated on the stream current at upload(); recording this one
        keeps the caching allocator from handing its memory out again while
        work enqueued here may still read it."""
        cur = torch.cuda.current_stream(self.device)
        self.workspace.record_stream(cur)
        return cur.cuda_stream

    def _inputs(self, q, k, v, bias):
        nq, nk = self.Tq * self.H * self.D, self.Tk * self.H * self.D
        nb = int(self.info.bias_elems) if self.has_bias else 0
        return [(q, "q", self.in_dtype, nq), (k, "k", self.in_dtype, nk), (v, "v", self.in_dtype, nk),
                (bias, "bias", self.in_dtype, nb)]

    def forward(self, q, k, v, bias=None, o=None, lse=None, want_lse=True):
        pq, pk, pv, pb, _, _ = _args(*self._inputs(q, k, v, bias), (o, "o", self.out_dtype, self.Tq * self.H * self.D),
                                     (lse, "lse", "f32", self.Tq * self.H))
        if self.workspace is None:
            self.upload()
        if o is None:
            o = torch.empty(self.Tq, self.H, self.D, dtype=_TORCH_DT[self.out_dtype], device=self.device)
        if lse is None and want_lse and self.act == "softmax" and not self.block_diagonal:
            lse = torch.empty(self.Tq, self.H, dtype=torch.float32, device=self.device)
        _b.jattn_fwd(self.plan, pq, pk, pv, pb, _ptr(o), _ptr(lse), self.workspace.data_ptr(), self._stream())
        return o, lse

    def backward(self, q, k, v, dout, o=None, lse=None, bias=None, dq=None, dk=None, dv=None, dbias=None,
                 stages=_b.JATTN_BWD_ALL):
        nq, nk = self.Tq * self.H * self.D, self.Tk * self.H * self.D
        pq, pk, pv, pb = _args(*self._inputs(q, k, v, bias), (o, "o", self.out_dtype, nq),
                               (lse, "lse", "f32", self.Tq * self.H), (dout, "dout", self.in_dtype, nq),
                               (dq, "dq", self.grad_dtype, nq), (dk, "dk", self.grad_dtype, nk),
                               (dv, "dv", self.grad_dtype, nk),
                               (dbias, "dbias", self.dbias_dtype,
                                int(self.info.bias_elems) if self.want_dbias else 0))[:4]
        if self.workspace is None:
            self.upload()
        gdt = _TORCH_DT[self.grad_dtype]
        dq = dq if dq is not None else torch.empty(self.Tq, self.H, self.D, dtype=gdt, device=self.device)
        dk = dk if dk is not None else torch.empty(self.Tk, self.H, self.D, dtype=gdt, device=self.device)
        dv = dv if dv is not None else torch.empty(self.Tk, self.H, self.D, dtype=gdt, device=self.device)
        if self.want_dbias and dbias is None:
            dbias = torch.empty(int(self.info.bias_elems), dtype=_TORCH_DT[self.dbias_dtype], device=self.device)
        args = (pq, pk, pv, pb, _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                _ptr(dv), _ptr(dbias), self.workspace.data_ptr(), self._stream())
        if stages == _b.JATTN_BWD_ALL:
            _b.jattn_bwd(self.plan, *args)
        else:
            _b.jattn_bwd_stages(self.plan, stages, *args)
        return dq, dk, dv, dbias

    # ---- MXFP8 ("Mixed Ultra-Low-Precision Training": low-precision attention) ----
    def mx_empty(self, rows: str = "q", transposed: bool = True) -> MxTensor:
        """Device buffers for an MXFP8 tensor with the plan's query ("q") or
        key/value ("kv") rows."""
        nc, nt, ns = _b.jattn_mx_sizes(self.plan, _b.JATTN_MX_Q if rows == "q" else _b.JATTN_MX_KV)
        u8 = dict(dtype=torch.uint8, device=self.device)
        return MxTensor(torch.empty(max(nc, 16), **u8), torch.empty(max(nt, 16), **u8) if transposed else None,
                        torch.empty(max(ns, 16), **u8))

    def mx_quantize(self, x: torch.Tensor, rows: str = "q", transposed: bool = True,
                    out: Optional[MxTensor] = None) -> MxTensor:
        """Quantise a bf16 [T, H, D] tensor with the plan's query ("q") or
        key/value ("kv") rows into an MXFP8 tensor (library kernel)."""
        which = _b.JATTN_MX_Q if rows == "q" else _b.JATTN_MX_KV
        T = self.Tq if rows == "q" else self.Tk
        nc, nt, ns = _b.jattn_mx_sizes(self.plan, which)
        px = _args((x, "x", "bf16", T * self.H * self.D))[0]
        if self.workspace is None:
            self.upload()
        m = out if out is not None else self.mx_empty(rows, transposed)
        if m.codes.numel() < nc or m.scales.numel() < ns or (m.codes_t is not None and m.codes_t.numel() < nt):
            raise ValueError("MXFP8 output buffers are smaller than the plan needs")
        _b.jattn_mx_quantize(self.plan, which, px, m.c(), self.workspace.data_ptr(), self._stream())
        return m

    def mx_forward(self, q: MxTensor, k: MxTensor, v: MxTensor, o=None, lse=None, want_lse=True):
        """MXFP8 forward on quantised Q, K, V (q.codes, k.codes, v.codes_t)."""
        _args((o, "o", self.out_dtype, self.Tq * self.H * self.D), (lse, "lse", "f32", self.Tq * self.H))
        if self.workspace is None:
            self.upload()
        if o is None:
            o = torch.empty(self.Tq, self.H, self.D, dtype=_TORCH_DT[self.out_dtype], device=self.device)
        if lse is None and want_lse and self.act == "softmax":
            lse = torch.empty(self.Tq, self.H, dtype=torch.float32, device=self.device)
        _b.jattn_mx_fwd(self.plan, q.c(), k.c(), v.c(), _ptr(o), _ptr(lse), self.workspace.data_ptr(),
                        self._stream())
        return o, lse

    def mx_backward(self, q: MxTensor, k: MxTensor, v: MxTensor, dout: MxTensor, o=None, lse=None, dq=None,
                    dk=None, dv=None, stages=_b.JATTN_BWD_ALL):
        """MXFP8 backward (include/jattn.h, jattn_mx_bwd); returns (dQ, dK, dV)."""
        nq, nk = self.Tq * self.H * self.D, self.Tk * self.H * self.D
        _args((o, "o", self.out_dtype, nq), (lse, "lse", "f32", self.Tq * self.H),
              (dq, "dq", self.grad_dtype, nq), (dk, "dk", self.grad_dtype, nk), (dv, "dv", self.grad_dtype, nk))
        if self.workspace is None:
            self.upload()
        gdt = _TORCH_DT[self.grad_dtype]
        dq = dq if dq is not None else torch.empty(self.Tq, self.H, self.D, dtype=gdt, device=self.device)
        dk = dk if dk is not None else torch.empty(self.Tk, self.H, self.D, dtype=gdt, device=self.device)
        dv = dv if dv is not None else torch.empty(self.Tk, self.H, self.D, dtype=gdt, device=self.device)
        _b.jattn_mx_bwd(self.plan, stages, q.c(), k.c(), v.c(), _ptr(o), _ptr(lse), dout.c(), _ptr(dq), _ptr(dk),
                        _ptr(dv), self.workspace.data_ptr(), self._stream())
        return dq, dk, dv

    def __del__(self):
        try:
            _b.jattn_plan_destroy(self.plan)
        except Exception:
            pass


_DT_OF = {torch.bfloat16: "bf16", torch.float32: "f32"}


def qk_norm(x: torch.Tensor, out_dtype: Optional[str] = None, out: Optional[torch.Tensor] = None,
            rnorm: Optional[torch.Tensor] = None):
    """QK-norm forward: each row x[..., :] (last dim D) scaled to unit L2 length
    by the library's kernel.  Returns (y, rnorm) with rnorm = 1 / max(||x||, eps)."""
    D = x.shape[-1]
    rows = x.numel() // D
    xdt = _DT_OF[x.dtype]
    odt = out_dtype or (_DT_OF[out.dtype] if out is not None else xdt)
    px = _args((x, "x", xdt, x.numel()), (out, "out", odt, x.numel()), (rnorm, "rnorm", "f32", rows))[0]
    y = out if out is not None else torch.empty(x.shape, dtype=_TORCH_DT[odt], device=x.device)
    r = rnorm if rnorm is not None else torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _b.jattn_l2norm_fwd(px, _ptr(y), _ptr(r), rows, D, _DT[xdt], _DT[odt],
                        torch.cuda.current_stream(x.device).cuda_stream)
    return y, r


def qk_norm_backward(x: torch.Tensor, dy: torch.Tensor, out_dtype: Optional[str] = None,
                     out: Optional[torch.Tensor] = None):
    """QK-norm backward: dL/dx from the forward input x and dL/dy."""
    D = x.shape[-1]
    rows = x.numel() // D
    xdt, gdt = _DT_OF[x.dtype], _DT_OF[dy.dtype]
    odt = out_dtype or (_DT_OF[out.dtype] if out is not None else gdt)
    px, pdy, _ = _args((x, "x", xdt, x.numel()), (dy, "dy", gdt, x.numel()), (out, "out", odt, x.numel()))
    dx = out if out is not None else torch.empty(x.shape, dtype=_TORCH_DT[odt], device=x.device)
    _b.jattn_l2norm_bwd(px, pdy, _ptr(dx), rows, D, _DT[xdt], _DT[gdt],
                        _DT[odt], torch.cuda.current_stream(x.device).cuda_stream)
    return dx


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Host array from inputs.py (bf16 bits or float32) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> exact float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()
