"""The torch binding refuses a tensor that does not match the plan (dtype,
element count, device) before any pointer reaches the library: the C ABI takes
bare pointers, so such a tensor would otherwise be read or written past its end
on the GPU. CPU only: every check fires before a device is touched."""
import pytest
import torch

from jagged_variable_length_amd import attention as A

H, D = 2, 64


def _op(**kw):
    return A.JaggedAttention([0, 5, 12], [0, 7, 9], H, D, **kw)


def _t(n, dtype=torch.bfloat16):
    return torch.zeros(n, dtype=dtype)


def _sizes(op):
    return op.Tq * H * D, op.Tk * H * D


def test_forward_refuses_a_wrong_dtype():
    op = _op()
    nq, nk = _sizes(op)
    with pytest.raises(ValueError, match="q: dtype"):
        op.forward(_t(nq, torch.float32), _t(nk), _t(nk))


def test_forward_refuses_too_few_elements():
    op = _op()
    nq, nk = _sizes(op)
    with pytest.raises(ValueError, match="k: .* elements"):
        op.forward(_t(nq), _t(nk - 1), _t(nk))
    with pytest.raises(ValueError, match="o: .* elements"):
        op.forward(_t(nq), _t(nk), _t(nk), o=_t(nq - D))
    with pytest.raises(ValueError, match="lse: .* elements"):
        op.forward(_t(nq), _t(nk), _t(nk), lse=_t(op.Tq * H - 1, torch.float32))


def test_forward_refuses_a_short_bias():
    op = _op(has_bias=True)
    nq, nk = _sizes(op)
    nb = int(op.info.bias_elems)
    assert nb == H * (5 * 7 + 7 * 2)
    with pytest.raises(ValueError, match="bias: .* elements"):
        op.forward(_t(nq), _t(nk), _t(nk), bias=_t(nb - 1))


def test_forward_refuses_host_tensors():
    op = _op()
    nq, nk = _sizes(op)
    with pytest.raises(ValueError, match="q: must be a device tensor"):
        op.forward(_t(nq), _t(nk), _t(nk))


def test_backward_checks_every_gradient():
    op = _op(has_bias=True, want_dbias=True, grad_dtype="f32", dbias_dtype="f32")
    nq, nk = _sizes(op)
    nb = int(op.info.bias_elems)
    f32 = torch.float32
    base = dict(o=_t(nq), lse=_t(op.Tq * H, f32), bias=_t(nb))
    with pytest.raises(ValueError, match="dout: .* elements"):
        op.backward(_t(nq), _t(nk), _t(nk), _t(nq - 1), **base)
    with pytest.raises(ValueError, match="dq: dtype"):
        op.backward(_t(nq), _t(nk), _t(nk), _t(nq), dq=_t(nq), **base)
    with pytest.raises(ValueError, match="dv: .* elements"):
        op.backward(_t(nq), _t(nk), _t(nk), _t(nq), dv=_t(nk - 1, f32), **base)
    with pytest.raises(ValueError, match="dbias: dtype"):
        op.backward(_t(nq), _t(nk), _t(nk), _t(nq), dbias=_t(nb), **base)
    with pytest.raises(ValueError, match="dbias: .* elements"):
        op.backward(_t(nq), _t(nk), _t(nk), _t(nq), dbias=_t(nb - 1, f32), **base)


def test_qk_norm_refuses_short_outputs():
    x = torch.zeros(10, H, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out: .* elements"):
        A.qk_norm(x, out=torch.zeros(9, H, D, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="rnorm: .* elements"):
        A.qk_norm(x, rnorm=torch.zeros(10 * H - 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="dy: .* elements"):
        A.qk_norm_backward(x, torch.zeros(9, H, D, dtype=torch.float32))
    with pytest.raises(ValueError, match="x: must be a device tensor"):
        A.qk_norm(x)
