"""CPU-only checks of the C ABI: the library loads, exports what the header
declares, validates its arguments on the host, and plans bit-exactly like the
reference planner.  No GPU call is made here."""
import ctypes
import os
import re

import numpy as np
import pytest

from jagged_variable_length_amd import binding as B
from jagged_variable_length_amd import inputs as gen
from oracle import plan as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libjattn.so not built (run python -m jagged_variable_length_amd.build)")
    return B.lib()


def _header_functions():
    text = open(os.path.join(ROOT, "include", "jattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(jattn_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported(lib):
    names = _header_functions()
    assert set(names) == set(B.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_strerror_covers_codes(lib):
    for code in range(0, -10, -1):
        assert B.jattn_strerror(code) != "unknown status"
    assert B.jattn_strerror(-100) == "unknown status"


def _desc(**kw):
    d = B.jattn_desc()
    d.B, d.H, d.D = kw.get("B", 2), kw.get("H", 2), kw.get("D", 64)
    d.scale = kw.get("scale", 0.0)
    d.act = kw.get("act", B.JATTN_SOFTMAX)
    d.mask = kw.get("mask", B.JATTN_MASK_NONE)
    d.has_bias = kw.get("has_bias", 0)
    d.want_dbias = kw.get("want_dbias", 0)
    d.in_dtype = kw.get("in_dtype", B.JATTN_BF16)
    d.out_dtype = kw.get("out_dtype", B.JATTN_BF16)
    d.grad_dtype = kw.get("grad_dtype", B.JATTN_BF16)
    d.split_operands = kw.get("split", 0)
    d.order = kw.get("order", B.JATTN_HEAVY_FIRST)
    d.num_workers = kw.get("num_workers", 0)
    d.window_left, d.window_right = kw.get("window", (0, 0))
    d.rope, d.rope_base = kw.get("rope", 0), kw.get("rope_base", 0.0)
    d.dbias_dtype = kw.get("dbias_dtype", B.JATTN_BF16)
    return d


@pytest.mark.parametrize("kw,qo,ko,code", [
    (dict(), [1, 3, 5], [0, 2, 4], B.JATTN_E_OFFSETS),        # offsets[0] != 0
    (dict(), [0, 3, 2], [0, 2, 4], B.JATTN_E_OFFSETS),        # decreasing
    (dict(), [0, 3, 2 ** 31], [0, 2, 4], B.JATTN_E_OFFSETS),  # total >= 2^31
    (dict(D=48), [0, 3, 5], [0, 2, 4], B.JATTN_E_SHAPE),
    (dict(H=0), [0, 3, 5], [0, 2, 4], B.JATTN_E_SHAPE),
    (dict(B=-1), [0], [0], B.JATTN_E_SHAPE),
    (dict(mask=B.JATTN_MASK_BLOCKDIAG64), [0, 3, 5], [0, 2, 4], B.JATTN_E_SHAPE),  # lq != lk
    (dict(act=7), [0, 3, 5], [0, 3, 5], B.JATTN_E_UNSUPPORTED),
    (dict(in_dtype=B.JATTN_F32), [0, 3, 5], [0, 3, 5], B.JATTN_E_UNSUPPORTED),  # f32 in, bf16 out
    (dict(in_dtype=B.JATTN_F32, out_dtype=B.JATTN_F32, grad_dtype=B.JATTN_F32, D=128),
     [0, 3, 5], [0, 3, 5], B.JATTN_E_UNSUPPORTED),
    (dict(want_dbias=1), [0, 3, 5], [0, 3, 5], B.JATTN_E_ARG),
    (dict(order=9), [0, 3, 5], [0, 3, 5], B.JATTN_E_ARG),
    (dict(mask=B.JATTN_MASK_BLOCKDIAG64, act=B.JATTN_GELU_ERF), [0, 3, 5], [0, 3, 5], B.JATTN_E_UNSUPPORTED),
    (dict(mask=B.JATTN_MASK_BLOCKDIAG64, has_bias=1), [0, 3, 5], [0, 3, 5], B.JATTN_E_UNSUPPORTED),
    (dict(mask=B.JATTN_MASK_BLOCKDIAG64, in_dtype=B.JATTN_F32, out_dtype=B.JATTN_F32, grad_dtype=B.JATTN_F32),
     [0, 3, 5], [0, 3, 5], B.JATTN_E_UNSUPPORTED),
    (dict(mask=B.JATTN_MASK_BLOCKDIAG64, num_workers=7), [0, 3, 5], [0, 3, 5], B.JATTN_E_ARG),
    (dict(mask=3), [0, 3, 5], [0, 3, 5], B.JATTN_E_UNSUPPORTED),
    (dict(mask=B.JATTN_MASK_WINDOW), [0, 3, 5], [0, 2, 4], B.JATTN_E_SHAPE),  # lq != lk
    (dict(mask=B.JATTN_MASK_WINDOW, window=(-1, 4)), [0, 3, 5], [0, 3, 5], B.JATTN_E_ARG),
    (dict(mask=B.JATTN_MASK_WINDOW, window=(4, -2)), [0, 3, 5], [0, 3, 5], B.JATTN_E_ARG),
    (dict(mask=B.JATTN_MASK_WINDOW, in_dtype=B.JATTN_F32, out_dtype=B.JATTN_F32, grad_dtype=B.JATTN_F32),
     [0, 3, 5], [0, 3, 5], B.JATTN_E_UNSUPPORTED),
    (dict(mask=B.JATTN_MASK_WINDOW, has_bias=1, want_dbias=1), [0, 3, 5], [0, 3, 5], B.JATTN_E_UNSUPPORTED),
    (dict(act=B.JATTN_GELU_POLY, in_dtype=B.JATTN_F32, out_dtype=B.JATTN_F32, grad_dtype=B.JATTN_F32),
     [0, 3, 5], [0, 3, 5], B.JATTN_E_UNSUPPORTED),
    (dict(act=4), [0, 3, 5], [0, 3, 5], B.JATTN_E_UNSUPPORTED),
    (dict(rope=1), [0, 3, 5], [0, 3, 5], B.JATTN_E_UNSUPPORTED),  # RoPE needs block mode
    (dict(rope=2, mask=B.JATTN_MASK_BLOCKDIAG64), [0, 3, 5], [0, 3, 5], B.JATTN_E_ARG),
    (dict(rope=1, rope_base=0.5, mask=B.JATTN_MASK_BLOCKDIAG64), [0, 3, 5], [0, 3, 5], B.JATTN_E_ARG),
])
def test_plan_create_rejects(lib, kw, qo, ko, code):
    d = _desc(**kw)
    with pytest.raises(B.JattnError) as e:
        B.jattn_plan_create(d, qo, ko)
    assert e.value.code == code
    assert B.jattn_last_error() != ""


@pytest.mark.parametrize("kw,L,ok", [
    # one sample's rows must span < 2^31 bytes (H * D * 2 = 512 bytes a bf16 row) ...
    (dict(B=1, H=2, D=128), (1 << 22) - 1, True),
    (dict(B=1, H=2, D=128), 1 << 22, False),
    # ... in its widest type: fp32 outputs or gradients make a row 1024 bytes
    (dict(B=1, H=2, D=128, out_dtype=B.JATTN_F32), (1 << 21) - 1, True),
    (dict(B=1, H=2, D=128, out_dtype=B.JATTN_F32), 1 << 21, False),
    (dict(B=1, H=2, D=128, grad_dtype=B.JATTN_F32), 1 << 21, False),
    # a head's bf16 bias block must span < 2^30 bytes: 23170^2 * 2 < 2^30 <= 23171^2 * 2
    (dict(B=1, has_bias=1), 23170, True),
    (dict(B=1, has_bias=1), 23171, False),
    # a head's fp32 dBias block must span < 2^30 bytes: 16383^2 * 4 < 2^30 = 16384^2 * 4
    (dict(B=1, has_bias=1, want_dbias=1, dbias_dtype=B.JATTN_F32), 16383, True),
    (dict(B=1, has_bias=1, want_dbias=1, dbias_dtype=B.JATTN_F32), 16384, False),
    (dict(B=1, has_bias=1, want_dbias=1), 23170, True),
])
def test_per_sample_size_limits(lib, kw, L, ok):
    """The largest per-sample sizes are accepted, one more row is refused
    (every per-(sample, head) byte offset stays inside the 32-bit range of a
    buffer descriptor); plan creation is host-only."""
    d = _desc(**kw)
    if ok:
        p = B.jattn_plan_create(d, [0, L], [0, L])
        B.jattn_plan_destroy(p)
    else:
        with pytest.raises(B.JattnError) as e:
            B.jattn_plan_create(d, [0, L], [0, L])
        assert e.value.code == B.JATTN_E_SHAPE


def test_null_arguments(lib):
    out = ctypes.c_void_p()
    qo = np.array([0, 1], np.int64)
    assert lib.jattn_plan_create(None, qo.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                 qo.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ctypes.byref(out)) == B.JATTN_E_NULL
    d = _desc(B=1)
    assert lib.jattn_plan_create(ctypes.byref(d), None, None, ctypes.byref(out)) == B.JATTN_E_NULL
    assert lib.jattn_plan_info(None, None) == B.JATTN_E_NULL
    assert lib.jattn_fwd(None, None, None, None, None, None, None, None, None) == B.JATTN_E_NULL
    assert lib.jattn_bwd(*([None] * 14)) == B.JATTN_E_NULL


def test_launch_validation_never_touches_gpu(lib):
    """Bad pointers are rejected on the host before any HIP call."""
    d = _desc(B=2, H=2, D=64)
    p = B.jattn_plan_create(d, [0, 3, 5], [0, 2, 4])
    try:
        fake = 0x10000000  # never dereferenced: validation fails first
        with pytest.raises(B.JattnError) as e:
            B.jattn_fwd(p, fake, fake, fake, None, fake, None, None, None)  # no workspace
        assert e.value.code == B.JATTN_E_WORKSPACE
        with pytest.raises(B.JattnError) as e:
            B.jattn_fwd(p, fake + 2, fake, fake, None, fake, None, fake, None)  # misaligned q
        assert e.value.code == B.JATTN_E_ALIGN
        with pytest.raises(B.JattnError) as e:
            B.jattn_fwd(p, None, fake, fake, None, fake, None, fake, None)
        assert e.value.code == B.JATTN_E_NULL
        with pytest.raises(B.JattnError) as e:
            B.jattn_plan_upload(p, fake, 16, None)  # too small
        assert e.value.code == B.JATTN_E_WORKSPACE
    finally:
        B.jattn_plan_destroy(p)


def test_bias_required_when_declared(lib):
    d = _desc(B=2, H=2, D=64, has_bias=1)
    p = B.jattn_plan_create(d, [0, 3, 5], [0, 2, 4])
    try:
        fake = 0x10000000
        with pytest.raises(B.JattnError) as e:
            B.jattn_fwd(p, fake, fake, fake, None, fake, None, fake, None)
        assert e.value.code == B.JATTN_E_NULL
    finally:
        B.jattn_plan_destroy(p)


# ---------------------------------------------------------------------------
# plans: bit-exact against the reference planner
# ---------------------------------------------------------------------------
def _compare_plan(p, lq, lk, H, block):
    info = B.jattn_plan_info(p)
    parts = [("block", B.JATTN_PLAN_BLOCK, info.block)] if block else [
        ("fwd", B.JATTN_PLAN_FWD, info.fwd), ("dkdv", B.JATTN_PLAN_DKDV, info.dkdv),
        ("dq", B.JATTN_PLAN_DQ, info.dq)]
    return info, parts


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("order", ["heavy_first", "zigzag", "lpt"])
def test_plans_match_reference_planner(lib, cfg, order):
    w = gen.WORKLOADS[cfg]
    lq, lk = gen.make_lengths(cfg, cfg)
    qo, ko = gen.offsets_from_lengths(lq), gen.offsets_from_lengths(lk)
    d = _desc(B=w.B, H=w.H, D=w.D, act={"softmax": 0, "gelu": 1, "silu": 2}[w.act],
              mask=1 if w.block_diagonal else 0, has_bias=int(w.bias), want_dbias=int(w.want_dbias),
              in_dtype=B.JATTN_F32 if w.dtype == "f32" else B.JATTN_BF16,
              out_dtype=B.JATTN_F32 if w.out_dtype == "f32" else B.JATTN_BF16,
              grad_dtype=B.JATTN_F32 if w.grad_dtype == "f32" else B.JATTN_BF16,
              order={"heavy_first": 0, "zigzag": 1, "lpt": 2}[order], num_workers=0 if cfg else 7)
    p = B.jattn_plan_create(d, qo, ko)
    try:
        info, parts = _compare_plan(p, lq, lk, w.H, w.block_diagonal)
        assert info.Tq == qo[-1] and info.Tk == ko[-1]
        for kind, which, kp in parts:
            units = B.jattn_plan_export(p, which * 2 + 0).reshape(-1, 4)
            offs = B.jattn_plan_export(p, which * 2 + 1)
            ref_units, ref_offs = P.plan(kind, lq.tolist(), lk.tolist(), w.H, kp.tile_rows, kp.step_rows,
                                         kp.num_workers, order)
            assert kp.n_units == len(ref_units)
            np.testing.assert_array_equal(units, np.array(ref_units, dtype=np.int32).reshape(-1, 4))
            np.testing.assert_array_equal(offs, np.array(ref_offs, dtype=np.int32))
        pairs = sum(min(64, l - s) ** 2 for l in lq for s in range(0, l, 64)) if w.block_diagonal \
            else int(np.sum(lq * lk))
        assert info.flops_fwd == pytest.approx(4.0 * w.H * w.D * pairs, rel=1e-12)
    finally:
        B.jattn_plan_destroy(p)


@pytest.mark.parametrize("seed", range(6))
def test_random_plans_match(lib, seed):
    rng = np.random.default_rng(100 + seed)
    Bn = int(rng.integers(1, 40))
    lq = rng.integers(0, 400, Bn)
    lk = rng.integers(0, 300, Bn) if seed % 2 else lq.copy()
    qo, ko = gen.offsets_from_lengths(lq), gen.offsets_from_lengths(lk)
    W = int(rng.integers(1, 50))
    block = seed % 2 == 0 and seed % 4 == 0
    if block:
        W += W % 2  # block plans run two workers per workgroup
    for order in range(3):
        d = _desc(B=Bn, H=3, D=64, order=order, num_workers=W, mask=1 if block else 0)
        p = B.jattn_plan_create(d, qo, ko)
        try:
            info, parts = _compare_plan(p, lq, lk, 3, block)
            for kind, which, kp in parts:
                units = B.jattn_plan_export(p, which * 2).reshape(-1, 4)
                offs = B.jattn_plan_export(p, which * 2 + 1)
                # the plan's own worker count of the pass: dK/dV at D = 64 without a
                # bias runs two workgroups per CU over twice the workers asked for;
                # the forward at D = 64 with 128-row tiles and 32-key steps three
                # over three times as many; dQ with 128-row tiles two or three
                if kind == "dkdv":
                    assert kp.num_workers in (W, 2 * W)
                elif kind == "fwd":
                    three = (kp.tile_rows, kp.step_rows) == (128, 32)
                    assert kp.num_workers == (3 * W if three else W)
                else:
                    assert kp.num_workers in (W, 2 * W, 3 * W)
                ref_u, ref_o = P.plan(kind, lq.tolist(), lk.tolist(), 3, kp.tile_rows, kp.step_rows,
                                      kp.num_workers, ["heavy_first", "zigzag", "lpt"][order])
                np.testing.assert_array_equal(units, np.array(ref_u, np.int32).reshape(-1, 4))
                np.testing.assert_array_equal(offs, np.array(ref_o, np.int32))
        finally:
            B.jattn_plan_destroy(p)


_LONG_Q = [300, 200, 100]


@pytest.mark.parametrize("kw,lq,lk,fwd,dkdv", [
    # bf16 at D <= 64 without bias or window, long queries: the forward on
    # 128-row tiles with 32-key steps over 3x the workers; dK/dV on 128-key
    # tiles with two workgroups per CU over 2x
    (dict(D=64), _LONG_Q, [100, 90, 80], (128, 32, 48), (128, 32)),
    (dict(D=32), _LONG_Q, [100, 90, 80], (128, 32, 48), (128, 32)),
    (dict(D=64, act=B.JATTN_SILU), _LONG_Q, [100, 90, 80], (128, 32, 48), (128, 32)),
    # erf-GELU keeps one dK/dV workgroup per CU (the forward rule holds)
    (dict(D=64, act=B.JATTN_GELU_ERF), _LONG_Q, [100, 90, 80], (128, 32, 48), (128, 16)),
    # 32-key dK/dV tiles (mean lk <= 32) keep one
    (dict(D=64), _LONG_Q, [20, 30, 10], (128, 32, 48), (32, 16)),
    # D = 128 softmax without bias or window: the forward's 128 x 32 tiles run
    # two workgroups per CU over 2x the workers (GDPA keeps 256 x 32)
    (dict(D=128), _LONG_Q, [100, 90, 80], (128, 32, 32), (128, 16)),
    (dict(D=128, act=B.JATTN_GELU_ERF), _LONG_Q, [100, 90, 80], (256, 32, 16), (128, 16)),
    # a bias, fp32 inputs, a window or short queries: neither rule
    (dict(D=128, has_bias=1), _LONG_Q, [100, 90, 80], (256, 32, 16), (128, 16)),
    (dict(D=64, has_bias=1), _LONG_Q, [100, 90, 80], (256, 32, 16), (128, 16)),
    (dict(D=64, in_dtype=B.JATTN_F32, out_dtype=B.JATTN_F32, grad_dtype=B.JATTN_F32), _LONG_Q, [100, 90, 80],
     (128, 64, 16), (128, 16)),
    (dict(D=64, mask=B.JATTN_MASK_WINDOW, window=(40, 7)), _LONG_Q, _LONG_Q, (128, 64, 16), (128, 16)),
    (dict(D=64), [20, 30, 10], [100, 90, 80], (32, 128, 16), (128, 32)),
])
def test_plan_occupancy_rules(lib, kw, lq, lk, fwd, dkdv):
    """Tile shape and worker count of the forward, and key tile and worker
    count of dK/dV, on each side of the rules that run two or three
    workgroups per CU (host only: plan creation makes no GPU call)."""
    d = _desc(B=len(lq), num_workers=16, **kw)
    p = B.jattn_plan_create(d, gen.offsets_from_lengths(np.array(lq)), gen.offsets_from_lengths(np.array(lk)))
    try:
        info = B.jattn_plan_info(p)
        assert (info.fwd.tile_rows, info.fwd.step_rows, info.fwd.num_workers) == fwd
        assert (info.dkdv.tile_rows, info.dkdv.num_workers) == dkdv
        # dQ at D = 128 (bf16 softmax, long queries, no bias, window or split):
        # 128-row tiles over 32-key steps, two workgroups per CU over twice the
        # workers; every other dQ keeps the workers asked for
        dq_many = (d.in_dtype == B.JATTN_BF16 and d.act == B.JATTN_SOFTMAX and not d.has_bias
                   and d.mask == B.JATTN_MASK_NONE and sum(lq) > 48 * len(lq))
        if dq_many and d.D == 128 and not d.split_operands:
            assert (info.dq.tile_rows, info.dq.step_rows, info.dq.num_workers) == (128, 32, 32)
        elif dq_many and d.D <= 64:
            # also two workgroups per CU at D <= 64
            assert (info.dq.tile_rows, info.dq.step_rows, info.dq.num_workers) == (128, 32, 32)
        else:
            assert info.dq.num_workers == 16
    finally:
        B.jattn_plan_destroy(p)


def test_empty_batch_plans(lib):
    d = _desc(B=0)
    p = B.jattn_plan_create(d, [0], [0])
    try:
        info = B.jattn_plan_info(p)
        assert info.Tq == 0 and info.fwd.n_units == 0
        # a forward over nothing is a no-op that touches no pointer
        B.jattn_fwd(p, None, None, None, None, None, None, None, None)
    finally:
        B.jattn_plan_destroy(p)


@pytest.mark.parametrize("seed", range(6))
def test_window_plans_match(lib, seed):
    """Windowed plans (tile skipping) bit-exact against the reference planner,
    and the plan's pair count against brute force."""
    rng = np.random.default_rng(200 + seed)
    Bn = int(rng.integers(1, 30))
    L = rng.integers(0, 700, Bn)
    L[0] = 0
    qo = gen.offsets_from_lengths(L)
    W = int(rng.integers(1, 40))
    window = [(0, 0), (5, 130), (200, 0), (63, 64), (2 ** 31 - 1, 1), (1000, 1000)][seed]
    D = [32, 64, 128][seed % 3]
    for order in range(3):
        d = _desc(B=Bn, H=3, D=D, order=order, num_workers=W, mask=B.JATTN_MASK_WINDOW, window=window,
                  act=seed % 3)
        p = B.jattn_plan_create(d, qo, qo)
        try:
            info, parts = _compare_plan(p, L, L, 3, False)
            assert (info.fwd.tile_rows, info.dq.tile_rows, info.dkdv.tile_rows) == (128, 128, 128)
            for kind, which, kp in parts:
                units = B.jattn_plan_export(p, which * 2).reshape(-1, 4)
                offs = B.jattn_plan_export(p, which * 2 + 1)
                ref_u, ref_o = P.plan(kind, L.tolist(), L.tolist(), 3, kp.tile_rows, kp.step_rows, W,
                                      ["heavy_first", "zigzag", "lpt"][order], window=window)
                np.testing.assert_array_equal(units, np.array(ref_u, np.int32).reshape(-1, 4))
                np.testing.assert_array_equal(offs, np.array(ref_o, np.int32))
            left, right = window
            pairs = sum(sum(min(n - 1, i + right) - max(0, i - left) + 1 for i in range(n)) for n in L.tolist())
            assert info.flops_fwd == pytest.approx(4.0 * 3 * D * pairs, rel=1e-12)
        finally:
            B.jattn_plan_destroy(p)


def test_l2norm_validation_never_touches_gpu(lib):
    fake = 0x10000000
    cases = [
        (dict(rows=-1), B.JATTN_E_SHAPE),
        (dict(D=48), B.JATTN_E_SHAPE),
        (dict(xt=7), B.JATTN_E_UNSUPPORTED),
        (dict(x=None), B.JATTN_E_NULL),
        (dict(x=fake + 8), B.JATTN_E_ALIGN),
        (dict(r=fake + 2), B.JATTN_E_ALIGN),
    ]
    for kw, code in cases:
        with pytest.raises(B.JattnError) as e:
            B.jattn_l2norm_fwd(kw.get("x", fake), fake, kw.get("r", None), kw.get("rows", 10), kw.get("D", 64),
                               kw.get("xt", B.JATTN_BF16), B.JATTN_BF16, None)
        assert e.value.code == code, kw
    with pytest.raises(B.JattnError) as e:
        B.jattn_l2norm_bwd(fake, None, fake, 10, 64, B.JATTN_BF16, B.JATTN_F32, B.JATTN_F32, None)
    assert e.value.code == B.JATTN_E_NULL
    with pytest.raises(B.JattnError) as e:
        B.jattn_l2norm_bwd(fake, fake, fake, 10, 64, B.JATTN_BF16, B.JATTN_F32, 5, None)
    assert e.value.code == B.JATTN_E_UNSUPPORTED
    # zero rows: a no-op that touches no pointer
    B.jattn_l2norm_fwd(None, None, None, 0, 64, B.JATTN_BF16, B.JATTN_BF16, None)
    B.jattn_l2norm_bwd(None, None, None, 0, 64, B.JATTN_BF16, B.JATTN_BF16, B.JATTN_BF16, None)


def test_rope_plan_grows_by_theta_table(lib):
    """Block plans with RoPE carry D/2 fp64 angles in their uploaded image."""
    L = [70, 129]
    off = gen.offsets_from_lengths(L)
    sizes = []
    for rope in (0, 1):
        p = B.jattn_plan_create(_desc(B=2, H=2, D=128, mask=B.JATTN_MASK_BLOCKDIAG64, rope=rope), off, off)
        try:
            sizes.append(B.jattn_plan_info(p).workspace_bytes)
        finally:
            B.jattn_plan_destroy(p)
    assert sizes[1] - sizes[0] in range(64 * 8, 64 * 8 + 512)
