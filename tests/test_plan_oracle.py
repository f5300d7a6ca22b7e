"""Pins for the reference tile planner (integer work, brute force on small batches)."""
import numpy as np
import pytest

from oracle import plan as P


def _cover(units, kind, lq, lk, H, tile, step, block=64):
    """Brute force: each valid (b, h, i, j) pair is reached exactly once."""
    seen = {}
    for b, h, t, cost in units:
        if kind in ("fwd", "dq"):
            rows = range(t * tile, min((t + 1) * tile, lq[b]))
            cols = range(lk[b])
            assert cost == -(-lk[b] // step)
        elif kind == "dkdv":
            cols = range(t * tile, min((t + 1) * tile, lk[b]))
            rows = range(lq[b])
            assert cost == -(-lq[b] // step)
        else:
            rows = range(t * block, min((t + 1) * block, lq[b]))
            cols = rows
            assert cost == 1
        assert len(rows) > 0 or len(cols) > 0, "empty unit"
        for i in rows:
            for j in cols:
                key = (b, h, i, j)
                assert key not in seen
                seen[key] = 1
    expect = 0
    for b in range(len(lq)):
        if kind == "block":
            expect += H * sum(min(64, lq[b] - s) ** 2 for s in range(0, lq[b], 64))
        else:
            expect += H * lq[b] * lk[b]
    assert len(seen) == expect


@pytest.mark.parametrize("kind", ["fwd", "dkdv", "dq", "block"])
@pytest.mark.parametrize("order", ["heavy_first", "zigzag", "lpt"])
def test_plan_covers_every_pair_once(kind, order):
    rng = np.random.default_rng(3)
    lq = rng.integers(0, 200, 9).tolist()
    lk = lq if kind == "block" else rng.integers(0, 150, 9).tolist()
    lq[2] = 0
    if kind != "block":
        lk[4] = 0
    H = 3
    tile, step = (64, 32) if kind != "block" else (64, 64)
    ordered, off = P.plan(kind, lq, lk, H, tile, step, W=7, order=order)
    assert off[0] == 0 and off[-1] == len(ordered)
    assert all(off[i] <= off[i + 1] for i in range(len(off) - 1))
    _cover(ordered, kind, lq, lk, H, tile, step)
    # every zero-length partner shows up as a cost-0 zero-fill unit
    n_units = len(P.enumerate_units(kind, lq, lk, H, tile, step))
    assert len(ordered) == n_units


def test_heavy_first_and_zigzag_rules():
    lq = [300, 10, 700, 64, 65, 1]
    lk = [100, 900, 5, 64, 400, 3]
    units = P.enumerate_units("fwd", lq, lk, 2, 64, 64)
    ranked = sorted(units, key=lambda u: -u[3])
    costs = [u[3] for u in ranked]
    assert costs == sorted(costs, reverse=True)
    W = 4
    hf, off = P.deal(units, W, "heavy_first")
    for w in range(W):
        assert hf[off[w]:off[w + 1]] == ranked[w::W]
    zz, off = P.deal(units, W, "zigzag")
    for i, u in enumerate(ranked):
        r, s = divmod(i, W)
        w = s if r % 2 == 0 else W - 1 - s
        assert u in zz[off[w]:off[w + 1]]
    # ties keep (b, h, t) order
    same = [u for u in ranked if u[3] == ranked[0][3]]
    assert same == sorted(same, key=lambda u: (u[0], u[1], u[2]))


def test_lpt_balance_bound():
    """Greedy least-loaded: max load <= mean + largest unit (classic LPT bound)."""
    rng = np.random.default_rng(5)
    lq = np.clip(np.rint(np.exp(np.log(300) + rng.standard_normal(64))), 8, 1000).astype(int).tolist()
    units = P.enumerate_units("fwd", lq, lq, 4, 128, 64)
    W = 37
    ordered, off = P.deal(units, W, "lpt")
    loads = P.worker_loads(ordered, off)
    total = sum(u[3] for u in units)
    assert sum(loads) == total
    assert max(loads) <= total / W + max(u[3] for u in units)


def test_block_plan_requires_equal_lengths():
    with pytest.raises(ValueError):
        P.enumerate_units("block", [5], [6], 1, 64, 64)
