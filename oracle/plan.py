"""Reference tile planner (pure Python integers).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import this module.  It is written
from the plan specification, independently of the C++ planner inside the
HIP library; the two must agree bit for bit.

Source: "Training GEM at LLM scale" (Meta engineering post), section
"Generalized Dot-Product Attention (GDPA)", item "Software-level tile
scheduling for jagged tensors": valid tiles are listed on the CPU ahead of
time, empty tiles are never scheduled, and tiles are handed to compute units
in zigzag order.

Specification implemented here:
  1. enumerate units in (b, h, t) order
       fwd / dq : (b, h, q-tile t)  for lq_b > 0, t < ceil(lq_b / tile_rows),
                  cost = ceil(lk_b / step_rows)            (0 when lk_b = 0)
       dkdv     : (b, h, kv-tile t) for lk_b > 0, t < ceil(lk_b / tile_rows),
                  cost = ceil(lq_b / step_rows)            (0 when lq_b = 0)
       block    : (b, h, 64-block t) for l_b > 0, cost = 1
     a unit of cost 0 only writes zeros (zero-length partner sample).
     Sliding window (left, right), lq_b == lk_b ("BlockAttention" section:
     the sliding-window kernel skips the tiles that lie outside the
     window): a unit's steps are only those that meet its tile's window.
       fwd / dq : rows r0..r1 of the tile see keys max(0, r0 - left) ..
                  min(lk - 1, r1 + right); steps first_key // step_rows ..
                  last_key // step_rows
       dkdv     : keys c0..c1 are seen by rows max(0, c0 - right) ..
                  min(lq - 1, c1 + left), likewise
     cost = number of those steps.  The first step is not stored: it follows
     from the tile index and the window.
  2. stable sort by cost, descending (ties stay in (b, h, t) order)
  3. deal to W workers
       heavy_first : sorted position i -> worker i mod W
       zigzag      : round r = i div W, slot s = i mod W;
                     worker s if r even else W - 1 - s
       lpt         : each unit in sorted order goes to the worker with the
                     smallest accumulated cost (ties: lowest worker index)
  4. CSR: worker w owns units[offsets[w] : offsets[w+1]], in dealt order.
"""
from __future__ import annotations

import heapq

KIND_FWD = "fwd"
KIND_DKDV = "dkdv"
KIND_DQ = "dq"
KIND_BLOCK = "block"

ORDER_HEAVY_FIRST = "heavy_first"
ORDER_ZIGZAG = "zigzag"
ORDER_LPT = "lpt"


def _ceil_div(a, b):
    return -(-a // b)


def window_steps(t, tile_rows, step_rows, n_tile, n_step, near, far):
    """Inner-loop steps (first, count) of tile t of a sliding-window unit.

    The tile covers rows t*tile_rows .. of a sequence of n_tile rows; its
    partners (n_step of them) range from row - near to row + far."""
    r0 = t * tile_rows
    r1 = min(n_tile, r0 + tile_rows) - 1
    first = max(0, r0 - near)
    last = min(n_step - 1, r1 + far)
    if last < first:
        return first // step_rows, 0
    return first // step_rows, last // step_rows - first // step_rows + 1


def enumerate_units(kind, lq, lk, H, tile_rows, step_rows, block=64, window=None):
    """List of (b, h, t, cost) tuples in (b, h, t) order."""
    units = []
    for b in range(len(lq)):
        nq, nk = int(lq[b]), int(lk[b])
        if window is not None and kind != KIND_BLOCK and nq != nk:
            raise ValueError("sliding-window mode needs lq == lk")
        if kind in (KIND_FWD, KIND_DQ):
            if nq == 0:
                continue
            n_tiles, cost = _ceil_div(nq, tile_rows), _ceil_div(nk, step_rows)
            if window is not None:
                for h in range(H):
                    for t in range(n_tiles):
                        units.append((b, h, t, window_steps(t, tile_rows, step_rows, nq, nk,
                                                            window[0], window[1])[1]))
                continue
        elif kind == KIND_DKDV:
            if nk == 0:
                continue
            n_tiles, cost = _ceil_div(nk, tile_rows), _ceil_div(nq, step_rows)
            if window is not None:
                for h in range(H):
                    for t in range(n_tiles):
                        units.append((b, h, t, window_steps(t, tile_rows, step_rows, nk, nq,
                                                            window[1], window[0])[1]))
                continue
        elif kind == KIND_BLOCK:
            if nq != nk:
                raise ValueError("block mode needs lq == lk")
            if nq == 0:
                continue
            n_tiles, cost = _ceil_div(nq, block), 1
        else:
            raise ValueError(kind)
        for h in range(H):
            for t in range(n_tiles):
                units.append((b, h, t, cost))
    return units


def deal(units, W, order):
    """Order ``units`` over ``W`` workers; returns (ordered_units, offsets)."""
    if W <= 0:
        raise ValueError("W must be positive")
    ranked = sorted(units, key=lambda u: -u[3])  # stable: ties keep (b, h, t) order
    per_worker = [[] for _ in range(W)]
    if order == ORDER_HEAVY_FIRST:
        for i, u in enumerate(ranked):
            per_worker[i % W].append(u)
    elif order == ORDER_ZIGZAG:
        for i, u in enumerate(ranked):
            r, s = divmod(i, W)
            per_worker[s if r % 2 == 0 else W - 1 - s].append(u)
    elif order == ORDER_LPT:
        heap = [(0, w) for w in range(W)]
        for u in ranked:
            load, w = heapq.heappop(heap)
            per_worker[w].append(u)
            heapq.heappush(heap, (load + u[3], w))
    else:
        raise ValueError(order)
    ordered, offsets = [], [0]
    for lst in per_worker:
        ordered.extend(lst)
        offsets.append(len(ordered))
    return ordered, offsets


def plan(kind, lq, lk, H, tile_rows, step_rows, W, order, block=64, window=None):
    return deal(enumerate_units(kind, lq, lk, H, tile_rows, step_rows, block, window), W, order)


def worker_loads(ordered, offsets):
    """Total cost per worker."""
    return [sum(u[3] for u in ordered[offsets[w]:offsets[w + 1]]) for w in range(len(offsets) - 1)]
