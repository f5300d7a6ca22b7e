// Host-side tile planner for jagged attention.
//
// "Training GEM at LLM scale" (Meta engineering post), section
// "Generalized Dot-Product Attention (GDPA)", item "Software-level tile
// scheduling for jagged tensors": the valid tiles of a jagged batch are listed
// on the CPU before launch, empty tiles are never scheduled, and tiles are
// assigned to compute units in zigzag order to even out the load.
//
// Units and their cost (inner-loop steps):
//   fwd / dq : (b, h, q-tile)   for lq_b > 0, cost = ceil(lk_b / step_rows)
//   dkdv     : (b, h, kv-tile)  for lk_b > 0, cost = ceil(lq_b / step_rows)
//   block    : (b, h, 64-block) for l_b > 0,  cost = 1
// Cost-0 units (partner length zero) only write zeros.
// Sliding window (section "BlockAttention": the window kernel never visits
// tiles outside the window), lq == lk: a fwd/dq tile of rows r0..r1 sees
// keys max(0, r0 - left) .. min(lk - 1, r1 + right), a dkdv tile of keys
// c0..c1 is seen by rows max(0, c0 - right) .. min(lq - 1, c1 + left); the
// cost is the number of steps those ranges meet.  The kernels derive the
// first step from the tile index (window_first_step), so the unit record
// stays (b, h, tile, cost).  Units are stably
// sorted by cost, descending, then dealt to workers round-robin
// (heavy-first), boustrophedon (zigzag) or to the least-loaded worker (LPT).
#pragma once

#include <stdint.h>

#include <vector>

namespace jattn {

enum UnitKind { kKindFwd = 0, kKindDkdv = 1, kKindDq = 2, kKindBlock = 3 };
enum Order { kHeavyFirst = 0, kZigzag = 1, kLpt = 2 };

struct UnitList {
  int32_t tile_rows = 0;
  int32_t step_rows = 0;
  int32_t num_workers = 0;
  std::vector<int32_t> units;    // 4 int32 per unit: b, h, tile, cost
  std::vector<int32_t> offsets;  // num_workers + 1
  int64_t n_units() const { return (int64_t)units.size() / 4; }
};

// Sliding-window sides; a negative left means no window.
struct Window {
  int32_t left = -1, right = -1;
  bool on() const { return left >= 0; }
};

// lq, lk: per-sample lengths (already validated).
void plan_units(UnitKind kind, const std::vector<int32_t>& lq, const std::vector<int32_t>& lk, int H,
                int tile_rows, int step_rows, int num_workers, Order order, UnitList* out,
                Window win = Window());

}  // namespace jattn
