#include "planner.hpp"

#include <algorithm>
#include <functional>
#include <queue>
#include <utility>

namespace jattn {

namespace {

inline int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

struct Unit {
  int32_t b, h, t, cost;
};

// Steps of a windowed unit: tile t (tile_rows rows of n_tile) meets partner
// rows row - near .. row + far of n_step; returns the step count.
int32_t window_cost(int32_t t, int32_t tile_rows, int32_t step_rows, int32_t n_tile, int32_t n_step,
                    int64_t near, int64_t far) {
  const int64_t r0 = (int64_t)t * tile_rows;
  const int64_t r1 = std::min<int64_t>(n_tile, r0 + tile_rows) - 1;
  const int64_t first = std::max<int64_t>(0, r0 - near);
  const int64_t last = std::min<int64_t>(n_step - 1, r1 + far);
  if (last < first) return 0;
  return (int32_t)(last / step_rows - first / step_rows + 1);
}

}  // namespace

void plan_units(UnitKind kind, const std::vector<int32_t>& lq, const std::vector<int32_t>& lk, int H,
                int tile_rows, int step_rows, int num_workers, Order order, UnitList* out, Window win) {
  out->tile_rows = tile_rows;
  out->step_rows = step_rows;
  out->num_workers = num_workers;
  out->units.clear();
  out->offsets.assign((size_t)num_workers + 1, 0);

  // 1. enumerate in (b, h, t) order
  std::vector<Unit> all;
  const int B = (int)lq.size();
  for (int b = 0; b < B; ++b) {
    int32_t n_tiles = 0, cost = 0;
    switch (kind) {
      case kKindFwd:
      case kKindDq:
        if (lq[b] == 0) continue;
        n_tiles = ceil_div(lq[b], tile_rows);
        cost = ceil_div(lk[b], step_rows);
        break;
      case kKindDkdv:
        if (lk[b] == 0) continue;
        n_tiles = ceil_div(lk[b], tile_rows);
        cost = ceil_div(lq[b], step_rows);
        break;
      case kKindBlock:
        if (lq[b] == 0) continue;
        n_tiles = ceil_div(lq[b], tile_rows);
        cost = 1;
        break;
    }
    const bool windowed = win.on() && kind != kKindBlock;
    for (int h = 0; h < H; ++h)
      for (int t = 0; t < n_tiles; ++t) {
        int32_t c = cost;
        if (windowed)
          c = kind == kKindDkdv ? window_cost(t, tile_rows, step_rows, lk[b], lq[b], win.right, win.left)
                                : window_cost(t, tile_rows, step_rows, lq[b], lk[b], win.left, win.right);
        all.push_back(Unit{b, h, t, c});
      }
  }

  // 2. stable sort by cost, descending
  std::stable_sort(all.begin(), all.end(), [](const Unit& x, const Unit& y) { return x.cost > y.cost; });

  // 3. deal to workers
  const int W = num_workers;
  std::vector<std::vector<Unit>> per(W);
  if (order == kLpt) {
    typedef std::pair<int64_t, int> Slot;  // (accumulated cost, worker)
    std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> heap;
    for (int w = 0; w < W; ++w) heap.push(Slot(0, w));
    for (const Unit& u : all) {
      Slot s = heap.top();
      heap.pop();
      per[s.second].push_back(u);
      heap.push(Slot(s.first + u.cost, s.second));
    }
  } else {
    for (size_t i = 0; i < all.size(); ++i) {
      const int64_t round = (int64_t)(i / (size_t)W);
      const int slot = (int)(i % (size_t)W);
      const int w = (order == kZigzag && (round & 1)) ? (W - 1 - slot) : slot;
      per[w].push_back(all[i]);
    }
  }

  // 4. CSR in worker order
  out->units.reserve(all.size() * 4);
  for (int w = 0; w < W; ++w) {
    for (const Unit& u : per[w]) {
      out->units.push_back(u.b);
      out->units.push_back(u.h);
      out->units.push_back(u.t);
      out->units.push_back(u.cost);
    }
    out->offsets[(size_t)w + 1] = (int32_t)(out->units.size() / 4);
  }
}

}  // namespace jattn
