// Host-side planning of the prefill launch: which tiles run narrow.
//
// The prefill kernel's workgroups each compute one output tile, and the
// dispatcher starts them in launch order on the first free workgroup slot
// (kPrefillWgsPerCu per CU).  When a launch holds a little more work than a
// whole number of rounds of slots, the last round is partly filled: most
// slots sit idle while a few tiles finish.  Giving the tiles of that round
// half the width (twice as many, each half as long) lets them spread over
// every slot.  plan_narrow_columns picks how many 256-column tile columns at
// the end of the launch's last projection to split that way, by list
// scheduling the launch with the measured tile costs below.
//
// Plain C++ (no HIP), so that the host tests can build it on its own.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <vector>

namespace bl {

// Cost of one tile in microseconds at two workgroups per CU on MI355X:
// a fixed part (first slab latency, epilogue) plus a part per slab of 128
// codes.  Measured with per-workgroup timestamps on the d=2560 / ffn=6912
// FFN at M=2048; only their ratios matter to the plan.
constexpr double kWideTileFixedUs = 10.0;
constexpr double kWideTileSlabUs = 1.4;
constexpr double kNarrowTileFixedUs = 6.5;
constexpr double kNarrowTileSlabUs = 0.8;

// One class of tiles of equal cost, in launch order.
struct TileClass {
  int64_t count;
  double us;
};

// End time of list scheduling: every tile, in order, starts on the slot that
// frees first.  Slots freeing at the same time are kept as one group, so the
// cost grows with the number of distinct free times, not with the tiles.
inline double list_schedule_end(const TileClass* cls, int n, int64_t slots) {
  struct Group {
    double t;
    int64_t n;
  };
  std::vector<Group> g{{0.0, slots}};  // sorted by t
  double end = 0.0;
  for (int c = 0; c < n; ++c) {
    int64_t left = cls[c].count;
    while (left > 0) {
      const Group e = g.front();
      const int64_t take = std::min(e.n, left);
      left -= take;
      if (e.n > take)
        g.front().n = e.n - take;
      else
        g.erase(g.begin());
      const double f = e.t + cls[c].us;
      end = std::max(end, f);
      auto it = std::lower_bound(g.begin(), g.end(), f, [](const Group& a, double t) { return a.t < t; });
      if (it != g.end() && it->t == f)
        it->n += take;
      else
        g.insert(it, Group{f, take});
    }
  }
  return end;
}

// K parts of each projection.  A projection whose K (in slabs of 128
// codes) is more than twice the launch's average load per slot would keep
// its workgroups busy long after the rest of the launch: it is split (at
// least min_part slabs per part, at most max_split parts), and the parts'
// int32 sums are added afterwards.  When the tiles, so split, all run at
// once, the longest tile sets the time, so parts are about the average load.
// When they take more than one round of workgroups, every slot runs two or
// more tiles anyway, and parts of up to twice the average fit the schedule:
// fewer parts, less partial-sum traffic and a cheaper adding pass (8B-class
// layer at M = 512: 2 parts of 56 slabs instead of 3 of 38, 138.4 -> 133.8
// us per step; 3B-class layer at M = 512: 94.2 -> 89.2 us).
//   slabs[i]: K slabs of projection i;  tiles[i]: its output tiles
//   ksplit[i], kspw[i] (out): parts, and slabs per part (the last may be shorter)
inline void plan_ksplit(int count, const int64_t* slabs, const int64_t* tiles, int64_t slots,
                        int64_t min_part, int max_split, int* ksplit, int* kspw) {
  double work = 0.0;
  for (int i = 0; i < count; ++i) work += (double)tiles[i] * (double)slabs[i];
  int64_t target = (int64_t)(work / (double)std::max<int64_t>(slots, 1)) + 1;
  target = std::max<int64_t>(target, min_part);
  int64_t tiles_fine = 0;  // tiles with parts of about the average load
  for (int i = 0; i < count; ++i) {
    int64_t p = 1;
    if (slabs[i] > 2 * target) p = std::min<int64_t>(max_split, (slabs[i] + target - 1) / target);
    tiles_fine += tiles[i] * p;
  }
  const int64_t part_max = tiles_fine > slots ? 2 * target : target;
  for (int i = 0; i < count; ++i) {
    ksplit[i] = 1;
    kspw[i] = (int)slabs[i];
    if (slabs[i] <= 2 * target) continue;
    int64_t parts = std::min<int64_t>(max_split, (slabs[i] + part_max - 1) / part_max);
    const int64_t per = (slabs[i] + parts - 1) / parts;
    parts = (slabs[i] + per - 1) / per;  // no empty part
    ksplit[i] = (int)parts;
    kspw[i] = (int)per;
  }
}

// Tile columns (of kWideBN outputs) at the end of the last projection to run
// as narrow tiles (kNarrowBN outputs); 0 keeps every tile wide.
//   count:     projections in launch order
//   slabs[i]:  K slabs (of 128 codes) of one tile of projection i (one K part)
//   ncols[i]:  output columns of projection i
//   parts[i]:  K parts of projection i (null: 1 each); the last projection
//              is narrowed only when it has one
//   tiles_m:   tiles along the token rows
//   slots:     workgroups that run at once on the device
template <int kWideBN, int kNarrowBN>
inline int plan_narrow_columns(int count, const int64_t* slabs, const int64_t* ncols, int64_t tiles_m,
                               int64_t slots, const int* parts = nullptr) {
  if (count < 1 || tiles_m < 1 || slots < 1) return 0;
  if (parts && parts[count - 1] != 1) return 0;
  std::vector<TileClass> cls(count + 1);
  int64_t tiles = 0;
  for (int i = 0; i < count; ++i) {
    const int64_t tn = (ncols[i] + kWideBN - 1) / kWideBN;
    cls[i] = TileClass{tiles_m * tn * (parts ? parts[i] : 1),
                       kWideTileFixedUs + kWideTileSlabUs * (double)slabs[i]};
    tiles += cls[i].count;
  }
  if (tiles <= slots) return 0;  // one round: nothing waits for a slot
  // past 16 rounds the last round's idle slots cost little; skip the plan
  if (tiles > 16 * slots) return 0;
  const int last = count - 1;
  const int64_t wide_cols = (ncols[last] + kWideBN - 1) / kWideBN;
  // narrowing more than about one round of tiles cannot even it out further
  const int64_t max_c = std::min<int64_t>(wide_cols, (slots + tiles_m - 1) / tiles_m + 1);
  const double narrow_us = kNarrowTileFixedUs + kNarrowTileSlabUs * (double)slabs[last];
  double best = list_schedule_end(cls.data(), count, slots);
  int best_c = 0;
  for (int64_t c = 1; c <= max_c; ++c) {
    const int64_t keep = wide_cols - c;  // wide tile columns left in front
    const int64_t narrow_n = ncols[last] - keep * kWideBN;
    cls[last] = TileClass{tiles_m * keep, kWideTileFixedUs + kWideTileSlabUs * (double)slabs[last]};
    cls[count] = TileClass{tiles_m * ((narrow_n + kNarrowBN - 1) / kNarrowBN), narrow_us};
    const double e = list_schedule_end(cls.data(), count + 1, slots);
    if (e < best * 0.99) {  // a clear gain only
      best = e;
      best_c = (int)c;
    }
  }
  return best_c;
}

}  // namespace bl
