// Host-side split-KV planner for mla_decode: turns the host copy of the
// requests' lengths into a balanced launch list.
//
// 1. Chunk length L.  Every request of length T is cut into ceil(T / L)
//    chunks (one for T = 0, which then writes o = 0, lse = -inf).  A chunk
//    is processed by row_groups workgroups (each owns 128 or 64 of the
//    request's q_len * n_h query rows).  L is chosen to minimise an estimate
//    of the launch's makespan, (waves of resident workgroups) x (L + a fixed
//    per-chunk cost), over the lengths L = ceil(max T / s) rounded up to 64.
// 2. Placement.  Workgroups are handed to the eight XCDs round-robin, so the
//    workgroup in launch slot s runs on XCD s % 8 and each XCD works through
//    its own slots in order.  Requests are placed longest first on the least
//    loaded XCD, whole when that keeps the XCD within one chunk of the
//    average load (its chunks then share that XCD's L2 for the query rows
//    and for the partials the combine reads back), else chunk by chunk.
//    The row groups of one chunk take consecutive slots of the same XCD, so
//    the second reads the chunk's cache rows from that L2.  Each XCD's
//    chunks run longest first.
// 3. Output.  The launch list (int32 x 4 per slot: {b | rg << 24, j0, j1,
//    part}, b = -1 for an idle slot) and part_ptr [batch + 1]: the partial
//    blocks of request b are part_ptr[b] .. part_ptr[b+1] - 1, and a request
//    with one chunk has none (its workgroups write o_lat directly).
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "plan.h"

namespace mla {

namespace {

constexpr int kChunkCost = 256;  // fixed cost of a chunk (prologue, epilogue) in cache rows
constexpr int kXcds = 8;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t chunks_of(int64_t T, int64_t L) { return T <= 0 ? 1 : ceil_div(T, L); }

}  // namespace

int choose_split(const int32_t* lens, int batch, const PlanShape& sh) {
  int64_t max_t = 0;
  for (int b = 0; b < batch; ++b) max_t = std::max<int64_t>(max_t, lens[b]);
  if (max_t <= 64) return 64;
  const int64_t resident = static_cast<int64_t>(kXcds) * sh.resident_per_xcd;
  int64_t best_l = 0;
  double best = 0.0;
  int64_t prev = -1;
  for (int64_t s = 1; s <= 4096; ++s) {
    int64_t L = ceil_div(ceil_div(max_t, s), 64) * 64;
    if (L < 256 && s > 1) break;
    if (L == prev) continue;
    prev = L;
    int64_t groups = 0;
    for (int b = 0; b < batch; ++b) groups += chunks_of(lens[b], L) * sh.row_groups;
    const double est = static_cast<double>(ceil_div(groups, resident)) * static_cast<double>(L + kChunkCost);
    if (best_l == 0 || est < best) {  // ties keep the longer chunk (fewer partials)
      best = est;
      best_l = L;
    }
  }
  return static_cast<int>(best_l);
}

bool build_plan(const int32_t* lens, int batch, const PlanShape& sh, int split_tokens, PlanResult* out) {
  const int64_t L = split_tokens;
  out->split_tokens = split_tokens;
  out->max_seq_len = 0;
  out->num_items = 0;
  out->max_splits = 0;
  out->num_partials = 0;
  out->part_ptr.assign(static_cast<size_t>(batch) + 1, 0);
  struct Item {
    int b, j0, j1, part;
  };
  std::vector<std::vector<Item>> by_req(batch);
  std::vector<int64_t> req_cost(batch, 0);
  for (int b = 0; b < batch; ++b) {
    const int64_t T = lens[b];
    if (T < 0) return false;
    out->max_seq_len = std::max<int>(out->max_seq_len, static_cast<int>(T));
    const int64_t n = chunks_of(T, L);
    out->max_splits = std::max<int>(out->max_splits, static_cast<int>(n));
    out->part_ptr[b] = out->num_partials;
    for (int64_t k = 0; k < n; ++k) {
      const int j0 = static_cast<int>(k * L), j1 = static_cast<int>(std::min(T, (k + 1) * L));
      const int part = n == 1 ? -1 : out->num_partials++;
      by_req[b].push_back({b, j0, j1, part});
      req_cost[b] += (j1 - j0) + kChunkCost;
    }
    out->num_items += static_cast<int>(n);
  }
  out->part_ptr[batch] = out->num_partials;

  // placement
  int64_t total = std::accumulate(req_cost.begin(), req_cost.end(), int64_t{0});
  const int64_t target = ceil_div(total, kXcds), slack = L + kChunkCost;
  std::vector<int> order(batch);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int c) { return req_cost[a] > req_cost[c]; });
  int64_t load[kXcds] = {};
  std::vector<Item> queue[kXcds];
  auto least = [&]() { return static_cast<int>(std::min_element(load, load + kXcds) - load); };
  for (int b : order) {
    const int x = least();
    if (load[x] + req_cost[b] <= target + slack) {
      for (const Item& it : by_req[b]) queue[x].push_back(it);
      load[x] += req_cost[b];
    } else {
      for (const Item& it : by_req[b]) {
        const int y = least();
        queue[y].push_back(it);
        load[y] += (it.j1 - it.j0) + kChunkCost;
      }
    }
  }
  size_t per_xcd = 0;
  for (auto& q : queue) {
    std::stable_sort(q.begin(), q.end(), [](const Item& a, const Item& c) { return a.j1 - a.j0 > c.j1 - c.j0; });
    per_xcd = std::max(per_xcd, q.size() * static_cast<size_t>(sh.row_groups));
  }
  out->num_slots = static_cast<int>(per_xcd * kXcds);
  out->list.assign(static_cast<size_t>(out->num_slots) * 4, 0);
  for (int x = 0; x < kXcds; ++x) {
    size_t pos = 0;
    for (const Item& it : queue[x])
      for (int rg = 0; rg < sh.row_groups; ++rg, ++pos) {
        int32_t* e = &out->list[(x + kXcds * pos) * 4];
        e[0] = it.b | (rg << 24);
        e[1] = it.j0;
        e[2] = it.j1;
        e[3] = it.part;
      }
    for (; pos < per_xcd; ++pos) out->list[(x + kXcds * pos) * 4] = -1;  // idle slot
  }
  return true;
}

uint64_t fnv1a(uint64_t h, const void* data, size_t n) {
  const unsigned char* p = static_cast<const unsigned char*>(data);
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 0x100000001b3ull;
  }
  return h;
}

PlanLayout plan_layout(int batch, int num_slots, int64_t partial_rows_bytes) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  PlanLayout l;
  l.list = 256;  // the first 256 bytes are a header
  l.part_ptr = l.list + up(static_cast<size_t>(num_slots) * 16);
  l.partials = l.part_ptr + up((static_cast<size_t>(batch) + 1) * 4);
  l.total = l.partials + up(static_cast<size_t>(partial_rows_bytes));
  return l;
}

}  // namespace mla
