// Host-side split-KV planner shared by the C-ABI layer (see plan.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace mla {

struct PlanShape {
  int row_groups;        // workgroups per chunk (query rows / rows per workgroup)
  int resident_per_xcd;  // decode workgroups one XCD holds at once
};

struct PlanResult {
  int split_tokens, max_seq_len, num_items, max_splits, num_partials, num_slots;
  std::vector<int32_t> list;      // 4 per launch slot
  std::vector<int32_t> part_ptr;  // batch + 1
};

// Workspace of a planned decode: [header 256 B][launch list][part_ptr][partials]
struct PlanLayout {
  size_t list, part_ptr, partials, total;
};

int choose_split(const int32_t* lens, int batch, const PlanShape& sh);
bool build_plan(const int32_t* lens, int batch, const PlanShape& sh, int split_tokens, PlanResult* out);
uint64_t fnv1a(uint64_t h, const void* data, size_t n);
PlanLayout plan_layout(int batch, int num_slots, int64_t partial_rows_bytes);

}  // namespace mla
