// Which context chunk of which request a decode workgroup works on.  Shared
// by the bf16 and fp8 decode kernels.
//
// Two launch forms:
//   list     a launch list written by the host planner: entry s (int32 x 4)
//            = {b | rg << 24, j0, j1, part} for workgroup s, or b < 0 for an
//            idle slot.  part >= 0 is the chunk's partial row block; part < 0
//            means the request has this one chunk and the workgroup writes
//            o_lat directly.  The planner orders the list so that slot s runs
//            on XCD s % 8 (workgroups are handed to the XCDs round-robin).
//   uniform  every request is cut into chunks of split_tokens rows; the
//            workgroup's (request, row group, chunk) comes from its ids.
// In both forms the chunk is clamped to the request's length as the device
// holds it, so a length shorter than planned stays in bounds (the chunk
// becomes empty and writes an empty partial: o = 0, lse = -inf).
#pragma once

#include "device_common.h"

namespace mla {

struct DecodeUnit {
  int b, rg, j0, j1, T;
  int part;  // partial row block, or -1 when o_lat is written directly
};

__device__ __forceinline__ int clamp_len(const int32_t* seq_lens, int b, int max_seq_len) {
  int T = ((const MLA_CONST int32_t*)(seq_lens))[b];
  return T < 0 ? 0 : (T > max_seq_len ? max_seq_len : T);
}

// List form: false for an idle slot.
__device__ __forceinline__ bool unit_from_list(const int32_t* items, const int32_t* seq_lens,
                                               int max_seq_len, int slot, DecodeUnit& u) {
  const MLA_CONST int32_t* e = (const MLA_CONST int32_t*)(items) + 4 * static_cast<int64_t>(slot);
  const int w0 = e[0];
  if (w0 < 0) return false;
  u.b = w0 & 0xFFFFFF;
  u.rg = w0 >> 24;
  u.T = clamp_len(seq_lens, u.b, max_seq_len);
  u.j0 = e[1];
  u.j1 = max(u.j0, min(e[2], u.T));
  u.part = e[3];
  return true;
}

// Uniform form: false for a chunk past the end of its request (the combine
// skips those).
__device__ __forceinline__ bool unit_uniform(const int32_t* seq_lens, int max_seq_len, int split_tokens,
                                             int num_splits, int b, int rg, int split, DecodeUnit& u) {
  u.b = b;
  u.rg = rg;
  u.T = clamp_len(seq_lens, b, max_seq_len);
  u.j0 = split * split_tokens;
  const bool direct = num_splits == 1;
  if (!direct && u.j0 >= u.T) return false;
  u.j1 = min(u.j0 + split_tokens, u.T);
  u.part = direct ? -1 : b * num_splits + split;
  return true;
}

}  // namespace mla
