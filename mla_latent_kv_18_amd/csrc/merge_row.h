// The log-sum-exp merge of one row's context-chunk partials (the decode's
// combine step),
//   L = log sum_s exp(lse_s),   o = sum_s exp(lse_s - L) o_s.
// A wave merges one row: lane l owns values 8l .. 8l+7 of the 512.  The
// sums run in split order over wave-uniform values (the lse of split s < 64
// sits in lane s and is read with readlane), so no chain of cross-lane
// shuffles sits on the row's path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace mla {

__device__ __forceinline__ float lane_value(float v, int s) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), s));
}

// ns >= 0 splits.  lv: in lane s < 64 the lse of split s (lanes past the
// last split hold a copy of some split's); lse: split 0's lse, split s at
// lse[s * lse_stride] (read only for s >= 64).  x0: this lane's values of
// the first PRE splits, loaded beforehand (split index clamped to ns - 1);
// part_of(s) loads them for s >= PRE.  acc receives o; returns L (-inf when
// every split is empty, o = 0 then).
template <int PRE, typename PartOf>
__device__ __forceinline__ float merge_row(int ns, float lv, const float* lse, int64_t lse_stride,
                                           const bf16x8_t (&x0)[PRE], PartOf part_of, float (&acc)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  auto lse_at = [&](int s) { return s < 64 ? lane_value(lv, s) : lse[s * lse_stride]; };
  float mx = -INFINITY;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, lse_at(s));
  if (mx == -INFINITY) return -INFINITY;
  const float e_lane = lv == -INFINITY ? 0.f : __expf(lv - mx);
  float sum = 0.f;
  for (int s = 0; s < ns; ++s) {
    float e;
    if (s < 64) {
      e = lane_value(e_lane, s);
    } else {
      const float v = lse[s * lse_stride];
      e = v == -INFINITY ? 0.f : __expf(v - mx);
    }
    sum += e;
  }
  const float L = mx + __logf(sum);
  const float w_lane = lv == -INFINITY ? 0.f : __expf(lv - L);
  auto weight = [&](int s) {
    if (s < 64) return lane_value(w_lane, s);
    const float v = lse[s * lse_stride];
    return v == -INFINITY ? 0.f : __expf(v - L);
  };
#pragma unroll
  for (int j = 0; j < PRE; ++j)
    if (j < ns) {
      const float w = weight(j);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = fmaf(w, static_cast<float>(x0[j][k]), acc[k]);
    }
  for (int s0 = PRE; s0 < ns; s0 += PRE) {
    bf16x8_t y[PRE];
#pragma unroll
    for (int j = 0; j < PRE; ++j) y[j] = part_of(min(s0 + j, ns - 1));
#pragma unroll
    for (int j = 0; j < PRE; ++j)
      if (s0 + j < ns) {
        const float w = weight(s0 + j);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = fmaf(w, static_cast<float>(y[j][k]), acc[k]);
      }
  }
  return L;
}

}  // namespace mla
