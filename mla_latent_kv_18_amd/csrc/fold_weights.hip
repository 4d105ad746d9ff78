// Absorbed weights, formed once when a model is loaded (not per step):
//   output side  B_i = W^O_i W^UV_i      [MLA explainer, value-side absorption eq.(11)]
//   query side   A_i = W^UK_i^T W^UQ_i   [MLA explainer, matrix absorption eq.(7)-(8),
//                                          query-compression section]
// Both are a batch (one per head) of small products C_i = X_i Y_i whose
// operands sit at fixed strides inside the stacked weights, so one strided
// kernel serves both: C_i[r, c] = sum_k X_i[r, k] Y_i[k, c], fp32
// accumulation, stored in the activation dtype.
//
// 64 x 64 output tile per 256-thread workgroup, k in slices of 16 staged
// through LDS; each thread owns a 4 x 4 block of the tile.  The operands are
// read with their own strides (one of them is transposed for each of the
// two uses), which costs coalescing but not correctness; this runs once per
// model load.
#include "device_common.h"
#include "kernels.h"

namespace mla {
namespace {

template <typename T>
__device__ __forceinline__ float ld(const T* p) {
  return static_cast<float>(*p);
}

template <typename T>
__global__ void __launch_bounds__(256) fold_kernel(FoldArgs a) {
  constexpr int kT = 64, kK = 16;
  __shared__ float xs[kK][kT + 1];
  __shared__ float ys[kK][kT + 1];
  const T* x = static_cast<const T*>(a.x);
  const T* y = static_cast<const T*>(a.y);
  T* out = static_cast<T*>(a.out);
  const int i = blockIdx.z;
  const int r0 = blockIdx.y * kT, c0 = blockIdx.x * kT;
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;  // 4x4 block at rows 4tr.., columns 4tc..
  float acc[4][4] = {};
  const int64_t xb = static_cast<int64_t>(i) * a.xs_i, yb = static_cast<int64_t>(i) * a.ys_i;
  for (int k0 = 0; k0 < a.k; k0 += kK) {
    // 64 x 16 elements of each operand: 4 per thread
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e;      // 0..1023
      const int kk = idx / kT, rr = idx % kT;
      const int k = k0 + kk;
      const int r = r0 + rr, c = c0 + rr;
      xs[kk][rr] = (k < a.k && r < a.rows) ? ld(x + xb + static_cast<int64_t>(r) * a.xs_r + static_cast<int64_t>(k) * a.xs_k) : 0.f;
      ys[kk][rr] = (k < a.k && c < a.cols) ? ld(y + yb + static_cast<int64_t>(k) * a.ys_k + static_cast<int64_t>(c) * a.ys_c) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kK; ++kk) {
      float xv[4], yv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        xv[u] = xs[kk][4 * tr + u];
        yv[u] = ys[kk][4 * tc + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(xv[u], yv[v], acc[u][v]);
    }
    __syncthreads();
  }
  const int64_t ob = static_cast<int64_t>(i) * a.os_i;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = r0 + 4 * tr + u;
    if (r >= a.rows) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c = c0 + 4 * tc + v;
      if (c < a.cols) out[ob + static_cast<int64_t>(r) * a.os_r + static_cast<int64_t>(c) * a.os_c] = static_cast<T>(acc[u][v]);
    }
  }
}

}  // namespace

hipError_t launch_fold(const FoldArgs& a, bool bf16, hipStream_t st) {
  const dim3 grid((a.cols + 63) / 64, (a.rows + 63) / 64, a.batch);
  if (bf16)
    hipLaunchKernelGGL(fold_kernel<__bf16>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(fold_kernel<float>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
