// Achievable HBM read rate on this GPU, as a measured denominator beside the
// published 8 TB/s: the decode is bound by reading the latent cache from HBM
// [MLA explainer, why the KV cache is the bottleneck of inference], so its
// roofline fraction is read against both.  Two plain streaming readers of a
// buffer, each touching every byte once:
//   registers  16-byte loads, eight in flight per lane, 2048 workgroups of
//              256 threads (eight per CU), each reading one contiguous
//              range; the words are XOR-folded into one word per workgroup
//              so no load is dropped
//   lds copies the decode kernels' structure without their arithmetic: one
//              workgroup of four waves per CU, 36 KB tiles (nine 1 KB direct
//              global->LDS copies per wave), three tiles in flight, each
//              workgroup streaming one contiguous range of tiles
#include "kernels.h"
#include "lds_dma.h"

namespace mla {
namespace {

constexpr int kProbeTile = 36864;

__global__ void __launch_bounds__(256) hbm_read_regs_kernel(const uint4* __restrict__ buf, int64_t n16,
                                                            uint32_t* __restrict__ sink) {
  __shared__ uint32_t part[4];
  // workgroup b reads the contiguous 16-byte words [b * per, (b + 1) * per)
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  int64_t i = lo + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = buf[i + u * 256];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += 256) {
    const uint4 v = buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
hbm_read_lds_kernel(const char* __restrict__ buf, int64_t tiles) {
  __shared__ __attribute__((aligned(1024))) char lds[4 * kProbeTile];
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t per = (tiles + gridDim.x - 1) / gridDim.x;
  const int64_t k0 = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t k1 = k0 + per < tiles ? k0 + per : tiles;
  for (int64_t k = k0; k < k1; ++k) {
    wait_vmcnt<18>();  // at most two earlier tiles of this wave still in flight
    const char* t = buf + k * kProbeTile;
    const uint32_t dst = base + static_cast<uint32_t>(k & 3) * kProbeTile;
#pragma unroll
    for (int ii = 0; ii < 9; ++ii)
      dma16_sv(t, static_cast<uint32_t>((wave + 4 * ii) * 1024 + 16 * lane), dst + (wave + 4 * ii) * 1024);
  }
  wait_vmcnt<0>();
}

}  // namespace

hipError_t launch_hbm_read_probe(const void* buf, size_t bytes, int mode, uint32_t* sink, hipStream_t st) {
  if (mode == 0) {
    hipLaunchKernelGGL(hbm_read_regs_kernel, dim3(kProbeRegsGrid), dim3(256), 0, st,
                       static_cast<const uint4*>(buf), static_cast<int64_t>(bytes / 16), sink);
  } else {
    hipLaunchKernelGGL(hbm_read_lds_kernel, dim3(256), dim3(256), 0, st, static_cast<const char*>(buf),
                       static_cast<int64_t>(bytes / kProbeTile));
  }
  return hipGetLastError();
}

}  // namespace mla
