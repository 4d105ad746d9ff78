// Skinny bf16 GEMM for the projections around the attention block:
//
//   y[m][n] = sum_k x[m][k] * w[n][k]     x [M, K] (row stride ldx), w [N, K], y [M, N]
//
// used for the query path c^Q = W^DQ h, q^C = W^UQ c^Q, W^QR c^Q
// [MLA explainer, query-compression section eq.(17); decoupled RoPE
// eq.(15)] and for the output projection u = sum_i W^O_i o_i, or its
// absorbed form sum_i B_i o_lat_i with B_i = W^O_i W^UV_i [MLA explainer,
// value-side absorption eq.(11)].
//
// and, with many tokens over K = 512, for the prefill's key and value
// up-projections W^UK_i c and W^UV_i c (linear_ws_kernel below).
//
// In the decode step M is the step's token count (tens); N and K are
// thousands, so the weight read bounds the call.  bf16 operands, fp32
// accumulation on MFMA 32x32x16.
//
// grid (N/128 row groups, n_chunks K slices, token groups), 4 waves: wave v
// owns weight rows 32v..32v+31 of its group and reads the whole K slice, so
// every weight byte is read once.  A pass covers MT 32-token tiles.  The
// slice is walked in batches of 8 k-steps (128 columns): the workgroup
// copies the batch's activation tile (32 MT rows x 256 B) into LDS once,
// with 16-byte chunks swizzled by row so that the waves' fragment reads are
// conflict-free, and every wave reads its A operands from there; the weight
// rows go straight to registers.  The loads of batch b+1 are issued before
// the MFMAs of batch b (registers double-buffered, LDS tile too).  Token
// rows past M are clamped to the last row and never stored.  With one slice
// the bf16 result is stored directly; otherwise fp32 partials go to the
// workspace and linear_reduce_kernel sums them.
#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace mla {
namespace {

constexpr int kLinRows = 128;    // weight rows per workgroup (32 per wave)
constexpr int kLinBatch = 8;     // k-steps per wave whose loads are in flight together
constexpr int kLinMaxChunks = 32;
constexpr int kLinMaxZ = 16;

__device__ __forceinline__ bf16x8_t load8(const __bf16* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// Two weight matrices over the same activations run as one problem of
// N = n1 + n2 rows: row groups below n1 read w and store into y (rows n1
// apart), the others read w2 and store into y2 (rows N - n1 apart); fp32
// partials use the combined N.  A single matrix has n1 = N.
template <int MT>
__global__ void __launch_bounds__(256) linear_kernel(const __bf16* __restrict__ x, const __bf16* __restrict__ w,
                                                     int ldx, int M, int N, int K, int chunk_len,
                                                     float* __restrict__ partial, __bf16* __restrict__ y,
                                                     const __bf16* __restrict__ w2, int n1, __bf16* __restrict__ y2) {
  constexpr int kTile = 32 * MT * 256;  // bytes of one batch's activation tile
  constexpr int kPer = 2 * MT;          // 16-byte tile chunks copied per thread
  __shared__ __attribute__((aligned(16))) char xs[2][kTile];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5, l32 = lane & 31;
  const int n0 = blockIdx.x * kLinRows + 32 * wave, kc = blockIdx.y;
  const bool second = static_cast<int>(blockIdx.x) * kLinRows >= n1;
  const int ksteps = chunk_len / 16, nb = (ksteps + kLinBatch - 1) / kLinBatch;
  const int64_t k_begin = static_cast<int64_t>(kc) * chunk_len;
  const __bf16* wrow = (second ? w2 + static_cast<int64_t>(n0 - n1 + l32) * K : w + static_cast<int64_t>(n0 + l32) * K) +
                       k_begin + 8 * hf;
  for (int m0 = blockIdx.z * 32 * MT; m0 < M; m0 += gridDim.z * 32 * MT) {
    // chunk i = tid + 256 s of the tile: row r = i / 16, 16-byte chunk c = i % 16
    // (k-step c / 2 of the batch, half c % 2), stored at chunk c ^ (r % 16) of row r
    const __bf16* xrow[kPer];
    int xoff[kPer], xc[kPer];
#pragma unroll
    for (int s = 0; s < kPer; ++s) {
      const int i = tid + 256 * s, r = i >> 4, c = i & 15;
      xrow[s] = x + static_cast<int64_t>(min(m0 + r, M - 1)) * ldx + k_begin + 8 * (c & 1);
      xc[s] = c >> 1;
      xoff[s] = (r * 16 + (c ^ (r & 15))) * 16;
    }
    bf16x8_t bw[kLinBatch], xr[kPer];
    // k-steps past the slice (a partial last batch) load a valid column and
    // are zeroed in the weight operand, so every batch runs all its MFMAs
    auto load_batch = [&](int b, bf16x8_t (&wv)[kLinBatch], bf16x8_t (&xv)[kPer]) {
#pragma unroll
      for (int j = 0; j < kLinBatch; ++j) wv[j] = load8(wrow + 16 * min(kLinBatch * b + j, ksteps - 1));
#pragma unroll
      for (int s = 0; s < kPer; ++s) xv[s] = load8(xrow[s] + 16 * min(kLinBatch * b + xc[s], ksteps - 1));
      if (kLinBatch * (b + 1) > ksteps) {
#pragma unroll
        for (int j = 0; j < kLinBatch; ++j) {
          const int keep = kLinBatch * b + j < ksteps ? -1 : 0;
          wv[j] = __builtin_bit_cast(bf16x8_t, __builtin_bit_cast(i32x4_t, wv[j]) & keep);
        }
      }
    };
    load_batch(0, bw, xr);
    f32x16_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16_t{};
    for (int b = 0; b < nb; ++b) {
      char* buf = xs[b & 1];
#pragma unroll
      for (int s = 0; s < kPer; ++s) *reinterpret_cast<bf16x8_t*>(buf + xoff[s]) = xr[s];
      __syncthreads();
      bf16x8_t bwn[kLinBatch], xrn[kPer];
      if (b + 1 < nb) load_batch(b + 1, bwn, xrn);
      __builtin_amdgcn_sched_barrier(0);  // the next batch's loads go out before this batch's MFMAs
#pragma unroll
      for (int j = 0; j < kLinBatch; ++j)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const int row = 32 * mt + l32, chunk = 2 * j + hf;
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(buf + (row * 16 + (chunk ^ (row & 15))) * 16);
            acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bw[j], acc[mt], 0, 0, 0);
          }
#pragma unroll
      for (int j = 0; j < kLinBatch; ++j) bw[j] = bwn[j];
#pragma unroll
      for (int s = 0; s < kPer; ++s) xr[s] = xrn[s];
    }
    // accumulator register r of lane (hf, l32) holds token 8(r/4) + 4hf + r%4 of the tile, row n0 + l32
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 32 * mt + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (m < M) {
          if (partial != nullptr)
            partial[(static_cast<int64_t>(kc) * M + m) * N + n0 + l32] = acc[mt][r];
          else if (second)
            y2[static_cast<int64_t>(m) * (N - n1) + n0 - n1 + l32] = f32_to_bf16(acc[mt][r]);
          else
            y[static_cast<int64_t>(m) * n1 + n0 + l32] = f32_to_bf16(acc[mt][r]);
        }
      }
    __syncthreads();  // the next pass rewrites the tiles
  }
}

// Many tokens over a short contraction (the prefill's key and value
// up-projections, k = d_c = 512): the weight rows stay in registers for the
// whole call and only activation tiles move.  grid (N/256 row groups, Z
// token groups), 8 waves: wave v holds rows 32v..32v+31 of its group (32
// k-steps, 128 VGPRs).  Per pass of 64 tokens the workgroup copies the
// activation tile (64 rows x 1 KB) straight into LDS, one pass ahead of the
// one computed (two buffers); chunk c of row r sits at r * 64 + (c ^ (r % 16))
// so the fragment reads are conflict-free.  Each wave then runs 64 MFMAs and
// stores its 32 columns of the 64 rows.
constexpr int kWsRows = 256, kWsK = 512, kWsWaves = 8;
constexpr int kWsTile = 64 * kWsK * 2;              // 64 KB
constexpr int kWsCopies = kWsTile / 1024 / kWsWaves;  // copies per wave per pass

__global__ void __launch_bounds__(64 * kWsWaves) linear_ws_kernel(const __bf16* __restrict__ x, int ldx,
                                                                  const __bf16* __restrict__ w, int M, int N,
                                                                  __bf16* __restrict__ y) {
  __shared__ __attribute__((aligned(1024))) char xs_raw[2 * kWsTile];
  MLA_LDS char* xs = (MLA_LDS char*)xs_raw;
  const uint32_t xs_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(xs));
  const int lane = threadIdx.x & 63, hf = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * kWsRows + 32 * wave;
  bf16x8_t bw[kWsK / 16];
  {
    const __bf16* wrow = w + static_cast<int64_t>(n0 + l32) * kWsK + 8 * hf;
#pragma unroll
    for (int s = 0; s < kWsK / 16; ++s) bw[s] = load8(wrow + 16 * s);
    wait_vmcnt<0>();  // complete before the tile copies start counting
  }
  const int tiles = (M + 63) / 64;
  const int np = (tiles - static_cast<int>(blockIdx.y) + gridDim.y - 1) / gridDim.y;
  auto issue = [&](int pass, int buf) {
    const int m0 = (blockIdx.y + gridDim.y * pass) * 64;
#pragma unroll
    for (int j = 0; j < kWsCopies; ++j) {
      const int i = wave + kWsWaves * j, slot = 64 * i + lane;
      const int r = slot >> 6, c = (slot & 63) ^ (r & 15);
      const __bf16* g = x + static_cast<int64_t>(min(m0 + r, M - 1)) * ldx + 8 * c;
      dma16(g, xs_addr + buf * kWsTile + i * 1024);
    }
  };
  if (np > 0) issue(0, 0);
  for (int pass = 0; pass < np; ++pass) {
    if (pass + 1 < np) {
      issue(pass + 1, (pass + 1) & 1);
      wait_vmcnt<kWsCopies>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();  // every wave's copies of this pass have landed
    MLA_LDS char* buf = xs + (pass & 1) * kWsTile;
    const int m0 = (blockIdx.y + gridDim.y * pass) * 64;
    f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int s = 0; s < kWsK / 16; ++s)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int r = 32 * mt + l32, c = 2 * s + hf;
        const bf16x8_t a = *reinterpret_cast<MLA_LDS const bf16x8_t*>(buf + (r * 64 + (c ^ (r & 15))) * 16);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bw[s], acc[mt], 0, 0, 0);
      }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 32 * mt + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (m < M) y[static_cast<int64_t>(m) * N + n0 + l32] = f32_to_bf16(acc[mt][r]);
      }
    __builtin_amdgcn_s_barrier();  // every wave is done with this buffer before it is refilled
  }
}

// y[m][4q..4q+3] = bf16(sum over slices of the partials); grid (column
// quads / 256, M).  Every slice's quad is requested before any is summed
// (MAXC >= n_chunks loads; the ones past n_chunks repeat the last slice).
template <int MAXC>
__global__ void __launch_bounds__(256) linear_reduce_kernel(const float* __restrict__ partial, int n_chunks, int M,
                                                            int N, __bf16* __restrict__ y, int n1,
                                                            __bf16* __restrict__ y2) {
  const int m = blockIdx.y, q = blockIdx.x * 256 + threadIdx.x;
  if (4 * q >= N) return;
  f32x4_t v[MAXC];
#pragma unroll
  for (int kc = 0; kc < MAXC; ++kc)
    v[kc] = *reinterpret_cast<const f32x4_t*>(partial + (static_cast<int64_t>(min(kc, n_chunks - 1)) * M + m) * N + 4 * q);
  f32x4_t s = f32x4_t{};
#pragma unroll
  for (int kc = 0; kc < MAXC; ++kc)
    if (kc < n_chunks) s += v[kc];
  bf16x4_t b;
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = f32_to_bf16(s[i]);
  __bf16* dst = 4 * q < n1 ? y + static_cast<int64_t>(m) * n1 + 4 * q : y2 + static_cast<int64_t>(m) * (N - n1) + 4 * q - n1;
  *reinterpret_cast<bf16x4_t*>(dst) = b;
}

}  // namespace

// K slices: as many workgroups as stay resident together (two per CU, 512;
// more would run a second, partial round), at most 32 slices, each a whole
// number of 16-wide k-steps, and fp32 partials of at most half the weight
// bytes (measured on the V3 shapes at 64 tokens: W^DQ with 16 slices and
// W^QR with 4 run 2-5 us faster than with twice as many, W^O with 8 runs 7 us
// faster than with 16).
// The weight-stationary form serves k = 512 with at least 256 tokens and
// rows in groups of 256; it needs no workspace.
bool linear_weight_stationary(int m, int n, int k) { return k == kWsK && m >= 256 && n % kWsRows == 0; }

int linear_chunks(int m, int n, int k) {
  if (linear_weight_stationary(m, n, k)) return 1;
  const int groups = n / kLinRows;
  int c = 1;
  while (2 * c <= kLinMaxChunks && groups * 2 * c <= 512) c *= 2;
  const int64_t weight_bytes = static_cast<int64_t>(n) * k * 2;
  while (c > 1 && (k % (16 * c) != 0 || static_cast<int64_t>(c) * m * n * 4 > weight_bytes / 2)) c /= 2;
  return c;
}

size_t linear_workspace(int m, int n, int k) {
  const int c = linear_chunks(m, n, k);
  return c > 1 ? static_cast<size_t>(c) * m * n * sizeof(float) : 0;
}

hipError_t launch_linear(const LinearArgs& a, hipStream_t st) {
  if (linear_weight_stationary(a.m, a.n, a.k)) {
    // one workgroup per CU (128 KB of LDS each): as many token groups as fill the GPU once
    const int groups = a.n / kWsRows;
    int z = 256 / groups;
    z = z < 1 ? 1 : z;
    const int tiles = (a.m + 63) / 64;
    z = z > tiles ? tiles : z;
    hipLaunchKernelGGL(linear_ws_kernel, dim3(groups, z), dim3(64 * kWsWaves), 0, st,
                       static_cast<const __bf16*>(a.x), a.ldx, static_cast<const __bf16*>(a.w), a.m, a.n,
                       static_cast<__bf16*>(a.y));
    return hipGetLastError();
  }
  return launch_linear_pair(a, nullptr, 0, nullptr, st);
}

hipError_t launch_linear_pair(const LinearArgs& a, const void* w2, int n2, void* y2, hipStream_t st) {
  const int n = a.n + n2;
  const int chunks = linear_chunks(a.m, n, a.k);
  const int mt = a.m <= 32 ? 1 : 2;
  int groups = (a.m + 32 * mt - 1) / (32 * mt);
  groups = groups > kLinMaxZ ? kLinMaxZ : groups;
  float* partial = chunks > 1 ? static_cast<float*>(a.workspace) : nullptr;
  const dim3 grid(n / kLinRows, chunks, groups);
  auto kern = mt == 1 ? linear_kernel<1> : linear_kernel<2>;
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, static_cast<const __bf16*>(a.x), static_cast<const __bf16*>(a.w),
                     a.ldx, a.m, n, a.k, a.k / chunks, partial, static_cast<__bf16*>(a.y),
                     static_cast<const __bf16*>(w2), a.n, static_cast<__bf16*>(y2));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || chunks == 1) return e;
  auto red = chunks <= 4 ? linear_reduce_kernel<4>
             : chunks <= 8 ? linear_reduce_kernel<8>
             : chunks <= 16 ? linear_reduce_kernel<16> : linear_reduce_kernel<kLinMaxChunks>;
  hipLaunchKernelGGL(red, dim3((n / 4 + 255) / 256, a.m), dim3(256), 0, st, partial, chunks, a.m, n,
                     static_cast<__bf16*>(a.y), a.n, static_cast<__bf16*>(y2));
  return hipGetLastError();
}

}  // namespace mla
