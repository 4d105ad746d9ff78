// Per-step projections around the latent decode, bf16 activations and
// weights, fp32 accumulation on MFMA 32x32x16 (gfx950):
//
//   append:   kv = [W^DKV ; W^KR] h  (split over the d_model contraction into
//             fp32 partials), then RMSNorm on the d_c latent, RoPE on the
//             d_R key part, optional e4m3 quantisation, write to the slot
//             [MLA explainer, low-rank eq.(2), decoupled RoPE eq.(15),
//              trade-offs section (latent normalisation)]
//   absorb q: q_lat = W^UK_i^T q_nope per head, RoPE on q_pe
//             [MLA explainer, matrix absorption eq.(8)]
//   out proj: out = W^UV_i o_lat per head [MLA explainer eq.(10)]
//
// These calls touch O(weights) bytes per step, not O(context): they are
// weight-read bound; the grids are sized so that ~512 waves stream the
// weights at once.
#include <cmath>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kD = kDc + kDr;
constexpr int kDh = 128;

__device__ __forceinline__ bf16x8_t load8(const __bf16* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// ------------------------------------------------------------ append GEMM
// grid (576/32 column tiles, n_chunks slices of the d_model contraction),
// 4 waves; wave w takes 1/4 of the slice.  All operand loads of a wave are
// issued before its MFMAs; the 4 wave partials are summed through LDS.
// partial[kc][n][r] = sum_{k in slice kc} h[n][k] * W[r][k]
constexpr int kProjWaves = 4;
constexpr int kMaxMTiles = 1;  // 32-token tiles per pass; blockIdx.z picks the tile

__global__ void __launch_bounds__(256) append_proj_kernel(const __bf16* __restrict__ h,
                                                          const __bf16* __restrict__ w, int n_tokens,
                                                          int d_model, int chunk_len,
                                                          float* __restrict__ partial) {
  __shared__ f32x16_t red[kProjWaves][kMaxMTiles][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hf = lane >> 5, l32 = lane & 31;
  const int r0 = blockIdx.x * 32, kc = blockIdx.y;
  const int ksteps = chunk_len / 16 / kProjWaves;  // per wave
  const int k_begin = kc * chunk_len + wave * ksteps * 16;
  const __bf16* wrow = w + static_cast<int64_t>(r0 + l32) * d_model + k_begin + 8 * hf;
  for (int m0 = blockIdx.z * 32 * kMaxMTiles; m0 < n_tokens; m0 += gridDim.z * 32 * kMaxMTiles) {
    const int mts = min(kMaxMTiles, (n_tokens - m0 + 31) / 32);
    f32x16_t acc[kMaxMTiles];
#pragma unroll
    for (int mt = 0; mt < kMaxMTiles; ++mt) acc[mt] = f32x16_t{};
    for (int kb = 0; kb < ksteps; kb += 8) {
      bf16x8_t bw[8], ha[kMaxMTiles][8];
#pragma unroll
      for (int j = 0; j < 8; ++j) bw[j] = kb + j < ksteps ? load8(wrow + 16 * (kb + j)) : bf16x8_t{};
#pragma unroll
      for (int mt = 0; mt < kMaxMTiles; ++mt) {
        const int n = m0 + 32 * mt + l32;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          ha[mt][j] = (mt < mts && n < n_tokens && kb + j < ksteps)
                          ? load8(h + static_cast<int64_t>(n) * d_model + k_begin + 16 * (kb + j) + 8 * hf)
                          : bf16x8_t{};
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int mt = 0; mt < kMaxMTiles; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ha[mt][j], bw[j], acc[mt], 0, 0, 0);
    }
#pragma unroll
    for (int mt = 0; mt < kMaxMTiles; ++mt) red[wave][mt][lane] = acc[mt];
    __syncthreads();
    // thread t sums registers 4*(t/64) .. +3 of lane t%64 over the 4 waves
    const int rl = threadIdx.x & 63, rq = threadIdx.x >> 6;
    for (int mt = 0; mt < mts; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * rq + i;
        float v = 0.f;
#pragma unroll
        for (int wv = 0; wv < kProjWaves; ++wv) v += red[wv][mt][rl][r];
        const int n = m0 + 32 * mt + 8 * (r >> 2) + 4 * (rl >> 5) + (r & 3);
        if (n < n_tokens) partial[(static_cast<int64_t>(kc) * n_tokens + n) * kD + r0 + (rl & 31)] = v;
      }
    __syncthreads();
  }
}

constexpr int kMaxChunks = 16;  // contraction slices of the append GEMM

// One workgroup (256 threads) per token: reduce the partials, RMSNorm the
// latent, rotate the key part, convert, write the cache row.
template <bool FP8>
__global__ void __launch_bounds__(256) append_finish_kernel(
    const float* __restrict__ partial, int n_chunks, int n_tokens, const float* __restrict__ gamma,
    const int32_t* __restrict__ positions, const int64_t* __restrict__ slots, int64_t cache_slots,
    float eps, RopeTable64 rope, void* __restrict__ cache, float* __restrict__ cache_scale) {
  __shared__ float kv[kD];
  __shared__ float red[256];
  const int n = blockIdx.x, tid = threadIdx.x;
  const int64_t slot = slots[n];
  if (slot < 0 || slot >= cache_slots) return;
  // all chunk partials of this thread's columns are requested before any is summed
  {
    float v[kMaxChunks][3];
#pragma unroll
    for (int kc = 0; kc < kMaxChunks; ++kc)
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int c = tid + 256 * j;
        v[kc][j] = (kc < n_chunks && c < kD) ? partial[(static_cast<int64_t>(kc) * n_tokens + n) * kD + c] : 0.f;
      }
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int c = tid + 256 * j;
      float s = 0.f;
#pragma unroll
      for (int kc = 0; kc < kMaxChunks; ++kc) s += v[kc][j];
      if (c < kD) kv[c] = s;
    }
  }
  __syncthreads();
  float ss = 0.f;
  for (int c = tid; c < kDc; c += 256) ss = fmaf(kv[c], kv[c], ss);
  red[tid] = ss;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  const float inv_rms = rsqrtf(red[0] * (1.f / kDc) + eps);
  __syncthreads();
  float out[3];
  int cnt = 0;
  for (int c = tid; c < kD; c += 256, ++cnt) {
    float v;
    if (c < kDc) {
      v = kv[c] * inv_rms * gamma[c];
    } else {
      const int k = (c - kDc) & 31;
      float cs, sn;
      rope_cos_sin_inv(positions[n], rope.inv[k], &cs, &sn);
      const float x1 = kv[kDc + k], x2 = kv[kDc + 32 + k];
      v = (c - kDc) < 32 ? x1 * cs - x2 * sn : x1 * sn + x2 * cs;
    }
    out[cnt] = v;
  }
  if constexpr (!FP8) {
    __bf16* row = static_cast<__bf16*>(cache) + slot * kD;
    cnt = 0;
    for (int c = tid; c < kD; c += 256, ++cnt) row[c] = f32_to_bf16(out[cnt]);
  } else {
    float am = 0.f;
    cnt = 0;
    for (int c = tid; c < kD; c += 256, ++cnt) am = fmaxf(am, fabsf(out[cnt]));
    __syncthreads();
    red[tid] = am;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
      __syncthreads();
    }
    const float amax = red[0];
    const float scale = amax > 0.f ? amax / 448.f : 1.f;
    uint8_t* row = static_cast<uint8_t*>(cache) + slot * kD;
    cnt = 0;
    for (int c = tid; c < kD; c += 256, ++cnt) row[c] = static_cast<uint8_t>(f32_to_e4m3(out[cnt] / scale));
    if (tid == 0) cache_scale[slot] = scale;
  }
}

// --------------------------------------------------------------- absorb q
// grid (n_h, 4 column tiles of 128), 4 waves.  W^UK_i[:, 128 cols] is staged
// in LDS (128 rows x 16 chunks, chunk ch of row a at a*16 + (ch ^ 4(a%4)))
// and read transposed (ds_read_b64_tr_b16) as the B operand (K = a, N = c);
// wave w produces columns 32w..32w+31 of the tile for every token.
template <bool OUT_F32>
__global__ void __launch_bounds__(256) absorb_q_kernel(const __bf16* __restrict__ q_nope,
                                                       const __bf16* __restrict__ q_pe,
                                                       const __bf16* __restrict__ w_uk,
                                                       const int32_t* __restrict__ positions,
                                                       int n_tokens, int n_h, RopeTable64 rope,
                                                       void* __restrict__ q_out) {
  __shared__ __attribute__((aligned(16))) char wl[kDh * 256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hf = lane >> 5, l32 = lane & 31;
  const int head = blockIdx.x, ct = blockIdx.y;
  const __bf16* W = w_uk + static_cast<int64_t>(head) * kDh * kDc + ct * 128;
  {
    bf16x8_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = threadIdx.x + 256 * j;
      v[j] = load8(W + static_cast<int64_t>(i >> 4) * kDc + (i & 15) * 8);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = threadIdx.x + 256 * j, a = i >> 4, ch = i & 15;
      *reinterpret_cast<MLA_LDS bf16x8_t*>((MLA_LDS char*)wl + (a * 16 + (ch ^ (4 * (a & 3)))) * 16) = v[j];
    }
  }
  const int L = lane & 15, cg = (lane >> 4) & 1;
  bool staged = false;  // W slice visible to every wave
  for (int m0 = blockIdx.z * 32; m0 < n_tokens; m0 += gridDim.z * 32) {
    const int n_a = m0 + l32;
    bf16x8_t a[kDh / 16];
#pragma unroll
    for (int ks = 0; ks < kDh / 16; ++ks)
      a[ks] = n_a < n_tokens ? load8(q_nope + (static_cast<int64_t>(n_a) * n_h + head) * kDh + 16 * ks + 8 * hf)
                             : bf16x8_t{};
    if (!staged) {
      __syncthreads();
      staged = true;
    }
    f32x16_t acc = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < kDh / 16; ++ks) {
      i16x4_t part[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int row = 16 * ks + 8 * hf + 4 * h2 + (L >> 2);
        const int ch = 4 * wave + 2 * cg + ((L & 3) >> 1);
        const int off = (row * 16 + (ch ^ (4 * (row & 3)))) * 16 + 8 * (L & 1);
        part[h2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<MLA_LDS i16x4_t*>((MLA_LDS char*)wl + off));
      }
      const bf16x8_t bfr = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], bfr, acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = m0 + 8 * (r >> 2) + 4 * hf + (r & 3);
      if (n < n_tokens) {
        const int64_t idx = (static_cast<int64_t>(n) * n_h + head) * kD + ct * 128 + 32 * wave + l32;
        if constexpr (OUT_F32) static_cast<float*>(q_out)[idx] = acc[r];
        else static_cast<__bf16*>(q_out)[idx] = f32_to_bf16(acc[r]);
      }
    }
  }
  if (!staged) __syncthreads();
  if (ct == 0) {  // RoPE part of the latent query: thread = (token, 8 of the 32 pairs), own token tiles
    for (int i = threadIdx.x; i < n_tokens * 4; i += 256) {
      const int n = i >> 2, k0 = 8 * (i & 3);
      if (static_cast<int>((n >> 5) % gridDim.z) != static_cast<int>(blockIdx.z)) continue;
      const __bf16* qr = q_pe + (static_cast<int64_t>(n) * n_h + head) * kDr + k0;
      const bf16x8_t x1 = load8(qr), x2 = load8(qr + 32);
      const int pos = positions[n];
      const int64_t base = (static_cast<int64_t>(n) * n_h + head) * kD + kDc + k0;
      float y1[8], y2[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float cs, sn;
        rope_cos_sin_inv(pos, rope.inv[k0 + k], &cs, &sn);
        const float a = static_cast<float>(x1[k]), b = static_cast<float>(x2[k]);
        y1[k] = a * cs - b * sn;
        y2[k] = a * sn + b * cs;
      }
      if constexpr (OUT_F32) {
        float* o = static_cast<float*>(q_out) + base;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          o[k] = y1[k];
          o[32 + k] = y2[k];
        }
      } else {
        bf16x8_t o1, o2;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          o1[k] = f32_to_bf16(y1[k]);
          o2[k] = f32_to_bf16(y2[k]);
        }
        __bf16* o = static_cast<__bf16*>(q_out) + base;
        *reinterpret_cast<bf16x8_t*>(o) = o1;
        *reinterpret_cast<bf16x8_t*>(o + 32) = o2;
      }
    }
  }
}

// fp32 latent query rows -> two e4m3 planes + one fp32 scale per (token, head):
// x = row / scale (scale = max|row| / 448), hi = e4m3(x), lo = e4m3((x - hi) * 16),
// so row ~= scale * (hi + lo / 16) to about 8 significant bits.  The output
// row is [hi (576 codes) | lo (576 codes)].
__global__ void __launch_bounds__(64) quantize_rows_fp8_kernel(const float* __restrict__ src,
                                                               uint8_t* __restrict__ dst,
                                                               float* __restrict__ scale_out) {
  const int row = blockIdx.x, lane = threadIdx.x;
  const float* s = src + static_cast<int64_t>(row) * kD;
  float v[9];
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    v[i] = s[lane + 64 * i];
    am = fmaxf(am, fabsf(v[i]));
  }
  am = wave_max(am);
  const float scale = am > 0.f ? am / 448.f : 1.f;
  uint8_t* d = dst + static_cast<int64_t>(row) * (2 * kD);
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    const float x = v[i] / scale;
    const uint32_t hi = f32_to_e4m3(x);
    const uint32_t lo = f32_to_e4m3((x - e4m3_to_f32(hi)) * 16.f);
    d[lane + 64 * i] = static_cast<uint8_t>(hi);
    d[kD + lane + 64 * i] = static_cast<uint8_t>(lo);
  }
  if (lane == 0) scale_out[row] = scale;
}

// ------------------------------------------------------------- out proj
// grid (n_h, d_v/32 column tiles), 4 waves; wave w takes c in [128w, 128w+128)
// (8 k-steps), partials summed through LDS:
// out[n][i][v] = sum_c o[n][i][c] W[i][v][c]
__global__ void __launch_bounds__(256) out_proj_kernel(const __bf16* __restrict__ o_lat,
                                                       const __bf16* __restrict__ w_uv, int n_tokens,
                                                       int n_h, int d_v, __bf16* __restrict__ out) {
  __shared__ f32x16_t red[kProjWaves][kMaxMTiles][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hf = lane >> 5, l32 = lane & 31;
  const int head = blockIdx.x, vt = blockIdx.y;
  const int c_begin = wave * (kDc / kProjWaves);
  const __bf16* wrow = w_uv + (static_cast<int64_t>(head) * d_v + 32 * vt + l32) * kDc + c_begin + 8 * hf;
  bf16x8_t bw[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) bw[j] = load8(wrow + 16 * j);
  for (int m0 = blockIdx.z * 32 * kMaxMTiles; m0 < n_tokens; m0 += gridDim.z * 32 * kMaxMTiles) {
    const int mts = min(kMaxMTiles, (n_tokens - m0 + 31) / 32);
    bf16x8_t oa[kMaxMTiles][8];
#pragma unroll
    for (int mt = 0; mt < kMaxMTiles; ++mt) {
      const int n = m0 + 32 * mt + l32;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        oa[mt][j] = (mt < mts && n < n_tokens)
                        ? load8(o_lat + (static_cast<int64_t>(n) * n_h + head) * kDc + c_begin + 16 * j + 8 * hf)
                        : bf16x8_t{};
    }
    f32x16_t acc[kMaxMTiles];
#pragma unroll
    for (int mt = 0; mt < kMaxMTiles; ++mt) acc[mt] = f32x16_t{};
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int mt = 0; mt < kMaxMTiles; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[mt][j], bw[j], acc[mt], 0, 0, 0);
#pragma unroll
    for (int mt = 0; mt < kMaxMTiles; ++mt) red[wave][mt][lane] = acc[mt];
    __syncthreads();
    const int rl = threadIdx.x & 63, rq = threadIdx.x >> 6;
    for (int mt = 0; mt < mts; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * rq + i;
        float v = 0.f;
#pragma unroll
        for (int wv = 0; wv < kProjWaves; ++wv) v += red[wv][mt][rl][r];
        const int n = m0 + 32 * mt + 8 * (r >> 2) + 4 * (rl >> 5) + (r & 3);
        if (n < n_tokens) out[(static_cast<int64_t>(n) * n_h + head) * d_v + 32 * vt + (rl & 31)] = f32_to_bf16(v);
      }
    __syncthreads();
  }
}

// number of contraction slices: the largest divisor of d_model/64 up to 16,
// so that every wave of a slice gets a whole number of 16-wide k-steps
int append_chunks(int d_model) {
  const int units = d_model / 64;
  int best = 1;
  for (int kc = 1; kc <= 16; ++kc)
    if (units % kc == 0) best = kc;
  return best;
}

// 32-token tiles of the append GEMM run by separate workgroups (grid z), so
// that the latency chain of one workgroup (operand loads, MFMA, reduction,
// stores) covers one tile; beyond kMaxZ tiles a workgroup loops over several.
// (For absorb and out proj a second tile workgroup re-reads the same weight
// slice, which costs more than it saves: they keep one workgroup per slice.)
constexpr int kMaxZ = 16;
int token_tiles(int n_tokens) {
  const int t = (n_tokens + 32 * kMaxMTiles - 1) / (32 * kMaxMTiles);
  return t < 1 ? 1 : (t > kMaxZ ? kMaxZ : t);
}

RopeTable64 rope_table(float theta) {
  RopeTable64 t;
  for (int k = 0; k < 32; ++k) t.inv[k] = std::pow(static_cast<double>(theta), -2.0 * k / kDr);
  return t;
}

}  // namespace

size_t append_mfma_workspace(int n_tokens) {
  return static_cast<size_t>(16) * n_tokens * kD * sizeof(float);
}

hipError_t launch_append_mfma(const AppendArgs& a, hipStream_t st) {
  const float* partial;
  int n_chunks;
  if (a.w != nullptr) {
    n_chunks = append_chunks(a.d_model);
    float* ws = static_cast<float*>(a.workspace);
    hipLaunchKernelGGL(append_proj_kernel, dim3(kD / 32, n_chunks, token_tiles(a.n_tokens)), dim3(256), 0, st,
                       static_cast<const __bf16*>(a.hidden), static_cast<const __bf16*>(a.w),
                       a.n_tokens, a.d_model, a.d_model / n_chunks, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    partial = ws;
  } else {
    n_chunks = 1;
    partial = static_cast<const float*>(a.hidden);
  }
  if (a.cache_dtype == 2)
    hipLaunchKernelGGL(append_finish_kernel<true>, dim3(a.n_tokens), dim3(256), 0, st, partial,
                       n_chunks, a.n_tokens, a.gamma, a.positions, a.slots, a.cache_slots, a.eps,
                       rope_table(a.theta), a.cache, a.cache_scale);
  else
    hipLaunchKernelGGL(append_finish_kernel<false>, dim3(a.n_tokens), dim3(256), 0, st, partial,
                       n_chunks, a.n_tokens, a.gamma, a.positions, a.slots, a.cache_slots, a.eps,
                       rope_table(a.theta), a.cache, a.cache_scale);
  return hipGetLastError();
}

size_t absorb_mfma_workspace(int n_tokens, int n_h, int cache_dtype) {
  return cache_dtype == 2 ? static_cast<size_t>(n_tokens) * n_h * kD * sizeof(float) : 0;
}

hipError_t launch_absorb_q_mfma(const AbsorbArgs& a, hipStream_t st) {
  const dim3 grid(a.n_h, kDc / 128);  // one workgroup per W slice: staging it twice costs more than it saves
  if (a.cache_dtype == 2) {
    hipLaunchKernelGGL(absorb_q_kernel<true>, grid, dim3(256), 0, st,
                       static_cast<const __bf16*>(a.q_nope), static_cast<const __bf16*>(a.q_pe),
                       static_cast<const __bf16*>(a.w_uk), a.positions, a.n_tokens, a.n_h, rope_table(a.theta),
                       a.workspace);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(quantize_rows_fp8_kernel, dim3(a.n_tokens * a.n_h), dim3(64), 0, st,
                       static_cast<const float*>(a.workspace), static_cast<uint8_t*>(a.q_lat),
                       a.q_scale);
  } else {
    hipLaunchKernelGGL(absorb_q_kernel<false>, grid, dim3(256), 0, st,
                       static_cast<const __bf16*>(a.q_nope), static_cast<const __bf16*>(a.q_pe),
                       static_cast<const __bf16*>(a.w_uk), a.positions, a.n_tokens, a.n_h, rope_table(a.theta),
                       a.q_lat);
  }
  return hipGetLastError();
}

hipError_t launch_out_proj_mfma(const OutProjArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(out_proj_kernel, dim3(a.n_h, a.d_v / 32), dim3(256), 0, st,
                     static_cast<const __bf16*>(a.o_lat), static_cast<const __bf16*>(a.w_uv),
                     a.n_tokens, a.n_h, a.d_v, static_cast<__bf16*>(a.out));
  return hipGetLastError();
}

}  // namespace mla
