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
// grid (576/32 column tiles, kc chunks of the d_model contraction), one wave.
// partial[kc][n][r] = sum_{k in chunk kc} h[n][k] * W[r][k]
__global__ void __launch_bounds__(64) append_proj_kernel(const __bf16* __restrict__ h,
                                                         const __bf16* __restrict__ w, int n_tokens,
                                                         int d_model, int chunk_len,
                                                         float* __restrict__ partial) {
  const int lane = threadIdx.x, hf = lane >> 5, l32 = lane & 31;
  const int r0 = blockIdx.x * 32, kc = blockIdx.y;
  const int k_begin = kc * chunk_len;
  const __bf16* wrow = w + static_cast<int64_t>(r0 + l32) * d_model + k_begin + 8 * hf;
  for (int m0 = 0; m0 < n_tokens; m0 += 128) {
    f32x16_t acc[4] = {f32x16_t{}, f32x16_t{}, f32x16_t{}, f32x16_t{}};
    const int mt_count = min(4, (n_tokens - m0 + 31) / 32);
    for (int ks = 0; ks < chunk_len / 16; ++ks) {
      const bf16x8_t bw = load8(wrow + 16 * ks);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt < mt_count) {
          const int n = m0 + 32 * mt + l32;
          bf16x8_t a = bf16x8_t{};
          if (n < n_tokens) a = load8(h + static_cast<int64_t>(n) * d_model + k_begin + 16 * ks + 8 * hf);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bw, acc[mt], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt < mt_count) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = m0 + 32 * mt + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (n < n_tokens) partial[(static_cast<int64_t>(kc) * n_tokens + n) * kD + r0 + l32] = acc[mt][r];
        }
      }
    }
  }
}

// One workgroup (256 threads) per token: reduce the partials, RMSNorm the
// latent, rotate the key part, convert, write the cache row.
template <bool FP8>
__global__ void __launch_bounds__(256) append_finish_kernel(
    const float* __restrict__ partial, int n_chunks, int n_tokens, const float* __restrict__ gamma,
    const int32_t* __restrict__ positions, const int64_t* __restrict__ slots, int64_t cache_slots,
    float eps, float theta, void* __restrict__ cache, float* __restrict__ cache_scale) {
  __shared__ float kv[kD];
  __shared__ float red[256];
  const int n = blockIdx.x, tid = threadIdx.x;
  const int64_t slot = slots[n];
  if (slot < 0 || slot >= cache_slots) return;
  for (int c = tid; c < kD; c += 256) {
    float s = 0.f;
    for (int kc = 0; kc < n_chunks; ++kc) s += partial[(static_cast<int64_t>(kc) * n_tokens + n) * kD + c];
    kv[c] = s;
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
      rope_cos_sin(positions[n], k, kDr, theta, &cs, &sn);
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
// grid (n_h, 4 column tiles of 128), one wave.  W^UK_i[:, 128 cols] is staged
// in LDS (128 rows x 16 chunks, chunk ch of row a at a*16 + (ch ^ 4(a%4))) and
// read transposed (ds_read_b64_tr_b16) as the B operand (K = a, N = c).
template <bool OUT_F32>
__global__ void __launch_bounds__(64) absorb_q_kernel(const __bf16* __restrict__ q_nope,
                                                      const __bf16* __restrict__ q_pe,
                                                      const __bf16* __restrict__ w_uk,
                                                      const int32_t* __restrict__ positions,
                                                      int n_tokens, int n_h, float theta,
                                                      void* __restrict__ q_out) {
  __shared__ __attribute__((aligned(16))) char wl[kDh * 256];
  const int lane = threadIdx.x, hf = lane >> 5, l32 = lane & 31;
  const int head = blockIdx.x, ct = blockIdx.y;
  const __bf16* W = w_uk + static_cast<int64_t>(head) * kDh * kDc + ct * 128;
  for (int i = lane; i < kDh * 16; i += 64) {
    const int a = i >> 4, ch = i & 15;
    const bf16x8_t v = load8(W + static_cast<int64_t>(a) * kDc + ch * 8);
    *reinterpret_cast<MLA_LDS bf16x8_t*>((MLA_LDS char*)wl + (a * 16 + (ch ^ (4 * (a & 3)))) * 16) = v;
  }
  __syncthreads();
  const int L = lane & 15, cg = (lane >> 4) & 1;
  for (int m0 = 0; m0 < n_tokens; m0 += 32) {
    f32x16_t acc[4] = {f32x16_t{}, f32x16_t{}, f32x16_t{}, f32x16_t{}};
    const int n_a = m0 + l32;
#pragma unroll
    for (int ks = 0; ks < kDh / 16; ++ks) {
      bf16x8_t a = bf16x8_t{};
      if (n_a < n_tokens) a = load8(q_nope + (static_cast<int64_t>(n_a) * n_h + head) * kDh + 16 * ks + 8 * hf);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        i16x4_t part[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int row = 16 * ks + 8 * hf + 4 * h2 + (L >> 2);
          const int ch = 4 * nt + 2 * cg + ((L & 3) >> 1);
          const int off = (row * 16 + (ch ^ (4 * (row & 3)))) * 16 + 8 * (L & 1);
          part[h2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<MLA_LDS i16x4_t*>((MLA_LDS char*)wl + off));
        }
        const bf16x8_t bfr = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bfr, acc[nt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = m0 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (n < n_tokens) {
          const int64_t idx = (static_cast<int64_t>(n) * n_h + head) * kD + ct * 128 + 32 * nt + l32;
          if constexpr (OUT_F32) static_cast<float*>(q_out)[idx] = acc[nt][r];
          else static_cast<__bf16*>(q_out)[idx] = f32_to_bf16(acc[nt][r]);
        }
      }
  }
  if (ct == 0) {  // RoPE part of the latent query
    for (int i = lane; i < n_tokens * 32; i += 64) {
      const int n = i >> 5, k = i & 31;
      float cs, sn;
      rope_cos_sin(positions[n], k, kDr, theta, &cs, &sn);
      const __bf16* qr = q_pe + (static_cast<int64_t>(n) * n_h + head) * kDr;
      const float x1 = static_cast<float>(qr[k]), x2 = static_cast<float>(qr[32 + k]);
      const int64_t base = (static_cast<int64_t>(n) * n_h + head) * kD + kDc;
      const float y1 = x1 * cs - x2 * sn, y2 = x1 * sn + x2 * cs;
      if constexpr (OUT_F32) {
        static_cast<float*>(q_out)[base + k] = y1;
        static_cast<float*>(q_out)[base + 32 + k] = y2;
      } else {
        static_cast<__bf16*>(q_out)[base + k] = f32_to_bf16(y1);
        static_cast<__bf16*>(q_out)[base + 32 + k] = f32_to_bf16(y2);
      }
    }
  }
}

// fp32 latent query rows -> e4m3 codes + one fp32 scale per (token, head).
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
#pragma unroll
  for (int i = 0; i < 9; ++i) dst[static_cast<int64_t>(row) * kD + lane + 64 * i] = static_cast<uint8_t>(f32_to_e4m3(v[i] / scale));
  if (lane == 0) scale_out[row] = scale;
}

// ------------------------------------------------------------- out proj
// grid (n_h, d_v/32 column tiles), one wave: out[n][i][v] = sum_c o[n][i][c] W[i][v][c]
__global__ void __launch_bounds__(64) out_proj_kernel(const __bf16* __restrict__ o_lat,
                                                      const __bf16* __restrict__ w_uv, int n_tokens,
                                                      int n_h, int d_v, __bf16* __restrict__ out) {
  const int lane = threadIdx.x, hf = lane >> 5, l32 = lane & 31;
  const int head = blockIdx.x, vt = blockIdx.y;
  const __bf16* wrow = w_uv + (static_cast<int64_t>(head) * d_v + 32 * vt + l32) * kDc + 8 * hf;
  for (int m0 = 0; m0 < n_tokens; m0 += 128) {
    f32x16_t acc[4] = {f32x16_t{}, f32x16_t{}, f32x16_t{}, f32x16_t{}};
    const int mt_count = min(4, (n_tokens - m0 + 31) / 32);
#pragma unroll 4
    for (int ks = 0; ks < kDc / 16; ++ks) {
      const bf16x8_t bw = load8(wrow + 16 * ks);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt < mt_count) {
          const int n = m0 + 32 * mt + l32;
          bf16x8_t a = bf16x8_t{};
          if (n < n_tokens) a = load8(o_lat + (static_cast<int64_t>(n) * n_h + head) * kDc + 16 * ks + 8 * hf);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bw, acc[mt], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt < mt_count) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = m0 + 32 * mt + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (n < n_tokens) out[(static_cast<int64_t>(n) * n_h + head) * d_v + 32 * vt + l32] = f32_to_bf16(acc[mt][r]);
        }
      }
    }
  }
}

int append_chunks(int d_model) {
  const int ksteps = d_model / 16;
  int best = 1;
  for (int kc = 1; kc <= 16; ++kc)
    if (ksteps % kc == 0) best = kc;
  return best;
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
    hipLaunchKernelGGL(append_proj_kernel, dim3(kD / 32, n_chunks), dim3(64), 0, st,
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
                       a.theta, a.cache, a.cache_scale);
  else
    hipLaunchKernelGGL(append_finish_kernel<false>, dim3(a.n_tokens), dim3(256), 0, st, partial,
                       n_chunks, a.n_tokens, a.gamma, a.positions, a.slots, a.cache_slots, a.eps,
                       a.theta, a.cache, a.cache_scale);
  return hipGetLastError();
}

size_t absorb_mfma_workspace(int n_tokens, int n_h, int cache_dtype) {
  return cache_dtype == 2 ? static_cast<size_t>(n_tokens) * n_h * kD * sizeof(float) : 0;
}

hipError_t launch_absorb_q_mfma(const AbsorbArgs& a, hipStream_t st) {
  const dim3 grid(a.n_h, kDc / 128);
  if (a.cache_dtype == 2) {
    hipLaunchKernelGGL(absorb_q_kernel<true>, grid, dim3(64), 0, st,
                       static_cast<const __bf16*>(a.q_nope), static_cast<const __bf16*>(a.q_pe),
                       static_cast<const __bf16*>(a.w_uk), a.positions, a.n_tokens, a.n_h, a.theta,
                       a.workspace);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(quantize_rows_fp8_kernel, dim3(a.n_tokens * a.n_h), dim3(64), 0, st,
                       static_cast<const float*>(a.workspace), static_cast<uint8_t*>(a.q_lat),
                       a.q_scale);
  } else {
    hipLaunchKernelGGL(absorb_q_kernel<false>, grid, dim3(64), 0, st,
                       static_cast<const __bf16*>(a.q_nope), static_cast<const __bf16*>(a.q_pe),
                       static_cast<const __bf16*>(a.w_uk), a.positions, a.n_tokens, a.n_h, a.theta,
                       a.q_lat);
  }
  return hipGetLastError();
}

hipError_t launch_out_proj_mfma(const OutProjArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(out_proj_kernel, dim3(a.n_h, a.d_v / 32), dim3(64), 0, st,
                     static_cast<const __bf16*>(a.o_lat), static_cast<const __bf16*>(a.w_uv),
                     a.n_tokens, a.n_h, a.d_v, static_cast<__bf16*>(a.out));
  return hipGetLastError();
}

}  // namespace mla
