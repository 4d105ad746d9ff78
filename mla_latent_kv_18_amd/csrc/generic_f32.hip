// Portable fp32 kernels for any MLA dims (no matrix cores).  They carry the
// small workloads whose widths do not fit the MFMA tiles (e.g. d_c = 32,
// d_R = 8) and serve as the fp32 instantiation of every call.
#include "device_common.h"
#include "kernels.h"

namespace mla {

// One workgroup per new token: kv = W h (or the given projection), RMSNorm
// on the latent, RoPE on the key part, write to the cache slot.
__global__ void __launch_bounds__(256) append_f32_kernel(
    const float* __restrict__ hidden, const float* __restrict__ w, const float* __restrict__ gamma,
    const int32_t* __restrict__ positions, const int64_t* __restrict__ slots, int d_model, int d_c,
    int d_r, int64_t cache_slots, float eps, float theta, float* __restrict__ cache) {
  extern __shared__ float smem[];  // [d_c + d_r] + [blockDim] reduction
  const int n = blockIdx.x;
  const int D = d_c + d_r;
  float* kv = smem;
  float* red = smem + D;
  const int64_t slot = slots[n];
  if (slot < 0 || slot >= cache_slots) return;
  for (int r = threadIdx.x; r < D; r += blockDim.x) {
    float acc;
    if (w != nullptr) {
      acc = 0.f;
      const float* hrow = hidden + static_cast<int64_t>(n) * d_model;
      const float* wrow = w + static_cast<int64_t>(r) * d_model;
      for (int k = 0; k < d_model; ++k) acc = fmaf(hrow[k], wrow[k], acc);
    } else {
      acc = hidden[static_cast<int64_t>(n) * D + r];
    }
    kv[r] = acc;
  }
  __syncthreads();
  float ss = 0.f;
  for (int r = threadIdx.x; r < d_c; r += blockDim.x) ss = fmaf(kv[r], kv[r], ss);
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const float inv_rms = rsqrtf(red[0] / static_cast<float>(d_c) + eps);
  float* row = cache + slot * D;
  for (int r = threadIdx.x; r < d_c; r += blockDim.x) row[r] = kv[r] * inv_rms * gamma[r];
  const int half = d_r / 2;
  const int pos = positions[n];
  for (int k = threadIdx.x; k < half; k += blockDim.x) {
    float c, s;
    rope_cos_sin(pos, k, d_r, theta, &c, &s);
    const float x1 = kv[d_c + k], x2 = kv[d_c + half + k];
    row[d_c + k] = x1 * c - x2 * s;
    row[d_c + half + k] = x1 * s + x2 * c;
  }
}

// One workgroup per (token, head): q_lat = W^UK_i^T q_nope ; RoPE(q_pe).
__global__ void __launch_bounds__(256) absorb_q_f32_kernel(
    const float* __restrict__ q_nope, const float* __restrict__ q_pe, const float* __restrict__ w_uk,
    const int32_t* __restrict__ positions, int n_h, int d_h, int d_c, int d_r, float theta,
    float* __restrict__ q_lat) {
  const int n = blockIdx.x / n_h, i = blockIdx.x % n_h;
  const float* q = q_nope + (static_cast<int64_t>(n) * n_h + i) * d_h;
  const float* W = w_uk + static_cast<int64_t>(i) * d_h * d_c;
  float* out = q_lat + (static_cast<int64_t>(n) * n_h + i) * (d_c + d_r);
  for (int c = threadIdx.x; c < d_c; c += blockDim.x) {
    float acc = 0.f;
    for (int a = 0; a < d_h; ++a) acc = fmaf(q[a], W[static_cast<int64_t>(a) * d_c + c], acc);
    out[c] = acc;
  }
  const float* qr = q_pe + (static_cast<int64_t>(n) * n_h + i) * d_r;
  const int half = d_r / 2;
  const int pos = positions[n];
  for (int k = threadIdx.x; k < half; k += blockDim.x) {
    float c, s;
    rope_cos_sin(pos, k, d_r, theta, &c, &s);
    out[d_c + k] = qr[k] * c - qr[half + k] * s;
    out[d_c + half + k] = qr[k] * s + qr[half + k] * c;
  }
}

// One workgroup per (request, query, head): single pass over the visible
// keys in chunks of blockDim tokens with a running max / sum (online
// softmax); the latent-weighted sum accumulates per output column.
__global__ void __launch_bounds__(256) decode_f32_kernel(
    const float* __restrict__ q_lat, const float* __restrict__ cache,
    const int32_t* __restrict__ block_table, int max_blocks, int num_blocks,
    const int32_t* __restrict__ seq_lens,
    int q_len, int n_h, int d_c, int d_r, int block_size, int max_seq_len, float scale,
    float* __restrict__ o_lat, float* __restrict__ lse) {
  extern __shared__ float smem[];  // q [D] | p [blockDim] | red [blockDim] | acc [d_c]
  const int D = d_c + d_r;
  const int head = blockIdx.x % n_h;
  const int t = (blockIdx.x / n_h) % q_len;
  const int b = blockIdx.x / (n_h * q_len);
  const int n = b * q_len + t;
  float* qs = smem;
  float* p = qs + D;
  float* red = p + blockDim.x;
  float* acc = red + blockDim.x;
  const float* q = q_lat + (static_cast<int64_t>(n) * n_h + head) * D;
  for (int d = threadIdx.x; d < D; d += blockDim.x) qs[d] = q[d];
  for (int c = threadIdx.x; c < d_c; c += blockDim.x) acc[c] = 0.f;
  int T = seq_lens[b];
  T = T < 0 ? 0 : (T > max_seq_len ? max_seq_len : T);
  const int visible = T - q_len + t + 1;  // keys 0 .. T - q_len + t
  float m = -INFINITY, l = 0.f;
  const int32_t* bt = block_table + static_cast<int64_t>(b) * max_blocks;
  auto row_of = [&](int j) -> int64_t {
    int blk = bt[j / block_size];
    blk = blk < 0 ? 0 : (blk >= num_blocks ? num_blocks - 1 : blk);
    return static_cast<int64_t>(blk) * block_size + j % block_size;
  };
  __syncthreads();
  for (int j0 = 0; j0 < visible; j0 += blockDim.x) {
    const int j = j0 + threadIdx.x;
    float s = -INFINITY;
    if (j < visible) {
      const float* kr = cache + row_of(j) * D;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], kr[d], dot);
      s = dot * scale;
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = blockDim.x / 2; o > 0; o >>= 1) {
      if (threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
      __syncthreads();
    }
    const float m_new = fmaxf(m, red[0]);
    const float alpha = (m == -INFINITY) ? 0.f : __expf(m - m_new);
    __syncthreads();
    const float pj = (s == -INFINITY) ? 0.f : __expf(s - m_new);
    p[threadIdx.x] = pj;
    red[threadIdx.x] = pj;
    __syncthreads();
    for (int o = blockDim.x / 2; o > 0; o >>= 1) {
      if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
      __syncthreads();
    }
    l = l * alpha + red[0];
    m = m_new;
    const int cnt = min(static_cast<int>(blockDim.x), visible - j0);
    for (int c = threadIdx.x; c < d_c; c += blockDim.x) {
      float a = acc[c] * alpha;
      for (int jj = 0; jj < cnt; ++jj) {
        const int jg = j0 + jj;
        a = fmaf(p[jj], cache[row_of(jg) * D + c], a);
      }
      acc[c] = a;
    }
    __syncthreads();
  }
  float* o = o_lat + (static_cast<int64_t>(n) * n_h + head) * d_c;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  for (int c = threadIdx.x; c < d_c; c += blockDim.x) o[c] = acc[c] * inv;
  if (lse != nullptr && threadIdx.x == 0)
    lse[static_cast<int64_t>(n) * n_h + head] = l > 0.f ? m + __logf(l) : -INFINITY;
}

// One workgroup per (token, head): out = W^UV_i o_lat.
__global__ void __launch_bounds__(256) out_proj_f32_kernel(const float* __restrict__ o_lat,
                                                           const float* __restrict__ w_uv, int n_h,
                                                           int d_c, int d_v, float* __restrict__ out) {
  const int n = blockIdx.x / n_h, i = blockIdx.x % n_h;
  const float* o = o_lat + (static_cast<int64_t>(n) * n_h + i) * d_c;
  const float* W = w_uv + static_cast<int64_t>(i) * d_v * d_c;
  for (int v = threadIdx.x; v < d_v; v += blockDim.x) {
    float acc = 0.f;
    const float* wr = W + static_cast<int64_t>(v) * d_c;
    for (int c = 0; c < d_c; ++c) acc = fmaf(o[c], wr[c], acc);
    out[(static_cast<int64_t>(n) * n_h + i) * d_v + v] = acc;
  }
}

// ------------------------------------------------------------- launchers
hipError_t launch_append_f32(const AppendArgs& a, hipStream_t st) {
  const int D = a.d_c + a.d_r;
  const size_t sh = (D + 256) * sizeof(float);
  hipLaunchKernelGGL(append_f32_kernel, dim3(a.n_tokens), dim3(256), sh, st,
                     static_cast<const float*>(a.hidden), static_cast<const float*>(a.w), a.gamma,
                     a.positions, a.slots, a.d_model, a.d_c, a.d_r, a.cache_slots, a.eps, a.theta,
                     static_cast<float*>(a.cache));
  return hipGetLastError();
}

hipError_t launch_absorb_q_f32(const AbsorbArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(absorb_q_f32_kernel, dim3(a.n_tokens * a.n_h), dim3(256), 0, st,
                     static_cast<const float*>(a.q_nope), static_cast<const float*>(a.q_pe),
                     static_cast<const float*>(a.w_uk), a.positions, a.n_h, a.d_h, a.d_c, a.d_r,
                     a.theta, static_cast<float*>(a.q_lat));
  return hipGetLastError();
}

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t st) {
  const int D = a.d_c + a.d_r;
  const int threads = 256;
  const size_t sh = (D + 2 * threads + a.d_c) * sizeof(float);
  hipLaunchKernelGGL(decode_f32_kernel, dim3(a.batch * a.q_len * a.n_h), dim3(threads), sh, st,
                     static_cast<const float*>(a.q_lat), static_cast<const float*>(a.cache),
                     a.block_table, a.max_blocks, a.num_blocks, a.seq_lens, a.q_len, a.n_h, a.d_c, a.d_r,
                     a.block_size, a.max_seq_len, a.scale, static_cast<float*>(a.o_lat), a.lse);
  return hipGetLastError();
}

hipError_t launch_out_proj_f32(const OutProjArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(out_proj_f32_kernel, dim3(a.n_tokens * a.n_h), dim3(256), 0, st,
                     static_cast<const float*>(a.o_lat), static_cast<const float*>(a.w_uv), a.n_h,
                     a.d_c, a.d_v, static_cast<float*>(a.out));
  return hipGetLastError();
}

}  // namespace mla
