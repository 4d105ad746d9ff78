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
// grid (576/(32 RT) row groups, n_chunks slices of the d_model contraction,
// token groups), 4 waves; wave w takes 1/4 of the slice for RT 32-row tiles
// of W.  A pass covers MT 32-token tiles: the weight and activation loads of
// a pass are all issued before its MFMAs (token rows past the end are
// clamped to the last row and never stored), and the 4 wave partials are
// summed through LDS.  Every row group re-reads the activations, so wider
// row groups re-read less of them.
// partial[kc][n][r] = sum_{k in slice kc} h[n][k] * W[r][k]
constexpr int kProjWaves = 4;
constexpr int kKBatch = 8;  // k-steps per wave whose loads are in flight together

template <int RT, int MT>
__global__ void __launch_bounds__(256) append_proj_kernel(const __bf16* __restrict__ h,
                                                          const __bf16* __restrict__ w, int n_tokens,
                                                          int d_model, int chunk_len,
                                                          float* __restrict__ partial) {
  __shared__ f32x16_t red[kProjWaves][RT][MT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hf = lane >> 5, l32 = lane & 31;
  const int r0 = blockIdx.x * 32 * RT, kc = blockIdx.y;
  const int ksteps = chunk_len / 16 / kProjWaves;  // per wave
  const int k_begin = kc * chunk_len + wave * ksteps * 16;
  for (int m0 = blockIdx.z * 32 * MT; m0 < n_tokens; m0 += gridDim.z * 32 * MT) {
    const int mts = min(MT, (n_tokens - m0 + 31) / 32);
    f32x16_t acc[RT][MT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = f32x16_t{};
    for (int kb = 0; kb < ksteps; kb += kKBatch) {
      bf16x8_t bw[RT][kKBatch], ha[MT][kKBatch];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const __bf16* wrow = w + static_cast<int64_t>(r0 + 32 * rt + l32) * d_model + k_begin + 8 * hf;
#pragma unroll
        for (int j = 0; j < kKBatch; ++j) bw[rt][j] = load8(wrow + 16 * min(kb + j, ksteps - 1));
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int n = min(m0 + 32 * mt + l32, n_tokens - 1);
        const __bf16* hrow = h + static_cast<int64_t>(n) * d_model + k_begin + 8 * hf;
#pragma unroll
        for (int j = 0; j < kKBatch; ++j) ha[mt][j] = load8(hrow + 16 * min(kb + j, ksteps - 1));
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the batch's loads in flight together
#pragma unroll
      for (int j = 0; j < kKBatch; ++j)
        if (kb + j < ksteps)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              acc[rt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ha[mt][j], bw[rt][j], acc[rt][mt], 0, 0, 0);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[wave][rt][mt][lane] = acc[rt][mt];
    __syncthreads();
    // thread t sums registers 4*(t/64) .. +3 of lane t%64 over the 4 waves
    const int rl = threadIdx.x & 63, rq = threadIdx.x >> 6;
    for (int mt = 0; mt < mts; ++mt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * rq + i;
          float v = 0.f;
#pragma unroll
          for (int wv = 0; wv < kProjWaves; ++wv) v += red[wv][rt][mt][rl][r];
          const int n = m0 + 32 * mt + 8 * (r >> 2) + 4 * (rl >> 5) + (r & 3);
          if (n < n_tokens)
            partial[(static_cast<int64_t>(kc) * n_tokens + n) * kD + r0 + 32 * rt + (rl & 31)] = v;
        }
    __syncthreads();
  }
}

constexpr int kMaxChunks = 16;  // contraction slices of the append GEMM

// One workgroup (256 threads) per token: reduce the partials, RMSNorm the
// latent, rotate the key part, convert, write the cache row.  Thread t < 144
// owns columns 4t..4t+3; all its partial quads are requested before any is
// summed, and the row's sum of squares and maximum go through wave
// reductions and one LDS word per wave.
template <bool FP8>
__global__ void __launch_bounds__(256) append_finish_kernel(
    const float* __restrict__ partial, int n_chunks, int n_tokens, const float* __restrict__ gamma,
    const int32_t* __restrict__ positions, const int64_t* __restrict__ slots, int64_t cache_slots,
    float eps, RopeTable64 rope, void* __restrict__ cache, float* __restrict__ cache_scale) {
  __shared__ __attribute__((aligned(16))) float kv[kD];
  __shared__ float red[2][4];
  const int n = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t slot = slots[n];
  if (slot < 0 || slot >= cache_slots) return;
  const bool own = tid < kD / 4;
  const int q = min(tid, kD / 4 - 1);  // threads past the row repeat its last quad and store nothing
  // the rotation of this thread's four key columns (threads 128..143 own
  // them; the others compute one they do not use) only needs the position:
  // it is requested first and evaluated while the partials are in flight
  const int rc = 4 * max(q - kDc / 4, 0);
  const int pos = positions[n];
  double inv_freq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) inv_freq[i] = rope.inv[(rc + i) & 31];
  __builtin_amdgcn_sched_barrier(0);
  f32x4_t v[kMaxChunks];
#pragma unroll
  for (int kc = 0; kc < kMaxChunks; ++kc)
    v[kc] = *reinterpret_cast<const f32x4_t*>(
        partial + (static_cast<int64_t>(min(kc, n_chunks - 1)) * n_tokens + n) * kD + 4 * q);
  const f32x4_t g = *reinterpret_cast<const f32x4_t*>(gamma + 4 * min(q, kDc / 4 - 1));
  __builtin_amdgcn_sched_barrier(0);
  float cs[4], sn[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) rope_cos_sin_inv(pos, inv_freq[i], &cs[i], &sn[i]);
  f32x4_t s = f32x4_t{};
#pragma unroll
  for (int kc = 0; kc < kMaxChunks; ++kc)
    if (kc < n_chunks) s += v[kc];
  if (own) *reinterpret_cast<f32x4_t*>(&kv[4 * q]) = s;
  float ss = q < kDc / 4 && own ? s[0] * s[0] + s[1] * s[1] + s[2] * s[2] + s[3] * s[3] : 0.f;
  ss = wave_sum(ss);
  if (lane == 0) red[0][wave] = ss;
  __syncthreads();
  const float inv_rms = rsqrtf((red[0][0] + red[0][1] + red[0][2] + red[0][3]) * (1.f / kDc) + eps);
  f32x4_t o;
  if (q < kDc / 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = s[i] * inv_rms * g[i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = rc + i, k = c & 31;
      const float x1 = kv[kDc + k], x2 = kv[kDc + 32 + k];
      o[i] = c < 32 ? x1 * cs[i] - x2 * sn[i] : x1 * sn[i] + x2 * cs[i];
    }
  }
  if constexpr (!FP8) {
    if (own) {
      bf16x4_t b;
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = f32_to_bf16(o[i]);
      *reinterpret_cast<bf16x4_t*>(static_cast<__bf16*>(cache) + slot * kD + 4 * q) = b;
    }
  } else {
    float am = 0.f;
    if (own)
#pragma unroll
      for (int i = 0; i < 4; ++i) am = fmaxf(am, fabsf(o[i]));
    am = wave_max(am);
    if (lane == 0) red[1][wave] = am;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
    const float scale = amax > 0.f ? amax / 448.f : 1.f;
    if (own) {
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) packed |= f32_to_e4m3(o[i] / scale) << (8 * i);
      *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(cache) + slot * kD + 4 * q) = packed;
    }
    if (tid == 0) cache_scale[slot] = scale;
  }
}

// --------------------------------------------------------------- absorb q
// grid (n_h, 4 column tiles of 128), 4 waves.  W^UK_i[:, 128 cols] is staged
// in LDS (128 rows x 16 chunks, chunk ch of row a at a*16 + (ch ^ 4(a%4)))
// and read transposed (ds_read_b64_tr_b16) as the B operand (K = a, N = c);
// wave w produces columns 32w..32w+31 of the tile, MT 32-token tiles per
// pass.  Column tile ct also rotates pairs 8ct..8ct+7 of the RoPE part: item
// i = (token i/8, pair 8ct + i%8), thread t takes items t, t+256, ...  The
// first pass's query rows and the first RoPE item's inputs are requested
// with the weight slice, and that item's cos/sin are evaluated while they
// are in flight; token rows past the end are clamped to the last row and
// never stored.
template <bool OUT_F32, int MT>
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
  // the first RoPE item's inputs are requested first, so that its rotation
  // only waits for them
  const int pair = 8 * ct + (threadIdx.x & 7);
  int item = min(static_cast<int>(threadIdx.x), 8 * n_tokens - 1);
  auto rope_in = [&](int n) { return q_pe + (static_cast<int64_t>(n) * n_h + head) * kDr + pair; };
  const int pos = positions[item >> 3];
  float x1 = static_cast<float>(*rope_in(item >> 3)), x2 = static_cast<float>(*(rope_in(item >> 3) + 32));
  const double inv_freq = rope.inv[pair];
  __builtin_amdgcn_sched_barrier(0);
  bf16x8_t v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = threadIdx.x + 256 * j;
    v[j] = load8(W + static_cast<int64_t>(i >> 4) * kDc + (i & 15) * 8);
  }
  bf16x8_t a[MT][kDh / 16];
  auto load_queries = [&](int m0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int n = min(m0 + 32 * mt + l32, n_tokens - 1);
      const __bf16* qr = q_nope + (static_cast<int64_t>(n) * n_h + head) * kDh + 8 * hf;
#pragma unroll
      for (int ks = 0; ks < kDh / 16; ++ks) a[mt][ks] = load8(qr + 16 * ks);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the pass's loads in flight together
  };
  load_queries(0);
  float cs, sn;
  rope_cos_sin_inv(pos, inv_freq, &cs, &sn);  // while the weight and query loads are in flight
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = threadIdx.x + 256 * j, r = i >> 4, ch = i & 15;
    *reinterpret_cast<MLA_LDS bf16x8_t*>((MLA_LDS char*)wl + (r * 16 + (ch ^ (4 * (r & 3)))) * 16) = v[j];
  }
  __syncthreads();
  const int L = lane & 15, cg = (lane >> 4) & 1;
  for (int m0 = 0;;) {
    f32x16_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16_t{};
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
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt][ks], bfr, acc[mt], 0, 0, 0);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = m0 + 32 * mt + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (n < n_tokens) {
          const int64_t idx = (static_cast<int64_t>(n) * n_h + head) * kD + ct * 128 + 32 * wave + l32;
          if constexpr (OUT_F32) static_cast<float*>(q_out)[idx] = acc[mt][r];
          else static_cast<__bf16*>(q_out)[idx] = f32_to_bf16(acc[mt][r]);
        }
      }
    m0 += 32 * MT;
    if (m0 >= n_tokens) break;
    load_queries(m0);
  }
  // RoPE part of the latent query
  for (int i = threadIdx.x; i < 8 * n_tokens; i += 256) {
    const int n = i >> 3;
    if (i != item) {
      item = i;
      x1 = static_cast<float>(*rope_in(n));
      x2 = static_cast<float>(*(rope_in(n) + 32));
      rope_cos_sin_inv(positions[n], inv_freq, &cs, &sn);
    }
    const int64_t base = (static_cast<int64_t>(n) * n_h + head) * kD + kDc + pair;
    const float y1 = x1 * cs - x2 * sn, y2 = x1 * sn + x2 * cs;
    if constexpr (OUT_F32) {
      static_cast<float*>(q_out)[base] = y1;
      static_cast<float*>(q_out)[base + 32] = y2;
    } else {
      static_cast<__bf16*>(q_out)[base] = f32_to_bf16(y1);
      static_cast<__bf16*>(q_out)[base + 32] = f32_to_bf16(y2);
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
// grid (n_h, d_v/(32 VT)), 4 waves; a workgroup owns VT 32-row tiles of
// W^UV_i, and wave w takes c in [128w, 128w+128) (8 k-steps) of each; the
// wave partials are summed through LDS:
// out[n][i][v] = sum_c o[n][i][c] W[i][v][c]
// A pass covers MT 32-token tiles whose o_lat loads are issued together (the
// first pass's with the weight loads); token rows past the end are clamped
// to the last row and never stored.  Every workgroup of a head reads that
// head's o_lat rows, so fewer, wider workgroups re-read less of them.
template <int VT, int MT>
__global__ void __launch_bounds__(256) out_proj_kernel(const __bf16* __restrict__ o_lat,
                                                       const __bf16* __restrict__ w_uv, int n_tokens,
                                                       int n_h, int d_v, __bf16* __restrict__ out) {
  __shared__ f32x16_t red[kProjWaves][VT][MT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hf = lane >> 5, l32 = lane & 31;
  const int head = blockIdx.x, v0 = 32 * VT * blockIdx.y;
  const int c_begin = wave * (kDc / kProjWaves);
  bf16x8_t bw[VT][8];
#pragma unroll
  for (int vt = 0; vt < VT; ++vt) {
    const __bf16* wrow =
        w_uv + (static_cast<int64_t>(head) * d_v + v0 + 32 * vt + l32) * kDc + c_begin + 8 * hf;
#pragma unroll
    for (int j = 0; j < 8; ++j) bw[vt][j] = load8(wrow + 16 * j);
  }
  bf16x8_t oa[MT][8];
  auto load_rows = [&](int m0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int n = min(m0 + 32 * mt + l32, n_tokens - 1);
      const __bf16* orow = o_lat + (static_cast<int64_t>(n) * n_h + head) * kDc + c_begin + 8 * hf;
#pragma unroll
      for (int j = 0; j < 8; ++j) oa[mt][j] = load8(orow + 16 * j);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the pass's loads in flight together
  };
  load_rows(0);
  for (int m0 = 0;;) {
    const int mts = min(MT, (n_tokens - m0 + 31) / 32);
    f32x16_t acc[VT][MT];
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[vt][mt] = f32x16_t{};
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int vt = 0; vt < VT; ++vt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[vt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[mt][j], bw[vt][j], acc[vt][mt], 0, 0, 0);
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[wave][vt][mt][lane] = acc[vt][mt];
    __syncthreads();
    // thread t sums registers 4*(t/64) .. +3 of lane t%64 over the 4 waves
    const int rl = threadIdx.x & 63, rq = threadIdx.x >> 6;
    for (int mt = 0; mt < mts; ++mt)
#pragma unroll
      for (int vt = 0; vt < VT; ++vt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * rq + i;
          float v = 0.f;
#pragma unroll
          for (int wv = 0; wv < kProjWaves; ++wv) v += red[wv][vt][mt][rl][r];
          const int n = m0 + 32 * mt + 8 * (r >> 2) + 4 * (rl >> 5) + (r & 3);
          if (n < n_tokens)
            out[(static_cast<int64_t>(n) * n_h + head) * d_v + v0 + 32 * vt + (rl & 31)] = f32_to_bf16(v);
        }
    m0 += 32 * MT;
    if (m0 >= n_tokens) break;
    __syncthreads();
    load_rows(m0);
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

// Grid shapes, measured at 64 tokens of the V3 shape (back-to-back calls):
// wider workgroups (2 or 3 row tiles per append workgroup, 2 or 4 W^UV row
// tiles per out-proj workgroup) re-read fewer activation bytes but run 1-6 us
// slower than one 32-row tile each, and two token tiles per append pass cost
// 2 us more than one.  Token groups of the append GEMM (kAppendMT 32-token
// tiles each) run in separate workgroups (grid z); beyond kMaxZ groups a
// workgroup loops over several.  (For absorb and out proj a second token
// workgroup would re-read the same weight slice: they keep one workgroup per
// slice and hold up to two token tiles per pass.)
constexpr int kAppendMT = 1;
constexpr int kAppendRT = 1;  // 32-row tiles of W per append workgroup (a divisor of 576 / 32 = 18)
constexpr int kOutVT = 1;    // 32-row tiles of W^UV_i per out-proj workgroup (a divisor of d_v / 32)
constexpr int kMaxZ = 16;
int token_groups(int n_tokens, int mt) {
  const int t = (n_tokens + 32 * mt - 1) / (32 * mt);
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
    auto kern = append_proj_kernel<kAppendRT, kAppendMT>;
    hipLaunchKernelGGL(kern, dim3(kD / (32 * kAppendRT), n_chunks, token_groups(a.n_tokens, kAppendMT)), dim3(256),
                       0, st,
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
  const bool one = a.n_tokens <= 32;  // one token tile per pass is enough
  const auto q_nope = static_cast<const __bf16*>(a.q_nope);
  const auto q_pe = static_cast<const __bf16*>(a.q_pe);
  const auto w_uk = static_cast<const __bf16*>(a.w_uk);
  if (a.cache_dtype == 2) {
    auto kern = one ? absorb_q_kernel<true, 1> : absorb_q_kernel<true, 2>;
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, q_nope, q_pe, w_uk, a.positions, a.n_tokens, a.n_h,
                       rope_table(a.theta), a.workspace);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(quantize_rows_fp8_kernel, dim3(a.n_tokens * a.n_h), dim3(64), 0, st,
                       static_cast<const float*>(a.workspace), static_cast<uint8_t*>(a.q_lat),
                       a.q_scale);
  } else {
    auto kern = one ? absorb_q_kernel<false, 1> : absorb_q_kernel<false, 2>;
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, q_nope, q_pe, w_uk, a.positions, a.n_tokens, a.n_h,
                       rope_table(a.theta), a.q_lat);
  }
  return hipGetLastError();
}

hipError_t launch_out_proj_mfma(const OutProjArgs& a, hipStream_t st) {
  constexpr int VT = kOutVT;
  auto kern = a.n_tokens <= 32 ? out_proj_kernel<VT, 1> : out_proj_kernel<VT, 2>;
  hipLaunchKernelGGL(kern, dim3(a.n_h, a.d_v / (32 * VT)), dim3(256), 0, st,
                     static_cast<const __bf16*>(a.o_lat), static_cast<const __bf16*>(a.w_uv),
                     a.n_tokens, a.n_h, a.d_v, static_cast<__bf16*>(a.out));
  return hipGetLastError();
}

}  // namespace mla
