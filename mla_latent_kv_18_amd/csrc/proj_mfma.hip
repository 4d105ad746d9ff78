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
#include "lds_dma.h"

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
constexpr int kAppendRTk = 1;  // 32-row tiles of W per append workgroup
constexpr int kAppendMTk = 1;  // 32-token tiles per append pass
constexpr int kKBatch = 8;  // k-steps per wave whose loads are in flight together

// workgroup (bx, by, bz) of a (D / (32 RT), n_chunks, gz) grid
// Hidden-state rows of one 32-token pass staged in LDS for the append GEMM
// (chunk_len <= kStageMaxLen): row r's 16-byte chunk c at r * (C + 1) + c
// with C = chunk_len / 8 chunks per row; the odd row stride puts the
// fragment reads of 32 rows at one column on 16 distinct bank groups.  The
// copies move whole 1 KB runs of that layout (the pad chunk repeats a valid
// one).  Fragment loads straight from global memory touched 32 rows per
// instruction.
constexpr int kStageMaxLen = 512;
constexpr int kStageBytes = (32 * (kStageMaxLen / 8 + 1) * 16 + 1023) / 1024 * 1024;  // 33 KB

template <int RT, int MT, int D>
__device__ __forceinline__ void append_proj_body(const __bf16* __restrict__ h, const __bf16* __restrict__ w,
                                                 int n_tokens, int d_model, int chunk_len,
                                                 float* __restrict__ partial, int bx, int by, int bz, int gz,
                                                 MLA_LDS f32x4_t (*red)[RT][MT][4][64], MLA_LDS char* hs) {
  static_assert(MT == 1, "the staged hidden rows hold one 32-token tile");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hf = lane >> 5, l32 = lane & 31;
  const int r0 = bx * 32 * RT, kc = by;
  const int ksteps = chunk_len / 16 / kProjWaves;  // per wave
  const int k_begin = kc * chunk_len + wave * ksteps * 16;
  const bool staged = chunk_len <= kStageMaxLen;
  const int row_chunks = chunk_len / 8, stride = row_chunks + 1;
  const uint32_t hs_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(hs));
  for (int m0 = bz * 32 * MT; m0 < n_tokens; m0 += gz * 32 * MT) {
    const int mts = min(MT, (n_tokens - m0 + 31) / 32);
    f32x16_t acc[RT][MT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = f32x16_t{};
    if (staged) {
      const int copies = (32 * stride + 63) / 64;
      for (int i = wave; i < copies; i += kProjWaves) {
        const int pidx = 64 * i + lane;
        const int r = min(pidx / stride, 31), c = min(pidx - (pidx / stride) * stride, row_chunks - 1);
        const int n = min(m0 + r, n_tokens - 1);
        dma16(h + static_cast<int64_t>(n) * d_model + kc * chunk_len + 8 * c, hs_addr + i * 1024);
      }
    }
    for (int kb = 0; kb < ksteps; kb += kKBatch) {
      bf16x8_t bw[RT][kKBatch], ha[MT][kKBatch];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const __bf16* wrow = w + static_cast<int64_t>(r0 + 32 * rt + l32) * d_model + k_begin + 8 * hf;
#pragma unroll
        for (int j = 0; j < kKBatch; ++j) bw[rt][j] = load8(wrow + 16 * min(kb + j, ksteps - 1));
      }
      if (staged) {
        wait_vmcnt<0>();
        __syncthreads();  // every wave's copies (and this batch's weight loads) have landed
#pragma unroll
        for (int j = 0; j < kKBatch; ++j) {
          const int c = 2 * (wave * ksteps + min(kb + j, ksteps - 1)) + hf;
          ha[0][j] = *reinterpret_cast<MLA_LDS const bf16x8_t*>(hs + (l32 * stride + c) * 16);
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int n = min(m0 + 32 * mt + l32, n_tokens - 1);
          const __bf16* hrow = h + static_cast<int64_t>(n) * d_model + k_begin + 8 * hf;
#pragma unroll
          for (int j = 0; j < kKBatch; ++j) ha[mt][j] = load8(hrow + 16 * min(kb + j, ksteps - 1));
        }
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
    if (staged) __syncthreads();  // every wave has read the staged rows (the reduction may share the area)
    // registers 4q..4q+3 of each lane go to LDS as one 16-byte quad, quads
    // of one q contiguous over the lanes (conflict-free stores and loads)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          red[wave][rt][mt][q][lane] = f32x4_t{acc[rt][mt][4 * q], acc[rt][mt][4 * q + 1], acc[rt][mt][4 * q + 2],
                                               acc[rt][mt][4 * q + 3]};
    __syncthreads();
    // thread t sums registers 4*(t/64) .. +3 of lane t%64 over the 4 waves
    const int rl = threadIdx.x & 63, rq = threadIdx.x >> 6;
    for (int mt = 0; mt < mts; ++mt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4_t v = red[0][rt][mt][rq][rl];
#pragma unroll
        for (int wv = 1; wv < kProjWaves; ++wv) v += red[wv][rt][mt][rq][rl];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * rq + i;
          const int n = m0 + 32 * mt + 8 * (r >> 2) + 4 * (rl >> 5) + (r & 3);
          if (n < n_tokens)
            partial[(static_cast<int64_t>(kc) * n_tokens + n) * D + r0 + 32 * rt + (rl & 31)] = v[i];
        }
      }
    __syncthreads();
  }
}

template <int RT, int MT, int D>
__global__ void __launch_bounds__(256) append_proj_kernel(const __bf16* __restrict__ h,
                                                          const __bf16* __restrict__ w, int n_tokens,
                                                          int d_model, int chunk_len,
                                                          float* __restrict__ partial) {
  __shared__ __attribute__((aligned(1024))) char lds[kStageBytes];
  static_assert(kProjWaves * RT * MT * 4 * 64 * 16 <= kStageBytes, "the reduction shares the staging area");
  append_proj_body<RT, MT, D>(h, w, n_tokens, d_model, chunk_len, partial, blockIdx.x, blockIdx.y, blockIdx.z,
                              gridDim.z, (MLA_LDS f32x4_t(*)[RT][MT][4][64])(MLA_LDS char*)lds, (MLA_LDS char*)lds);
}

constexpr int kMaxChunks = 16;  // contraction slices of the append GEMM

// One workgroup (256 threads) per token: reduce the partials, RMSNorm the
// latent, rotate the key part, convert, write the cache row.  Thread t < D/4
// owns columns 4t..4t+3; all its partial quads are requested before any is
// summed, and the row's sum of squares and maximum go through wave
// reductions and one LDS word per wave.  D = d_c + d_R (576, or 512 without
// the RoPE part).  Stored forms (OUT):
//   kOutBf16  the row in bf16
//   kOutFp8   e4m3 codes of row / s, s = max|row| / 448 in cache_scale[slot]
//   kOutFp4   MX FP4: per 32 columns one E8M0 scale 2^(floor(log2 max) - 2)
//             and E2M1 codes of x / scale (nearest, ties to even, saturating
//             at 6), two per byte (element 2i in the low nibble), then the
//             D/32 scale bytes and zero padding to 16 bytes
//   kOutFp8Kr e4m3 codes of the latent / s, s the smallest power of two with
//             max|latent| / s <= 448, in cache_scale[slot], then the RoPE
//             key in bf16 (a power-of-two s keeps code * s exact in bf16)
enum { kOutBf16 = 0, kOutFp8 = 1, kOutFp4 = 2, kOutFp8Kr = 3 };

template <int D, int OUT>
constexpr int stored_row_bytes() {
  return OUT == kOutBf16 ? 2 * D : OUT == kOutFp8 ? D : OUT == kOutFp4 ? (D / 2 + D / 32 + 15) / 16 * 16
                                                                        : kDc + 2 * (D - kDc);
}

// E2M1 code of y (magnitude index 0..7 for 0, 0.5, 1, 1.5, 2, 3, 4, 6 plus the
// sign bit): nearest value, ties to the even index, saturating at 6.
__device__ __forceinline__ uint32_t f32_to_e2m1(float y) {
  const float a = fabsf(y);
  uint32_t m = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
             : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.f ? 6u : 7u;
  return m | (__float_as_uint(y) >> 31 << 3);
}

template <int D, int OUT>
__global__ void __launch_bounds__(256) append_finish_kernel(
    const float* __restrict__ partial, int n_chunks, int n_tokens, const float* __restrict__ gamma,
    const int32_t* __restrict__ positions, const int64_t* __restrict__ slots, int64_t cache_slots,
    float eps, RopeTable64 rope, void* __restrict__ cache, float* __restrict__ cache_scale) {
  constexpr bool kRope = D > kDc;
  constexpr int kRow = stored_row_bytes<D, OUT>();
  __shared__ __attribute__((aligned(16))) float kv[D];
  __shared__ float red[2][4];
  const int n = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t slot = slots[n];
  if (slot < 0 || slot >= cache_slots) return;
  const bool own = tid < D / 4;
  const int q = min(tid, D / 4 - 1);  // threads past the row repeat its last quad and store nothing
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
        partial + (static_cast<int64_t>(min(kc, n_chunks - 1)) * n_tokens + n) * D + 4 * q);
  const f32x4_t g = *reinterpret_cast<const f32x4_t*>(gamma + 4 * min(q, kDc / 4 - 1));
  __builtin_amdgcn_sched_barrier(0);
  float cs[4] = {}, sn[4] = {};
  if constexpr (kRope) {
#pragma unroll
    for (int i = 0; i < 4; ++i) rope_cos_sin_inv(pos, inv_freq[i], &cs[i], &sn[i]);
  }
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
  uint8_t* row = static_cast<uint8_t*>(cache) + slot * kRow;
  if constexpr (OUT == kOutBf16) {
    if (own) {
      bf16x4_t b;
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = f32_to_bf16(o[i]);
      *reinterpret_cast<bf16x4_t*>(row + 8 * q) = b;
    }
  } else if constexpr (OUT == kOutFp4) {
    // the 8 threads of a 32-column block are 8 consecutive lanes
    float am = fmaxf(fmaxf(fabsf(o[0]), fabsf(o[1])), fmaxf(fabsf(o[2]), fabsf(o[3])));
    am = fmaxf(am, __shfl_xor(am, 1));
    am = fmaxf(am, __shfl_xor(am, 2));
    am = fmaxf(am, __shfl_xor(am, 4));
    int ex = 0;
    frexpf(am, &ex);                                  // am = f 2^ex, f in [0.5, 1)
    const int shared = am > 0.f ? min(max(ex - 3, -127), 127) : 0;
    uint32_t code[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) code[i] = f32_to_e2m1(ldexpf(o[i], -shared));
    if (own) {
      *reinterpret_cast<uint16_t*>(row + 2 * q) =
          static_cast<uint16_t>(code[0] | code[1] << 4 | code[2] << 8 | code[3] << 12);
      if ((q & 7) == 0) row[D / 2 + q / 8] = static_cast<uint8_t>(shared + 127);
      if (q == 0)
        for (int bt = D / 2 + D / 32; bt < kRow; bt += 2) *reinterpret_cast<uint16_t*>(row + bt) = 0;
    }
  } else {
    constexpr bool kLatentOnly = OUT == kOutFp8Kr;
    float am = 0.f;
    if (own && (!kLatentOnly || q < kDc / 4))
#pragma unroll
      for (int i = 0; i < 4; ++i) am = fmaxf(am, fabsf(o[i]));
    am = wave_max(am);
    if (lane == 0) red[1][wave] = am;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
    float scale = amax > 0.f ? amax / 448.f : 1.f;
    if (kLatentOnly && amax > 0.f) {
      int ex;
      const float f = frexpf(amax, &ex);  // amax = f 2^ex, f in [0.5, 1): amax / 2^(ex-9) <= 448 iff f <= 7/8
      scale = ldexpf(1.f, f <= 0.875f ? ex - 9 : ex - 8);
    }
    if (own) {
      if (!kLatentOnly || q < kDc / 4) {
        uint32_t packed = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) packed |= f32_to_e4m3(o[i] / scale) << (8 * i);
        *reinterpret_cast<uint32_t*>(row + 4 * q) = packed;
      } else {
        bf16x4_t b;
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = f32_to_bf16(o[i]);
        *reinterpret_cast<bf16x4_t*>(row + kDc + 8 * (q - kDc / 4)) = b;
      }
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
// workgroup (head, column tile ct) of an (n_h, d_c / 128) grid
template <bool OUT_F32, int MT, int DR>
__device__ __forceinline__ void absorb_q_body(const __bf16* __restrict__ q_nope, const __bf16* __restrict__ q_pe,
                                              const __bf16* __restrict__ w_uk,
                                              const int32_t* __restrict__ positions, int n_tokens, int n_h,
                                              const RopeTable64& rope, void* __restrict__ q_out, int head, int ct,
                                              MLA_LDS char* wl, MLA_LDS char* ql) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hf = lane >> 5, l32 = lane & 31;
  const __bf16* W = w_uk + static_cast<int64_t>(head) * kDh * kDc + ct * 128;
  // the first RoPE item's inputs are requested first, so that its rotation
  // only waits for them
  constexpr int kRowD = kDc + DR;  // width of a latent-query row
  const int pair = 8 * ct + (threadIdx.x & 7);
  int item = min(static_cast<int>(threadIdx.x), 8 * n_tokens - 1);
  auto rope_in = [&](int n) { return q_pe + (static_cast<int64_t>(n) * n_h + head) * kDr + pair; };
  float x1 = 0.f, x2 = 0.f;
  int pos = 0;
  if constexpr (DR > 0) {
    pos = positions[item >> 3];
    x1 = static_cast<float>(*rope_in(item >> 3));
    x2 = static_cast<float>(*(rope_in(item >> 3) + 32));
  }
  const double inv_freq = rope.inv[pair];
  __builtin_amdgcn_sched_barrier(0);
  bf16x8_t v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = threadIdx.x + 256 * j;
    v[j] = load8(W + static_cast<int64_t>(i >> 4) * kDc + (i & 15) * 8);
  }
  // The pass's query rows (the head's 128 content values, 256 B per token)
  // are copied into LDS four rows per 1 KB copy, chunk c of row r at
  // c ^ (r & 15), and every wave reads its A fragments from there (fragment
  // loads straight from global memory touched 32 rows per instruction).
  bf16x8_t a[MT][kDh / 16];
  const uint32_t ql_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ql));
  auto copy_queries = [&](int m0) {
#pragma unroll
    for (int i = wave; i < 8 * MT; i += kProjWaves) {
      const int r = 4 * i + (lane >> 4);
      const int n = min(m0 + r, n_tokens - 1);
      dma16(q_nope + (static_cast<int64_t>(n) * n_h + head) * kDh + 8 * ((lane & 15) ^ (r & 15)), ql_addr + i * 1024);
    }
  };
  auto read_queries = [&]() {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = 32 * mt + l32;
#pragma unroll
      for (int ks = 0; ks < kDh / 16; ++ks)
        a[mt][ks] = *reinterpret_cast<MLA_LDS const bf16x8_t*>(ql + (r * 16 + ((2 * ks + hf) ^ (r & 15))) * 16);
    }
  };
  copy_queries(0);
  float cs = 1.f, sn = 0.f;
  if constexpr (DR > 0) rope_cos_sin_inv(pos, inv_freq, &cs, &sn);  // while the weight and query loads are in flight
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = threadIdx.x + 256 * j, r = i >> 4, ch = i & 15;
    *reinterpret_cast<MLA_LDS bf16x8_t*>((MLA_LDS char*)wl + (r * 16 + (ch ^ (4 * (r & 3)))) * 16) = v[j];
  }
  wait_vmcnt<0>();
  __syncthreads();  // the weight slice and every wave's query rows are in LDS
  read_queries();
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
          const int64_t idx = (static_cast<int64_t>(n) * n_h + head) * kRowD + ct * 128 + 32 * wave + l32;
          if constexpr (OUT_F32) static_cast<float*>(q_out)[idx] = acc[mt][r];
          else static_cast<__bf16*>(q_out)[idx] = f32_to_bf16(acc[mt][r]);
        }
      }
    m0 += 32 * MT;
    if (m0 >= n_tokens) break;
    __syncthreads();  // every wave has read this pass's query rows
    copy_queries(m0);
    wait_vmcnt<0>();
    __syncthreads();
    read_queries();
  }
  // RoPE part of the latent query
  if constexpr (DR == 0) return;
  for (int i = threadIdx.x; i < 8 * n_tokens; i += 256) {
    const int n = i >> 3;
    if (i != item) {
      item = i;
      x1 = static_cast<float>(*rope_in(n));
      x2 = static_cast<float>(*(rope_in(n) + 32));
      rope_cos_sin_inv(positions[n], inv_freq, &cs, &sn);
    }
    const int64_t base = (static_cast<int64_t>(n) * n_h + head) * kRowD + kDc + pair;
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

template <bool OUT_F32, int MT, int DR>
__global__ void __launch_bounds__(256) absorb_q_kernel(const __bf16* __restrict__ q_nope,
                                                       const __bf16* __restrict__ q_pe,
                                                       const __bf16* __restrict__ w_uk,
                                                       const int32_t* __restrict__ positions,
                                                       int n_tokens, int n_h, RopeTable64 rope,
                                                       void* __restrict__ q_out) {
  __shared__ __attribute__((aligned(1024))) char wl[kDh * 256 + 32 * MT * kDh * 2];
  absorb_q_body<OUT_F32, MT, DR>(q_nope, q_pe, w_uk, positions, n_tokens, n_h, rope, q_out, blockIdx.x, blockIdx.y,
                                 (MLA_LDS char*)wl, (MLA_LDS char*)wl + kDh * 256);
}

// The append's down-projection and the latent query in one launch: the first
// n_append workgroups take the append GEMM's (x, y, z) grid, the rest the
// absorb grid (n_h, d_c / 128).  Both stream their own weights (W_dkv_kr,
// W^UK), so together they keep more of HBM busy than either alone.
struct AppendAbsorbArgs {
  const __bf16* h;
  const __bf16* w;
  int n_tokens, d_model, chunk_len;
  float* partial;
  int ax, ay, az;  // append grid
  const __bf16* q_nope;
  const __bf16* q_pe;
  const __bf16* w_uk;
  const int32_t* positions;
  int n_q, n_h;
  void* q_out;
};

// The two grids are interleaved (workgroup 2i appends, 2i+1 absorbs, while
// both have workgroups left), so that the dispatcher starts both weight
// streams at once; the two bodies share one LDS area.  Four waves per SIMD
// (at most 128 registers, 102 used): four workgroups fit a CU, so the 1088
// workgroups of the V3 shape at 64 tokens run in about one round.
template <int D, bool OUT_F32, int MT_Q, int DR>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4)))
append_absorb_kernel(AppendAbsorbArgs a, RopeTable64 rope) {
  constexpr int kAbsorbBytes = kDh * 256 + 32 * MT_Q * kDh * 2;  // weight slice + one pass's query rows
  __shared__ __attribute__((aligned(1024))) char lds[kStageBytes > kAbsorbBytes ? kStageBytes : kAbsorbBytes];
  const int id = blockIdx.x, n_append = a.ax * a.ay * a.az, ct_tiles = kDc / 128;
  const int n_absorb = a.n_h * ct_tiles, both = min(n_append, n_absorb);
  int ja = -1, jq = -1;
  if (id < 2 * both) {
    (id & 1 ? jq : ja) = id >> 1;
  } else if (n_append > both) {
    ja = id - both;
  } else {
    jq = id - both;
  }
  if (ja >= 0) {
    append_proj_body<kAppendRTk, kAppendMTk, D>(
        a.h, a.w, a.n_tokens, a.d_model, a.chunk_len, a.partial, ja % a.ax, (ja / a.ax) % a.ay,
        ja / (a.ax * a.ay), a.az, (MLA_LDS f32x4_t(*)[kAppendRTk][kAppendMTk][4][64])(MLA_LDS char*)lds,
        (MLA_LDS char*)lds);
  } else {
    absorb_q_body<OUT_F32, MT_Q, DR>(a.q_nope, a.q_pe, a.w_uk, a.positions, a.n_q, a.n_h, rope, a.q_out,
                                     jq / ct_tiles, jq % ct_tiles, (MLA_LDS char*)lds, (MLA_LDS char*)lds + kDh * 256);
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
// A pass covers MT 32-token tiles.  Their o_lat rows (the head's 512 latent
// values, 1 KB each) are copied whole into LDS, one row per direct 1 KB copy
// (token row r at r * 1024, its 16-byte chunk c at c ^ (r & 15), so that the
// fragment reads of 32 rows at one column hit 16 distinct bank groups), and
// every wave reads its A fragments from there; the first pass's copies are
// issued with the weight loads.  Fragment loads straight from global memory
// touched 32 rows per instruction.  Token rows past the end are clamped to
// the last row and never stored.  The cross-wave reduction reuses the LDS
// area.
template <int VT, int MT>
__global__ void __launch_bounds__(256) out_proj_kernel(const __bf16* __restrict__ o_lat,
                                                       const __bf16* __restrict__ w_uv, int n_tokens,
                                                       int n_h, int d_v, __bf16* __restrict__ out) {
  constexpr int kRowsBytes = 32 * MT * 1024;
  constexpr int kRedBytes = kProjWaves * VT * MT * 4 * 64 * 16;
  static_assert(kRedBytes <= kRowsBytes, "the reduction reuses the token rows' area");
  __shared__ __attribute__((aligned(1024))) char lds[kRowsBytes + 32 * VT * 1024];
  MLA_LDS char* ol = (MLA_LDS char*)lds;
  auto red = (MLA_LDS f32x4_t(*)[VT][MT][4][64])(MLA_LDS char*)lds;
  const uint32_t ol_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ol));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hf = lane >> 5, l32 = lane & 31;
  const int head = blockIdx.x, v0 = 32 * VT * blockIdx.y;
  const int c_begin = wave * (kDc / kProjWaves);
  // the workgroup's W^UV_i rows (1 KB each) go to LDS the same way, after
  // the token rows
  MLA_LDS char* wl = ol + kRowsBytes;
  const uint32_t wl_addr = ol_addr + kRowsBytes;
#pragma unroll
  for (int i = 0; i < 8 * VT; ++i) {
    const int r = wave + kProjWaves * i;
    dma16(w_uv + (static_cast<int64_t>(head) * d_v + v0 + r) * kDc + 8 * (lane ^ (r & 15)), wl_addr + r * 1024);
  }
  bf16x8_t bw[VT][8];
  bf16x8_t oa[MT][8];
  // copies of the pass's token rows: wave w moves rows w, w + 4, ...
  auto copy_rows = [&](int m0) {
#pragma unroll
    for (int i = 0; i < 8 * MT; ++i) {
      const int r = wave + kProjWaves * i;
      const int n = min(m0 + r, n_tokens - 1);
      dma16(o_lat + (static_cast<int64_t>(n) * n_h + head) * kDc + 8 * (lane ^ (r & 15)), ol_addr + r * 1024);
    }
  };
  auto read_rows = [&]() {
    wait_vmcnt<0>();
    __syncthreads();  // every wave's rows (and weight loads) have landed
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = 32 * mt + l32;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        oa[mt][j] = *reinterpret_cast<MLA_LDS const bf16x8_t*>(ol + r * 1024 + 16 * ((16 * wave + 2 * j + hf) ^ (r & 15)));
    }
  };
  auto read_weights = [&]() {
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      const int r = 32 * vt + l32;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        bw[vt][j] = *reinterpret_cast<MLA_LDS const bf16x8_t*>(wl + r * 1024 + 16 * ((16 * wave + 2 * j + hf) ^ (r & 15)));
    }
  };
  copy_rows(0);
  read_rows();
  read_weights();
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
    __syncthreads();  // every wave has read its rows: the area takes the reduction
    // registers 4q..4q+3 of each lane as one 16-byte quad, quads of one q
    // contiguous over the lanes (conflict-free stores and loads)
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          red[wave][vt][mt][q][lane] = f32x4_t{acc[vt][mt][4 * q], acc[vt][mt][4 * q + 1], acc[vt][mt][4 * q + 2],
                                               acc[vt][mt][4 * q + 3]};
    __syncthreads();
    // thread t sums registers 4*(t/64) .. +3 of lane t%64 over the 4 waves
    const int rl = threadIdx.x & 63, rq = threadIdx.x >> 6;
    for (int mt = 0; mt < mts; ++mt)
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        f32x4_t v = red[0][vt][mt][rq][rl];
#pragma unroll
        for (int wv = 1; wv < kProjWaves; ++wv) v += red[wv][vt][mt][rq][rl];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * rq + i;
          const int n = m0 + 32 * mt + 8 * (r >> 2) + 4 * (rl >> 5) + (r & 3);
          if (n < n_tokens)
            out[(static_cast<int64_t>(n) * n_h + head) * d_v + v0 + 32 * vt + (rl & 31)] = f32_to_bf16(v[i]);
        }
      }
    m0 += 32 * MT;
    if (m0 >= n_tokens) break;
    __syncthreads();  // the reduction is read: the area takes the next rows
    copy_rows(m0);
    read_rows();
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
constexpr int kAppendMT = kAppendMTk;
constexpr int kAppendRT = kAppendRTk;  // 32-row tiles of W per append workgroup (a divisor of 576 / 32 = 18)
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

template <int D>
hipError_t launch_append_finish(const AppendArgs& a, const float* partial, int n_chunks, hipStream_t st) {
  auto finish = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(a.n_tokens), dim3(256), 0, st, partial, n_chunks, a.n_tokens, a.gamma,
                       a.positions, a.slots, a.cache_slots, a.eps, rope_table(a.theta), a.cache, a.cache_scale);
  };
  switch (a.cache_dtype) {
    case 2: finish(append_finish_kernel<D, kOutFp8>); break;
    case 3: finish(append_finish_kernel<D, kOutFp4>); break;
    case 4: finish(append_finish_kernel<D, kOutFp8Kr>); break;
    default: finish(append_finish_kernel<D, kOutBf16>); break;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_append_d(const AppendArgs& a, hipStream_t st) {
  const float* partial;
  int n_chunks;
  if (a.w != nullptr) {
    n_chunks = append_chunks(a.d_model);
    float* ws = static_cast<float*>(a.workspace);
    auto kern = append_proj_kernel<kAppendRT, kAppendMT, D>;
    hipLaunchKernelGGL(kern, dim3(D / (32 * kAppendRT), n_chunks, token_groups(a.n_tokens, kAppendMT)), dim3(256),
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
  return launch_append_finish<D>(a, partial, n_chunks, st);
}

hipError_t launch_append_mfma(const AppendArgs& a, hipStream_t st) {
  return a.d_r == 0 ? launch_append_d<kDc>(a, st) : launch_append_d<kD>(a, st);
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
  if (a.d_r == 0) {  // no RoPE part: rows of d_c, bf16
    auto kern = one ? absorb_q_kernel<false, 1, 0> : absorb_q_kernel<false, 2, 0>;
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, q_nope, q_pe, w_uk, a.positions, a.n_tokens, a.n_h,
                       rope_table(a.theta), a.q_lat);
  } else if (a.cache_dtype == 2) {
    auto kern = one ? absorb_q_kernel<true, 1, kDr> : absorb_q_kernel<true, 2, kDr>;
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, q_nope, q_pe, w_uk, a.positions, a.n_tokens, a.n_h,
                       rope_table(a.theta), a.workspace);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(quantize_rows_fp8_kernel, dim3(a.n_tokens * a.n_h), dim3(64), 0, st,
                       static_cast<const float*>(a.workspace), static_cast<uint8_t*>(a.q_lat),
                       a.q_scale);
  } else {
    auto kern = one ? absorb_q_kernel<false, 1, kDr> : absorb_q_kernel<false, 2, kDr>;
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, q_nope, q_pe, w_uk, a.positions, a.n_tokens, a.n_h,
                       rope_table(a.theta), a.q_lat);
  }
  return hipGetLastError();
}

// The down-projection of the append and the latent query in one launch,
// then the append's finish (and, for an fp8 cache, the query's quantisation).
template <int D, int DR>
hipError_t launch_append_absorb_d(const AppendArgs& a, const AbsorbArgs& q, hipStream_t st) {
  const int n_chunks = append_chunks(a.d_model);
  AppendAbsorbArgs g;
  g.h = static_cast<const __bf16*>(a.hidden);
  g.w = static_cast<const __bf16*>(a.w);
  g.n_tokens = a.n_tokens;
  g.d_model = a.d_model;
  g.chunk_len = a.d_model / n_chunks;
  g.partial = static_cast<float*>(a.workspace);
  g.ax = D / (32 * kAppendRT);
  g.ay = n_chunks;
  g.az = token_groups(a.n_tokens, kAppendMT);
  g.q_nope = static_cast<const __bf16*>(q.q_nope);
  g.q_pe = static_cast<const __bf16*>(q.q_pe);
  g.w_uk = static_cast<const __bf16*>(q.w_uk);
  g.positions = q.positions;
  g.n_q = q.n_tokens;
  g.n_h = q.n_h;
  const bool fp8 = q.cache_dtype == 2;
  g.q_out = fp8 ? q.workspace : q.q_lat;
  const dim3 grid(g.ax * g.ay * g.az + q.n_h * (kDc / 128));
  const RopeTable64 rope = rope_table(q.theta);
  // one token tile per absorb pass: the fused kernel then needs 136 rather
  // than 232 registers per lane, and three workgroups fit a CU instead of two
  // (measured 2-3 us less per V3 bs64 step than two tiles per pass)
  if (fp8)
    hipLaunchKernelGGL((append_absorb_kernel<D, true, 1, DR>), grid, dim3(256), 0, st, g, rope);
  else
    hipLaunchKernelGGL((append_absorb_kernel<D, false, 1, DR>), grid, dim3(256), 0, st, g, rope);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_append_finish<D>(a, g.partial, n_chunks, st);
  if (e != hipSuccess || !fp8) return e;
  hipLaunchKernelGGL(quantize_rows_fp8_kernel, dim3(q.n_tokens * q.n_h), dim3(64), 0, st,
                     static_cast<const float*>(q.workspace), static_cast<uint8_t*>(q.q_lat), q.q_scale);
  return hipGetLastError();
}

hipError_t launch_append_absorb_mfma(const AppendArgs& a, const AbsorbArgs& q, hipStream_t st) {
  return a.d_r == 0 ? launch_append_absorb_d<kDc, 0>(a, q, st) : launch_append_absorb_d<kD, kDr>(a, q, st);
}

hipError_t launch_out_proj_mfma(const OutProjArgs& a, hipStream_t st) {
  constexpr int VT = kOutVT;
  auto kern = out_proj_kernel<VT, 1>;  // 32 KB of token rows + 32 KB of weights: two workgroups per CU
  hipLaunchKernelGGL(kern, dim3(a.n_h, a.d_v / (32 * VT)), dim3(256), 0, st,
                     static_cast<const __bf16*>(a.o_lat), static_cast<const __bf16*>(a.w_uv),
                     a.n_tokens, a.n_h, a.d_v, static_cast<__bf16*>(a.out));
  return hipGetLastError();
}

}  // namespace mla
