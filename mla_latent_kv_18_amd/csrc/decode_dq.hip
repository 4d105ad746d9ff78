// Latent-cache decode over compressed or narrower cache rows (the cache
// variants of the MLA wiki note's open questions: an FP4 latent cache, a
// separate precision for the RoPE key, and MLA without the decoupled RoPE
// part as Kimi Linear uses it).  Same method as decode_mfma.hip -- absorbed
// attention as an MQA whose value is the latent part of the shared key row
// [MLA explainer, trade-offs section; eq.(9)-(10), eq.(16)] -- with the rows
// expanded to bf16 inside LDS, so the scores and the weighted sum run on the
// bf16 MFMA path and the cache is read from HBM in its stored size.
//
// Row formats (one cache row per token, rows contiguous within a block):
//   FP4-MX   d_c + d_R = 576 E2M1 codes, two per byte (element 2i in the
//            low nibble), then 18 E8M0 scales (one per 32 elements, value
//            2^(b - 127)), then 14 bytes of padding: 320 B.
//   FP8-KR   512 e4m3 latent codes (one power-of-two scale per token, fp32,
//            in the scale array beside the pool) and the 64-wide RoPE key in
//            bf16: 640 B.
//   NoPE     d_R = 0: 512 bf16 latent values: 1024 B.
//
// This kernel serves the shapes the pipelined stream of decode_mfma.hip does
// not (64-row workgroups: 64 heads, or more than 32 query positions); the
// 128-row shapes of all three formats go there.
//
// Per 32-token tile: the stored rows arrive by direct global->LDS copies
// into a staging buffer (three slots), are expanded into a bf16 tile
// (the swizzled layout of decode_mfma.hip: chunk c of row t at t * D/8 +
// (c ^ f(t))), and every wave then scores its 32 heads against the tile
// (S^T = K Q^T, Q register resident), takes the softmax numerators with a
// fixed reference (a second pass with the exact chunk maximum when a later
// tile exceeds it by more than 2^64), and adds V^T P^T with V read
// transposed from the same tile.  NoPE rows are already bf16: they are
// copied straight into the swizzled tile (three tile buffers).
// E2M1 values times their power-of-two block scale are exact in bf16 (the
// conversion instructions apply the exponent of the scale operand).  e4m3
// codes are expanded unscaled (exact) and their per-token scale s_j is applied
// in fp32 where the method allows it: the latent part of a score is
// s_j (q . codes_j), scored apart from the bf16 RoPE part, and the weighted
// sum takes P_j s_j (one bf16 rounding, as for P itself).
#include "decode_unit.h"
#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace mla {
namespace {

constexpr int kTileT = 32;
constexpr int kDc = 512;

template <int FMT>
struct DqFmt;
template <>
struct DqFmt<kDqFp4Mx> {
  static constexpr int D = 576, kRowBytes = 320;
  static constexpr bool kDirect = false, kScale = false;
};
template <>
struct DqFmt<kDqFp8Kr> {
  static constexpr int D = 576, kRowBytes = 640;
  static constexpr bool kDirect = false, kScale = true;
};
template <>
struct DqFmt<kDqBf16Nope> {
  static constexpr int D = 512, kRowBytes = 1024;
  static constexpr bool kDirect = true, kScale = false;
};

struct DqParams {
  const __bf16* q_lat;  // [N, n_h, D] bf16
  const uint8_t* cache;
  const float* cache_scale;
  const int32_t* block_table;
  const int32_t* seq_lens;
  __bf16* o_part;
  float* lse_part;
  __bf16* o_lat;
  float* lse;
  int max_blocks, num_blocks, block_size, q_len, n_h, max_seq_len;
  int split_tokens, num_splits, row_groups;
  float scale_log2;
  const int32_t* items;
};

__device__ __forceinline__ int swz(int t) {
  const int u = (t >> 1) & 7;
  return u ^ ((u & 1) << 2);
}

// eight E2M1 codes (element 2i in the low nibble of byte i) times 2^(e - 127)
__device__ __forceinline__ bf16x8_t fp4_word_to_bf16(uint32_t w, uint32_t e) {
  const float sc = __uint_as_float(e << 23);
  const bf16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
  const bf16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
  const bf16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
  const bf16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
  return bf16x8_t{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// eight e4m3 codes, unscaled (exact in bf16)
__device__ __forceinline__ bf16x8_t fp8_pair_to_bf16(i32x2_t w) {
  const bf16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.f, false);
  const bf16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.f, true);
  const bf16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.f, false);
  const bf16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.f, true);
  return bf16x8_t{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

template <int FMT, int WAVES>
struct DqGeom {
  using F = DqFmt<FMT>;
  static constexpr int D = F::D;
  static constexpr int kChunks = D / 8;                          // 16-byte chunks of a bf16 row
  static constexpr int kTileBytes = kTileT * D * 2;              // expanded bf16 tile
  static constexpr int kRawBytes = kTileT * F::kRowBytes;        // stored rows of a tile
  static constexpr int kCopies = (kRawBytes / 1024 + WAVES - 1) / WAVES;  // 1 KB copies per wave
  static constexpr int kStageBytes = kCopies * WAVES * 1024 + 256;        // + token scales
  static constexpr int kNStage = 3;
  static constexpr int kNTile = F::kDirect ? 3 : 2;
  static constexpr int kLds = kNTile * kTileBytes + (F::kDirect ? 0 : kNStage * kStageBytes);
  static constexpr int kWaveCopies = F::kDirect ? kTileBytes / 1024 / WAVES : kCopies + (F::kScale ? 1 : 0);
};

template <int FMT, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_dq_kernel(DqParams p) {
  using G = DqGeom<FMT, WAVES>;
  using F = DqFmt<FMT>;
  constexpr int D = G::D, kChunks = G::kChunks, kKSteps = D / 16;
  __shared__ __attribute__((aligned(1024))) char lds_raw[G::kLds];
  __shared__ float token_scales_raw[2 * kTileT];  // per bf16 buffer (formats with a token scale)
  __shared__ int second_pass;
  MLA_LDS float* token_scales = (MLA_LDS float*)token_scales_raw;
  MLA_LDS char* lds = (MLA_LDS char*)lds_raw;
  const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;

  DecodeUnit u;
  if (p.items != nullptr) {
    if (!unit_from_list(p.items, p.seq_lens, p.max_seq_len, blockIdx.x, u)) return;
  } else if (!unit_uniform(p.seq_lens, p.max_seq_len, p.split_tokens, p.num_splits, blockIdx.y,
                           blockIdx.x % p.row_groups, blockIdx.x / p.row_groups, u)) {
    return;  // empty chunk: the combine step skips it
  }
  const int b = u.b, rg = u.rg, T = u.T, j0 = u.j0, j1 = u.j1;
  const bool direct = u.part < 0;
  const MLA_CONST int32_t* block_table = (const MLA_CONST int32_t*)(p.block_table);
  const int n_tiles = j1 > j0 ? (j1 - j0 + kTileT - 1) / kTileT : 0;

  const int rows_per_req = p.q_len * p.n_h;
  const int row0 = rg * (32 * WAVES) + wave * 32;
  const int t_q = row0 / p.n_h;
  const int h0 = row0 % p.n_h;
  const int n_tok = b * p.q_len + t_q;
  const int vis_end = T - p.q_len + t_q + 1;  // keys < vis_end are visible
  const int my_h = h0 + (lane & 31);
  if (tid == 0) second_pass = 0;

  // latent query rows of this wave's heads: Q[h, 16s + 8hf .. +8]
  bf16x8_t qf[kKSteps];
  {
    const __bf16* qrow = p.q_lat + (static_cast<int64_t>(n_tok) * p.n_h + my_h) * D + 8 * hf;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * s);
    wait_vmcnt<0>();  // complete before the tile copies start counting
  }

  const int tq = lane & 31;
  const int fq = swz(tq);
  int qk_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) qk_off[q] = (tq * kChunks + (((2 * q) | hf) ^ fq)) * 16;
  const int L = lane & 15, cg = (lane >> 4) & 1;
  int pv_off[2][2][2];  // [ks][h2][ct parity]
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int row = 16 * ks + 8 * h2 + 4 * hf + (L >> 2);
      const int f = swz(row);
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int x = 4 * par + 2 * cg + ((L & 3) >> 1);
        pv_off[ks][h2][par] = (row * kChunks + (x ^ f)) * 16 + 8 * (L & 1);
      }
    }

  const int64_t bt_row = static_cast<int64_t>(b) * p.max_blocks;
  // first stored row of tile k, and the number of its rows before the sequence end
  auto tile_row = [&](int k) -> int64_t {
    const int tok0 = j0 + k * kTileT;
    int blk = block_table[bt_row + tok0 / p.block_size];
    blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
    return static_cast<int64_t>(blk) * p.block_size + tok0 % p.block_size;
  };
  auto last_row = [&](int k) { return min(kTileT, T - (j0 + k * kTileT)) - 1; };

  // copies of tile k; rows past the sequence end repeat its last row
  auto issue = [&](int k, int slot) {
    const int64_t r0 = tile_row(k);
    const int lr = last_row(k);
    const char* base = reinterpret_cast<const char*>(p.cache) + r0 * F::kRowBytes;
    if constexpr (F::kDirect) {  // bf16 rows straight into the swizzled tile
      const uint32_t dst = lds_addr + slot * G::kTileBytes;
#pragma unroll
      for (int ii = 0; ii < G::kWaveCopies; ++ii) {
        const int i = wave + ii * WAVES, s = 64 * i + lane;
        const int t = s / kChunks, c = (s - t * kChunks) ^ swz(t);
        dma16(base + static_cast<int64_t>(min(t, lr)) * F::kRowBytes + c * 16, dst + i * 1024);
      }
    } else {  // stored rows, flat, into a staging buffer
      const uint32_t dst = lds_addr + G::kNTile * G::kTileBytes + slot * G::kStageBytes;
#pragma unroll
      for (int ii = 0; ii < G::kCopies; ++ii) {
        const int i = wave + ii * WAVES;
        int off = (64 * i + lane) * 16;
        off = min(off, G::kRawBytes - 16);  // the copy past the tile refills its last chunk
        const int t = off / F::kRowBytes, col = off - t * F::kRowBytes;
        dma16(base + static_cast<int64_t>(min(t, lr)) * F::kRowBytes + col, dst + i * 1024);
      }
      if constexpr (F::kScale) {  // every wave copies the 32 token scales (same bytes)
        const float* sc = p.cache_scale + r0 + min(lane & 31, lr);
        dma4(sc, dst + G::kCopies * WAVES * 1024);
      }
    }
  };

  // expand staging buffer `slot` into bf16 tile `dst`: chunk (t, c) = bf16
  // elements 8c .. 8c+7 of row t.  Wave w expands rows R w .. R w + R-1: for
  // each of them lane l does latent chunk l (one stored word or pair, one
  // 16-byte store), then the rows' last eight chunks (the RoPE part) go eight
  // lanes to a row.  Row offsets are compile-time immediates; only the
  // swizzle term changes per row, and it is wave-uniform.
  constexpr int R = kTileT / WAVES;
  const int wrow0 = R * wave;
  const int xl = lane << 4;
  int tail_src[R / 8], tail_dst[R / 8];  // per-lane offsets of the tail chunks
#pragma unroll
  for (int i = 0; i < R / 8; ++i) {
    const int r = 8 * i + (lane >> 3), c = kDc / 8 + (lane & 7);
    tail_src[i] = r * F::kRowBytes + (FMT == kDqFp4Mx ? 4 * c : kDc + 16 * (lane & 7));
    tail_dst[i] = (r * kChunks + (c ^ swz(wrow0 + r))) * 16;
  }
  auto expand = [&](int slot, int dst) {
    MLA_LDS const char* st = lds + G::kNTile * G::kTileBytes + slot * G::kStageBytes;
    MLA_LDS char* tile = lds + dst * G::kTileBytes;
    if (F::kScale && tid < kTileT)  // the tile's token scales move with it: the staging slot is refilled early
      token_scales[32 * dst + tid] = *reinterpret_cast<const MLA_LDS float*>(st + G::kCopies * WAVES * 1024 + 4 * tid);
    MLA_LDS const char* sw = st + wrow0 * F::kRowBytes;
    MLA_LDS char* tw = tile + wrow0 * kChunks * 16;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int f = swz(wrow0 + j) << 4;  // wave-uniform
      bf16x8_t v;
      if constexpr (FMT == kDqFp4Mx) {
        const uint32_t w = *reinterpret_cast<const MLA_LDS uint32_t*>(sw + j * F::kRowBytes + 4 * lane);
        const uint32_t e = *reinterpret_cast<const MLA_LDS uint8_t*>(sw + j * F::kRowBytes + D / 2 + (lane >> 2));
        v = fp4_word_to_bf16(w, e);
      } else {
        const i32x2_t w = *reinterpret_cast<const MLA_LDS i32x2_t*>(sw + j * F::kRowBytes + 8 * lane);
        v = fp8_pair_to_bf16(w);
      }
      *reinterpret_cast<MLA_LDS bf16x8_t*>(tw + j * kChunks * 16 + (xl ^ f)) = v;
    }
#pragma unroll
    for (int i = 0; i < R / 8; ++i) {
      bf16x8_t v;
      if constexpr (FMT == kDqFp4Mx) {
        const uint32_t w = *reinterpret_cast<const MLA_LDS uint32_t*>(sw + tail_src[i]);
        const uint32_t e = *reinterpret_cast<const MLA_LDS uint8_t*>(
            sw + (8 * i + (lane >> 3)) * F::kRowBytes + D / 2 + (kDc / 8 + (lane & 7)) / 4);
        v = fp4_word_to_bf16(w, e);
      } else {
        v = *reinterpret_cast<const MLA_LDS bf16x8_t*>(sw + tail_src[i]);
      }
      *reinterpret_cast<MLA_LDS bf16x8_t*>(tw + tail_dst[i]) = v;
    }
  };

  constexpr float kSlack = 64.f;  // log2 headroom of the fixed softmax reference
  f32x16_t oacc[16];
  float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f;

  // scores, softmax numerators and weighted sum of one expanded tile
  // token_scale: the tile's 32 per-token scales in LDS (formats with kScale)
  auto compute = [&](MLA_LDS char* buf, MLA_LDS const float* token_scale, int k, bool& flagged) {
    // scores: the latent part (k-steps < d_c / 16) and the RoPE part in
    // separate accumulators when the latent carries a per-token scale
    f32x16_t sacc = f32x16_t{}, racc = f32x16_t{};
    bf16x8_t kf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      kf[s] = *reinterpret_cast<MLA_LDS const bf16x8_t*>(buf + qk_off[s & 3] + (2 * s & ~7) * 16);
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      const bf16x8_t cur = kf[s & 3];
      if (s + 4 < kKSteps)
        kf[s & 3] = *reinterpret_cast<MLA_LDS const bf16x8_t*>(buf + qk_off[(s + 4) & 3] + (2 * (s + 4) & ~7) * 16);
      if (F::kScale && s >= kDc / 16)
        racc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[s], racc, 0, 0, 0);
      else
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[s], sacc, 0, 0, 0);
    }
    // register r holds token 8(r/4) + 4hf + r%4 of the tile
    const int tok_base = j0 + k * kTileT + 4 * hf;
    float ts[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) ts[r] = F::kScale ? token_scale[8 * (r >> 2) + 4 * hf + (r & 3)] : 1.f;
    float sv[16];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tok = tok_base + 8 * (r >> 2) + (r & 3);
      const float sc = F::kScale ? fmaf(sacc[r], ts[r], racc[r]) : sacc[r];
      sv[r] = tok < vis_end ? sc * p.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    m_seen = fmaxf(m_seen, mx);
    if (m_ref == -INFINITY) m_ref = mx;  // nothing accumulated yet for this head
    flagged |= mx > m_ref + kSlack;
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    bf16x8_t pf[2];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = __builtin_amdgcn_exp2f(sv[r] - m_use);
      psum += pr;
      pf[r >> 3][r & 7] = f32_to_bf16(F::kScale ? pr * ts[r] : pr);  // the value rows are unscaled codes
    }
    l_run += psum;
    i16x4_t vlo[2], vhi[2];
    auto vread = [&](int ks, int ct, int s2) {
      const int hi_off = (ct >> 1) * 128;
      vlo[s2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<MLA_LDS i16x4_t*>(buf + pv_off[ks][0][ct & 1] + hi_off));
      vhi[s2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<MLA_LDS i16x4_t*>(buf + pv_off[ks][1][ct & 1] + hi_off));
    };
    vread(0, 0, 0);
#pragma unroll
    for (int it = 0; it < 32; ++it) {
      const int ks = it >> 4, ct = it & 15;
      if (it + 1 < 32) vread((it + 1) >> 4, (it + 1) & 15, (it + 1) & 1);
      const bf16x8_t vf = __builtin_bit_cast(
          bf16x8_t, __builtin_shufflevector(vlo[it & 1], vhi[it & 1], 0, 1, 2, 3, 4, 5, 6, 7));
      oacc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], oacc[ct], 0, 0, 0);
    }
  };

  auto run_pass = [&]() -> bool {
    bool flagged = false;
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) oacc[ct] = f32x16_t{};
    l_run = 0.f;
    if constexpr (F::kDirect) {
      if (n_tiles > 0) issue(0, 0);
      if (n_tiles > 1) issue(1, 1);
      for (int k = 0; k < n_tiles; ++k) {
        if (k + 1 < n_tiles) wait_vmcnt<G::kWaveCopies>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();  // tile k visible to all; tile k-1 released by all
        if (k + 2 < n_tiles) issue(k + 2, (k + 2) % 3);
        compute(lds + (k % 3) * G::kTileBytes, nullptr, k, flagged);
      }
    } else {
      // Software pipelined by one tile: step k expands tile k+1 (VALU and
      // LDS work) in the same block as it scores and sums tile k (MFMA), so
      // the two can overlap.  Stored tile j sits in staging slot j % 3, its
      // expansion in bf16 buffer j & 1.
      if (n_tiles > 0) issue(0, 0);
      if (n_tiles > 1) issue(1, 1);
      if (n_tiles > 0) {
        if (n_tiles > 1) wait_vmcnt<G::kWaveCopies>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();  // stored tile 0 visible to all
        if (n_tiles > 2) issue(2, 2);
        expand(0, 0);
        __syncthreads();  // expanded tile 0 visible to all
      }
      for (int k = 0; k < n_tiles; ++k) {
        if (k + 1 < n_tiles) {
          if (k + 2 < n_tiles) wait_vmcnt<G::kWaveCopies>();
          else wait_vmcnt<0>();
          // stored tile k+1 visible to all; every wave is done expanding tile
          // k (its staging slot is free) and computing tile k-1 (its bf16
          // buffer is free for tile k+1)
          __builtin_amdgcn_s_barrier();
          if (k + 3 < n_tiles) issue(k + 3, k % 3);
          expand((k + 1) % 3, (k + 1) & 1);
        }
        compute(lds + (k & 1) * G::kTileBytes, token_scales + 32 * (k & 1), k, flagged);
        __syncthreads();  // expanded tile k+1 visible to all; tile k released
      }
    }
    return flagged;
  };

  const bool flagged = run_pass();
  if (__builtin_amdgcn_ballot_w64(flagged) != 0 && lane == 0) second_pass = 1;
  wait_vmcnt<0>();
  __syncthreads();
  if (second_pass) {
    __syncthreads();
    m_ref = m_seen;
    run_pass();
  }

  // epilogue: normalise, write o (rows of this wave) and lse
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
  const int my_row = row0 + (lane & 31);
  __bf16* orow;
  float* lrow;
  if (direct) {
    orow = p.o_lat + (static_cast<int64_t>(n_tok) * p.n_h + my_h) * kDc;
    lrow = p.lse != nullptr ? p.lse + static_cast<int64_t>(n_tok) * p.n_h + my_h : nullptr;
  } else {
    const int64_t pr = static_cast<int64_t>(u.part) * rows_per_req + my_row;
    orow = p.o_part + pr * kDc;
    lrow = p.lse_part + pr;
  }
#pragma unroll
  for (int ct = 0; ct < 16; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4_t v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = f32_to_bf16(oacc[ct][4 * j + i] * inv);
      *reinterpret_cast<bf16x4_t*>(orow + 32 * ct + 8 * j + 4 * hf) = v;
    }
  if (lrow != nullptr && hf == 0) *lrow = lse_v;
}

template <int FMT>
hipError_t launch_dq(const DqParams& p, dim3 grid, int waves, hipStream_t st) {
  if (waves == 4)
    hipLaunchKernelGGL((decode_dq_kernel<FMT, 4>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((decode_dq_kernel<FMT, 2>), grid, dim3(128), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_dq(const DecodeArgs& a, int fmt, hipStream_t st) {
  if (decode_pipe_supported(a.n_h, a.q_len)) return launch_decode_pipe(a, fmt, st);
  DqParams p;
  p.q_lat = static_cast<const __bf16*>(a.q_lat);
  p.cache = static_cast<const uint8_t*>(a.cache);
  p.cache_scale = a.cache_scale;
  p.block_table = a.block_table;
  p.seq_lens = a.seq_lens;
  const int64_t rows = partial_units(a) * a.q_len * a.n_h;
  p.o_part = static_cast<__bf16*>(a.workspace);
  p.lse_part = rows > 0 ? reinterpret_cast<float*>(p.o_part + rows * kDc) : nullptr;
  p.o_lat = static_cast<__bf16*>(a.o_lat);
  p.lse = a.lse;
  p.max_blocks = a.max_blocks;
  p.num_blocks = a.num_blocks;
  p.block_size = a.block_size;
  p.q_len = a.q_len;
  p.n_h = a.n_h;
  p.max_seq_len = a.max_seq_len;
  p.split_tokens = a.split_tokens;
  p.num_splits = a.num_splits;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.items = a.items;
  const int waves = decode_waves_per_group(a.n_h, a.q_len);
  p.row_groups = a.q_len * a.n_h / (32 * waves);
  if (a.items != nullptr && a.num_slots == 0) return hipSuccess;
  const dim3 grid = a.items != nullptr ? dim3(a.num_slots) : dim3(a.num_splits * p.row_groups, a.batch);
  hipError_t e;
  switch (fmt) {
    case kDqFp4Mx: e = launch_dq<kDqFp4Mx>(p, grid, waves, st); break;
    case kDqFp8Kr: e = launch_dq<kDqFp8Kr>(p, grid, waves, st); break;
    default: e = launch_dq<kDqBf16Nope>(p, grid, waves, st); break;
  }
  if (e != hipSuccess || rows == 0) return e;
  return launch_combine(a, st);
}

}  // namespace mla
