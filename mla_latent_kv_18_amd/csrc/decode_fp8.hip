// Latent-cache decode over an fp8 (OCP e4m3) cache on MI355X (gfx950).
//
// The cache row of a token is 576 e4m3 codes, [c^KV (512) ; k^R (64)], with
// one fp32 scale per token (stored value = code * scale).  The latent query
// row is two planes of 576 codes with one fp32 scale per (token, head),
// q ~= qscale * (hi + lo / 16).  Scores and the latent-weighted sum both run
// on the fp8 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4), softmax and
// accumulation in fp32 ([MLA explainer, trade-offs section]: absorbed MLA is
// an MQA whose single shared key row is also the value).
//
// Precision: the cache operand is used exactly as stored.  The two operands
// that are computed here, the query and the softmax weights, each carry a
// second e4m3 term (the rounding residual, pre-multiplied by 16), applied by
// a second MFMA on the same LDS operand whose E8M0 scale carries the 1/16.
// One e4m3 term alone (3 mantissa bits) puts the error of short contexts
// above a few percent of the output; two terms give about 8 significant bits.
//
// Work decomposition as in the bf16 kernel: a workgroup of WAVES waves owns
// 32*WAVES rows (query t, head h) of one request and one context chunk;
// every wave owns 32 rows of one query position.  Tiles are 64 tokens (one
// K-step of the fp8 MFMA), 36864 bytes, staged once into LDS and read by
// every wave.
//
// Per tile, per wave:
//   S^T[t, h] = sum_d K[t, d] Q[h, d]   two 32-token blocks (beta), 9 K-steps
//                                        of 64 latent dims, hi and lo query
//                                        terms; the code products are scaled
//                                        afterwards by kscale[t] * qscale[h].
//   P[t, h]   = 2^(s - m_ref) in fp32; the value side needs P[t,h]*kscale[t],
//               which is split into hi + lo e4m3 terms with a power-of-two
//               block scale per (head, 32-token block): the block maximum maps
//               into [128, 256) and the MFMA's own E8M0 B-operand scale
//               multiplies it back, so the accumulators are only ever touched
//               by MFMA.
//   O^T[c, h] += sum_t V^T[c, t] P'^T[t, h]  A = V^T via ds_read_b64_tr_b8.
//
// Operand layouts (measured on gfx950): for the 32x32x64 fp8 MFMA, lane l
// supplies row (A) / column (B) l % 32 and 32 K-values; bytes 0..15 of lanes
// n and n + 32 form K-block 0 of row/column n (E8M0 scale from lane n),
// bytes 16..31 form K-block 1 (scale from lane n + 32).  Byte b of lane l is
// bound to token tau(l / 32, b) = 32(b >> 4) + 8((b >> 2) & 3) + 4(l / 32) +
// (b & 3), which is exactly where the S^T accumulator registers of the two
// 32-token blocks hold that token, so P goes from the score registers to the
// B operand without any lane exchange.
//
// LDS tile, chunk-major: 36 sixteen-byte chunks x 64 rows; chunk c of row t
// sits at position 64c + (t ^ 4(c & 1)).  Each wave-wide direct copy then
// moves one chunk column (lane = row, so one per-lane base address serves all
// copies of a wave), the 16-lane b128 key reads touch 16 consecutive
// positions, and the two 16-lane halves of a transposed value read land in
// disjoint banks.
#include "decode_unit.h"
#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace mla {
namespace {

constexpr int kDc = 512;
constexpr int kD = 576;                               // bytes per cache row
constexpr int kTileT = 64;
constexpr int kTileBytes = kTileT * kD;               // 36864
constexpr int kLoadsPerTile = kTileBytes / (64 * 16);  // 36 wave-wide 16-byte loads

struct Fp8Params {
  const uint8_t* q_lat;
  const float* q_scale;
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
  int xcd_pack;  // row groups of one chunk placed 8 workgroups apart (same XCD)
  float scale_log2;
  const int32_t* items;  // planned launch list, or null for the uniform split
};

// buffer layout: [tile 36864 B][per-wave token scales, 256 B each]
template <int WAVES>
constexpr int buf_bytes() {
  return kTileBytes + WAVES * 256;
}

template <int WAVES, int NBUF>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_fp8_kernel(Fp8Params p) {
  __shared__ __attribute__((aligned(1024))) char tiles_raw[NBUF * buf_bytes<WAVES>()];
  __shared__ int second_pass;
  MLA_LDS char* tiles = (MLA_LDS char*)tiles_raw;
  const uint32_t tiles_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tiles));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5;
  DecodeUnit u;
  if (p.items != nullptr) {
    if (!unit_from_list(p.items, p.seq_lens, p.max_seq_len, blockIdx.x, u)) return;
  } else {
    int split, rgu;
    if (p.xcd_pack) {
      const int x8 = blockIdx.x & 7, rest = blockIdx.x >> 3;
      rgu = rest % p.row_groups;
      split = (rest / p.row_groups) * 8 + x8;
    } else {
      rgu = blockIdx.x % p.row_groups;
      split = blockIdx.x / p.row_groups;
    }
    if (split >= p.num_splits) return;
    if (!unit_uniform(p.seq_lens, p.max_seq_len, p.split_tokens, p.num_splits, blockIdx.y, rgu, split, u))
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
  const int vis_end = T - p.q_len + t_q + 1;
  const int my_h = h0 + (lane & 31);
  if (threadIdx.x == 0) second_pass = 0;

  // latent query codes of this wave's heads: Q[h, 64s + 32hf .. +32]
  i32x8_t qf[9], ql[9];  // hi and lo planes
  float qmul;
  {
    const int64_t qrow = static_cast<int64_t>(n_tok) * p.n_h + my_h;
    const uint8_t* q = p.q_lat + qrow * (2 * kD) + 32 * hf;
#pragma unroll
    for (int s = 0; s < 9; ++s) {
      qf[s] = *reinterpret_cast<const i32x8_t*>(q + 64 * s);
      ql[s] = *reinterpret_cast<const i32x8_t*>(q + kD + 64 * s);
    }
    qmul = p.q_scale[qrow] * p.scale_log2;
    wait_vmcnt<0>();
  }

  // per-lane LDS byte offsets (tile independent)
  const int tq = lane & 31;
  int qk_off[2];  // chunk 4s + 2hf + x of row tq + 32 beta: + 4096 s + 512 beta
#pragma unroll
  for (int x = 0; x < 2; ++x) qk_off[x] = 16 * (64 * (2 * hf + x) + (tq ^ (4 * x)));
  const int cg = (lane >> 4) & 1, li = lane & 15, kp = li >> 1, pb = li & 1;
  const int pv_row = 8 * (kp >> 2) + 4 * hf + (kp & 3);
  // bytes 8pb.. of chunk 2ct + cg of row 16j + pv_row: + 2048 ct + 256 j
  const int pv_off = 16 * (64 * cg + (pv_row ^ (4 * cg))) + 8 * pb;
  const int sc_off = kTileBytes + wave * 256 + 16 * hf;
  // copy i moves chunk i of every row: lane -> row lane ^ 4(i & 1); i = wave + WAVES*ii
  // has the parity of the wave
  const int dma_row = lane ^ (4 * (wave & 1));

  const int64_t bt_row = static_cast<int64_t>(b) * p.max_blocks;
  auto issue_tile = [&](int k, int bi) {
    const int tok0 = j0 + k * kTileT;
    const int valid = min(kTileT, T - tok0);
    int blk = block_table[bt_row + tok0 / p.block_size];
    blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
    const int64_t first = static_cast<int64_t>(blk) * p.block_size + tok0 % p.block_size;
    const uint8_t* rows = p.cache + first * kD;
    const uint32_t base = tiles_addr + bi * buf_bytes<WAVES>();
    const uint8_t* src = rows + static_cast<size_t>(dma_row < valid ? dma_row : valid - 1) * kD + 16 * wave;
#pragma unroll
    for (int ii = 0; ii < kLoadsPerTile / WAVES; ++ii)  // rows past the end repeat a valid row
      dma16(src + 16 * WAVES * ii, base + (wave + WAVES * ii) * 1024);
    // this wave's private copy of the 64 token scales
    dma4(p.cache_scale + first + (lane < valid ? lane : valid - 1), base + kTileBytes + wave * 256);
  };
  constexpr int kWaveLoads = kLoadsPerTile / WAVES + 1;

  constexpr float kSlack = 64.f;
  f32x16_t oacc[16];
  float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f;

  auto run_pass = [&]() -> bool {
    bool flagged = false;
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) oacc[ct] = f32x16_t{};
    l_run = 0.f;
#pragma unroll
    for (int k = 0; k < NBUF - 1; ++k)
      if (k < n_tiles) issue_tile(k, k);
    int bcur = 0;
    for (int k = 0; k < n_tiles; ++k) {
      if constexpr (NBUF >= 3) {
        if (k + 1 < n_tiles) wait_vmcnt<kWaveLoads>();
        else wait_vmcnt<0>();
      } else {
        wait_vmcnt<0>();
      }
      __builtin_amdgcn_s_barrier();  // tile k visible to all; tile k-1 released by all
      if (k + NBUF - 1 < n_tiles) issue_tile(k + NBUF - 1, bcur == 0 ? NBUF - 1 : bcur - 1);
      MLA_LDS char* buf = tiles + bcur * buf_bytes<WAVES>();
      bcur = bcur == NBUF - 1 ? 0 : bcur + 1;

      // S^T for the tile's two 32-token blocks; per K-step the four MFMAs
      // alternate between the two accumulators (hi terms, then lo terms)
      f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
      auto kread = [&](int s, int beta, int x) {
        return *reinterpret_cast<MLA_LDS const i32x4_t*>(buf + qk_off[x] + 512 * beta + 4096 * s);
      };
      i32x4_t kf[2][4];  // [K-step parity][2 beta + x]
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[0][i] = kread(0, i >> 1, i & 1);
#pragma unroll
      for (int s = 0; s < 9; ++s) {
        const int cur = s & 1;
        if (s + 1 < 9) {
#pragma unroll
          for (int i = 0; i < 4; ++i) kf[cur ^ 1][i] = kread(s + 1, i >> 1, i & 1);
        }
        const i32x8_t a0 = __builtin_shufflevector(kf[cur][0], kf[cur][1], 0, 1, 2, 3, 4, 5, 6, 7);
        const i32x8_t a1 = __builtin_shufflevector(kf[cur][2], kf[cur][3], 0, 1, 2, 3, 4, 5, 6, 7);
        sacc[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, qf[s], sacc[0], 0, 0, 0, 127, 0, 127);
        sacc[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, qf[s], sacc[1], 0, 0, 0, 127, 0, 127);
        sacc[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, ql[s], sacc[0], 0, 0, 0, 127, 0, 123);
        sacc[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, ql[s], sacc[1], 0, 0, 0, 127, 0, 123);
      }

      // token scales: register r of block beta holds token 32beta + 8(r/4) + 4hf + r%4
      f32x4_t ks[2][4];
#pragma unroll
      for (int beta = 0; beta < 2; ++beta)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
          ks[beta][a4] = *reinterpret_cast<MLA_LDS const f32x4_t*>(buf + sc_off + 4 * (32 * beta + 8 * a4));

      const int tok_base = j0 + k * kTileT + 4 * hf;
      float sv[2][16];
      float mx = -INFINITY;
#pragma unroll
      for (int beta = 0; beta < 2; ++beta)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = tok_base + 32 * beta + 8 * (r >> 2) + (r & 3);
          sv[beta][r] = tok < vis_end ? sacc[beta][r] * ks[beta][r >> 2][r & 3] * qmul : -INFINITY;
          mx = fmaxf(mx, sv[beta][r]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      m_seen = fmaxf(m_seen, mx);
      if (m_ref == -INFINITY) m_ref = mx;
      flagged |= mx > m_ref + kSlack;
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      float psum = 0.f;
      float pmax[2] = {0.f, 0.f};
#pragma unroll
      for (int beta = 0; beta < 2; ++beta)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = __builtin_amdgcn_exp2f(sv[beta][r] - m_use);
          psum += pr;
          sv[beta][r] = pr * ks[beta][r >> 2][r & 3];  // value-side weight P * kscale
          pmax[beta] = fmaxf(pmax[beta], sv[beta][r]);
        }
      l_run += psum;
      // per (head, 32-token block) power-of-two scale: the block max lands in
      // [128, 256); hi = e4m3(x), lo = e4m3((x - hi) * 16) with x = P' / 2^e
      i32x8_t ph, pl;
      int my_scale = 127;
#pragma unroll
      for (int beta = 0; beta < 2; ++beta) {
        const float bm = fmaxf(pmax[beta], __shfl_xor(pmax[beta], 32));
        int e = static_cast<int>((__float_as_uint(bm) >> 23) & 0xff);
        e = e < 11 ? 11 : (e > 254 ? 254 : e);
        const float div = __uint_as_float(static_cast<uint32_t>(e - 7) << 23);     // 2^(e - 134)
        const float div_lo = __uint_as_float(static_cast<uint32_t>(e - 11) << 23);  // div / 16
        if (beta == hf) my_scale = e - 7;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float* x = &sv[beta][4 * w];
          v2i16_t h2 = {0, 0};
          h2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h2, x[0], x[1], div, false);
          h2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h2, x[2], x[3], div, true);
          const int hw = __builtin_bit_cast(int, h2);
          const f32x2_t b01 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
          const f32x2_t b23 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
          v2i16_t l2 = {0, 0};
          l2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l2, x[0] - b01[0] * div, x[1] - b01[1] * div, div_lo, false);
          l2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l2, x[2] - b23[0] * div, x[3] - b23[1] * div, div_lo, true);
          ph[4 * beta + w] = hw;
          pl[4 * beta + w] = __builtin_bit_cast(int, l2);
        }
      }
      const int my_scale_lo = my_scale - 4;

      // O^T += V^T P'^T: 16 column tiles of 32 latent dims, one 64-token
      // K-step each, hi and lo terms; column tiles go in pairs so that the two
      // MFMAs on one accumulator are never back to back
      i32x2_t vr[4][4];
      auto vread = [&](int ct) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vr[ct & 3][j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<MLA_LDS i32x2_t*>(
              buf + pv_off + 2048 * ct + 256 * j));
      };
      auto vfrag = [&](int ct) {
        const i32x2_t* v = vr[ct & 3];
        return i32x8_t{v[0][0], v[0][1], v[1][0], v[1][1], v[2][0], v[2][1], v[3][0], v[3][1]};
      };
      vread(0);
      vread(1);
#pragma unroll
      for (int ct = 0; ct < 16; ct += 2) {
        if (ct + 2 < 16) {
          vread(ct + 2);
          vread(ct + 3);
        }
        const i32x8_t a0 = vfrag(ct), a1 = vfrag(ct + 1);
        oacc[ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, ph, oacc[ct], 0, 0, 0, 127, 0, my_scale);
        oacc[ct + 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, ph, oacc[ct + 1], 0, 0, 0, 127, 0, my_scale);
        oacc[ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, pl, oacc[ct], 0, 0, 0, 127, 0, my_scale_lo);
        oacc[ct + 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, pl, oacc[ct + 1], 0, 0, 0, 127, 0, my_scale_lo);
      }
    }
    return flagged;
  };

  const bool flagged = run_pass();
  if (__builtin_amdgcn_ballot_w64(flagged) != 0 && lane == 0) second_pass = 1;
  wait_vmcnt<0>();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  if (second_pass) {
    __builtin_amdgcn_s_barrier();
    m_ref = m_seen;
    run_pass();
  }

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

// Software-pipelined form for workgroups of four waves (128 rows of one
// query position), with q_len <= 32.  Step k of a wave is one instruction
// stream (decode_fp8_asm.inc, generated by gen_decode_fp8_asm.py): the 36
// score MFMAs of tile k+1 (two accumulators, hi and lo query terms) with the
// two-term encoding of tile k's value-side weights between them, then the 32
// weighted-sum MFMAs of tile k with the softmax of tile k+1 between them; the
// wave's nine copies of tile k+2 ride in the score phase.  The weights of a
// tile wait in a private LDS area of the wave from its softmax to its
// encoding in the next step.  Tiles use the 16-row-group layout described in
// the generator, so that each direct copy reads 16 rows x 64 contiguous bytes.
// LDS: three tile buffers (tile k values, tile k+1 keys, tile k+2 landing)
// and four 9 KB weight areas.
constexpr int kF8Bufs = 3;
constexpr int kF8BufBytes = kTileBytes + 256;  // tile + its 64 token scales
constexpr int kF8PBytes = 9216;                // P' (8 KB) + block maxima, per wave
constexpr int kF8Copies = kLoadsPerTile / 4;   // 9 per wave per tile

#include "decode_fp8_asm.inc"

#define MLA_F8_ACC                                                                           \
  [o0] "+a"(oacc[0]), [o1] "+a"(oacc[1]), [o2] "+a"(oacc[2]), [o3] "+a"(oacc[3]),            \
      [o4] "+a"(oacc[4]), [o5] "+a"(oacc[5]), [o6] "+a"(oacc[6]), [o7] "+a"(oacc[7]),        \
      [o8] "+a"(oacc[8]), [o9] "+a"(oacc[9]), [o10] "+a"(oacc[10]), [o11] "+a"(oacc[11]),    \
      [o12] "+a"(oacc[12]), [o13] "+a"(oacc[13]), [o14] "+a"(oacc[14]), [o15] "+a"(oacc[15])
#define MLA_F8_Q                                                                             \
  [qh0] "v"(qf[0]), [qh1] "v"(qf[1]), [qh2] "v"(qf[2]), [qh3] "v"(qf[3]), [qh4] "v"(qf[4]),  \
      [qh5] "v"(qf[5]), [qh6] "v"(qf[6]), [qh7] "v"(qf[7]), [qh8] "v"(qf[8]),                \
      [ql0] "v"(ql[0]), [ql1] "v"(ql[1]), [ql2] "v"(ql[2]), [ql3] "v"(ql[3]),                \
      [ql4] "v"(ql[4]), [ql5] "v"(ql[5]), [ql6] "v"(ql[6]), [ql7] "v"(ql[7]), [ql8] "v"(ql[8])
#define MLA_F8_KEYS [ka0] "v"(qk_off[0]), [ka1] "v"(qk_off[1]), [bk] "s"(bk)
#define MLA_F8_VALUES [vo] "v"(pv_off), [bv] "s"(bv)
#define MLA_F8_COMMON [pa] "v"(pa), [sw] "s"(sw)
#define MLA_F8_STATE [mref] "+v"(m_ref), [mseen] "+v"(m_seen), [lrun] "+v"(l_run), [exc] "+v"(excess)
#define MLA_F8_SOFTMAX_IN \
  [qmul] "v"(qmul), [vlim] "v"(vlim), [tok] "s"(tok), [bks] "s"(bk + kTileBytes), [domask] "s"(domask)
#define MLA_F8_COPY                                                                          \
  [cb] "s"(cb), [cd] "s"(cd), [cl] "s"(cl), [csb] "s"(csb), [csd] "s"(csd), [k576] "s"(kD),  \
      [rl] "v"(crow), [q16] "v"(ccol), [r0] "s"(cR[0]), [r1] "s"(cR[1]), [r2] "s"(cR[2]),    \
      [r3] "s"(cR[3]), [r4] "s"(cR[4]), [r5] "s"(cR[5]), [r6] "s"(cR[6]), [r7] "s"(cR[7]),   \
      [r8] "s"(cR[8]), [k0] "s"(cC[0]), [k1] "s"(cC[1]), [k2] "s"(cC[2]), [k3] "s"(cC[3]),   \
      [k4] "s"(cC[4]), [k5] "s"(cC[5]), [k6] "s"(cC[6]), [k7] "s"(cC[7]), [k8] "s"(cC[8]),    \
      [docopy] "s"(docopy)
#define MLA_F8_SCRATCH MLA_FP8_ASM_SCRATCH, "memory", "m0", "scc", "vcc"

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_fp8_pipe_kernel(Fp8Params p) {
  // tile buffers, then the waves' P' areas; at the start the first 144 KB
  // hold the waves' latent queries instead
  __shared__ __attribute__((aligned(1024))) char lds_raw[kF8Bufs * kF8BufBytes + 4 * kF8PBytes];
  static_assert(4 * kTileBytes <= kF8Bufs * kF8BufBytes + 4 * kF8PBytes, "query staging fits");
  MLA_LDS char* tiles = (MLA_LDS char*)lds_raw;
  const uint32_t tiles_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tiles));
  const uint32_t pbuf_addr = tiles_addr + kF8Bufs * kF8BufBytes;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5;
  DecodeUnit u;
  if (p.items != nullptr) {
    if (!unit_from_list(p.items, p.seq_lens, p.max_seq_len, blockIdx.x, u)) return;
  } else {
    int split, rgu;
    if (p.xcd_pack) {
      const int x8 = blockIdx.x & 7, rest = blockIdx.x >> 3;
      rgu = rest % p.row_groups;
      split = (rest / p.row_groups) * 8 + x8;
    } else {
      rgu = blockIdx.x % p.row_groups;
      split = blockIdx.x / p.row_groups;
    }
    if (split >= p.num_splits) return;
    if (!unit_uniform(p.seq_lens, p.max_seq_len, p.split_tokens, p.num_splits, blockIdx.y, rgu, split, u))
      return;  // empty chunk: the combine step skips it
  }
  const int b = u.b, rg = u.rg, T = u.T, j0 = u.j0, j1 = u.j1;
  const bool direct = u.part < 0;

  const MLA_CONST int32_t* block_table = (const MLA_CONST int32_t*)(p.block_table);
  const int n_tiles = j1 > j0 ? (j1 - j0 + kTileT - 1) / kTileT : 0;

  const int rows_per_req = p.q_len * p.n_h;
  const int row0 = rg * 128 + wave * 32;
  const int t_q = row0 / p.n_h;
  const int h0 = row0 % p.n_h;
  const int n_tok = b * p.q_len + t_q;
  const int vis_end = T - p.q_len + t_q + 1;
  const int my_h = h0 + (lane & 31);

  const int tq = lane & 31;
  // Latent query codes of this wave's heads: Q[h, 64s + 32hf .. +32] (hi and
  // lo planes).  The wave's 32 rows (1152 B each) are contiguous in q_lat;
  // they are copied with whole-kilobyte loads into a 36 KB slot of LDS, where
  // 16-byte chunk c of row r sits at chunk 72r + (c ^ (r & 6)): the two
  // chunks of a fragment stay adjacent and in order, and eight consecutive
  // rows land in distinct bank groups.  Loading them straight into registers
  // would take one 32-byte piece from each of 32 rows per load instruction.
  i32x8_t qf[9], ql[9];
  float qmul;
  {
    const int64_t qrow0 = static_cast<int64_t>(n_tok) * p.n_h + h0;
    const uint8_t* qsrc = p.q_lat + qrow0 * (2 * kD);
    const uint32_t slot = tiles_addr + wave * kTileBytes;
#pragma unroll
    for (int i = 0; i < kLoadsPerTile; ++i) {
      const int pos = 64 * i + lane, r = pos / 72, c = (pos % 72) ^ (r & 6);
      dma16_sv(qsrc, r * (2 * kD) + 16 * c, slot + 1024 * i);
    }
    // kept positive: the streams take the row maximum of S * kscale before scaling by it
    qmul = fmaxf(p.q_scale[qrow0 + tq] * p.scale_log2, 1.17549435e-38f);
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    MLA_LDS const char* qrow = tiles + wave * kTileBytes + 16 * (72 * tq);
    const int fr = tq & 6;
#pragma unroll
    for (int s = 0; s < 9; ++s) {
      const int c = 4 * s + 2 * hf;
      qf[s] = *reinterpret_cast<MLA_LDS const i32x8_t*>(qrow + 16 * (c ^ fr));
      ql[s] = *reinterpret_cast<MLA_LDS const i32x8_t*>(qrow + 16 * ((36 + c) ^ fr));
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): codes in registers
    __builtin_amdgcn_s_barrier();        // every wave done with its slot
  }

  // per-lane LDS byte offsets in the 16-row-group tile layout
  int qk_off[2];  // chunk 4s + 2hf + x of row tq + 32 beta: + 1024 s + 18432 beta
#pragma unroll
  for (int x = 0; x < 2; ++x) qk_off[x] = 16 * (576 * (tq >> 4) + 16 * (2 * hf + x) + ((tq & 15) ^ (4 * x)));
  const int cg = (lane >> 4) & 1, li = lane & 15, kp = li >> 1, pb = li & 1;
  const int pv_row = 8 * (kp >> 2) + 4 * hf + (kp & 3);
  const int pv_off = 16 * (16 * cg + (pv_row ^ (4 * cg))) + 8 * pb;  // + 512 ct + 9216 j
  const uint32_t pa = 16 * lane;
  const uint32_t sw = pbuf_addr + wave * kF8PBytes;

  // Copy ii of this wave fills slots 64i.. of a tile, i = wave + 4ii: row
  // cR[ii] + crow (16-row group i / 9, lane's row in it), byte column
  // cC[ii] + ccol (chunks 4(i % 9) + lane / 16).
  const uint32_t crow = (lane & 15) ^ (4 * ((lane >> 4) & 1));
  const uint32_t ccol = 16 * (lane >> 4);
  uint32_t cR[kF8Copies], cC[kF8Copies];
#pragma unroll
  for (int ii = 0; ii < kF8Copies; ++ii) {
    const int i = wave + 4 * ii;
    cR[ii] = 16 * (i / 9);
    cC[ii] = 64 * (i % 9);
  }
  const int64_t bt_row = static_cast<int64_t>(b) * p.max_blocks;
  // block-table entry of tile k, and the cache slot of tile k's first token given it
  auto block_of = [&](int k) { return block_table[bt_row + (j0 + k * kTileT) / p.block_size]; };
  auto row_from = [&](int blk, int k) -> int64_t {
    const int tok0 = j0 + k * kTileT;
    blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
    return static_cast<int64_t>(blk) * p.block_size + tok0 % p.block_size;
  };
  auto first_row = [&](int k) { return row_from(block_of(k), k); };
  auto last_row = [&](int k) { return min(kTileT, T - (j0 + k * kTileT)) - 1; };
  auto buf_addr = [&](int k) { return tiles_addr + (k % kF8Bufs) * kF8BufBytes; };
  auto issue_tile = [&](int k) {
    const int64_t first = first_row(k);
    const uint8_t* rows = p.cache + first * kD;
    const uint32_t last = static_cast<uint32_t>(last_row(k));
    const uint32_t dst = buf_addr(k);
#pragma unroll
    for (int ii = 0; ii < kF8Copies; ++ii)  // rows past the end repeat a valid row
      dma16_sv(rows, min(cR[ii] + crow, last) * kD + cC[ii] + ccol, dst + (wave + 4 * ii) * 1024);
    dma4(p.cache_scale + first + min(static_cast<uint32_t>(lane), last), dst + kTileBytes);
  };

  constexpr float kSlack = 64.f;
  f32x16_t oacc[16];
  float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f, excess = -INFINITY;
  const int vlim = vis_end - j0 - 4 * hf;  // token t of tile k visible iff t < vlim - 64k

  if (n_tiles > 0) issue_tile(0);
  if (n_tiles > 1) issue_tile(1);

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  auto run_pass = [&]() -> bool {
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) oacc[ct] = f32x16_t{};
    l_run = 0.f;
    excess = -INFINITY;
    if (n_tiles == 0) return false;
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // tiles 0 and 1 visible to all waves
    {
      const uint32_t bk = buf_addr(0);
      const int tok = 0, domask = 1;
      asm volatile(MLA_FP8_FIRST
                   : MLA_F8_STATE
                   : MLA_F8_Q, MLA_F8_KEYS, MLA_F8_COMMON, MLA_F8_SOFTMAX_IN
                   : MLA_F8_SCRATCH);
    }
    // Copy sources are looked up ahead: the block-table entry of tile k+4 is
    // read in step k and turned into a cache slot in step k+1, so no step
    // waits for a table read.
    int64_t first_next = n_tiles > 2 ? first_row(2) : 0;
    int blk_next = n_tiles > 3 ? block_of(3) : 0;
    for (int k = 0; k + 1 < n_tiles; ++k) {
      const int64_t first = first_next;
      // Tile k+1 landed and visible; tile k-1 released by all waves: every
      // LDS read of a shared buffer was waited for inside the streams, and
      // what may still be in flight are the wave's own P' writes.
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      const uint32_t bk = buf_addr(k + 1), bv = buf_addr(k);
      const int tok = kTileT * (k + 1);
      // Tile k+2 is copied while it exists.  The scored tile k+1 needs the
      // mask only near the chunk's end: a tile that ends 64 tokens before
      // the last one is visible in full for q_len <= 32.
      // The two guards are counts (zero = off) rather than booleans, so that
      // they stay scalar: a widened boolean lands in a vector register.
      const bool copying = k + 2 < n_tiles;
      const int docopy = max(n_tiles - k - 2, 0);
      const int domask = max(k + 4 - n_tiles, 0);
      const uint8_t* cb = p.cache + first * kD;
      const float* csb = p.cache_scale + first;
      const int cl = copying ? last_row(k + 2) : 0;
      const uint32_t cd = buf_addr(k + 2) + wave * 1024;
      const uint32_t csd = buf_addr(k + 2) + kTileBytes;
      asm volatile(MLA_FP8_STEP
                   : MLA_F8_ACC, MLA_F8_STATE
                   : MLA_F8_Q, MLA_F8_KEYS, MLA_F8_VALUES, MLA_F8_COMMON, MLA_F8_SOFTMAX_IN, MLA_F8_COPY
                   : MLA_F8_SCRATCH);
      if (k + 3 < n_tiles) first_next = row_from(blk_next, k + 3);
      if (k + 4 < n_tiles) blk_next = block_of(k + 4);
    }
    {  // encoding and weighted sum of the last tile (its weights are in this wave's area)
      const uint32_t bv = buf_addr(n_tiles - 1);
      asm volatile(MLA_FP8_LAST : MLA_F8_ACC : MLA_F8_VALUES, MLA_F8_COMMON : MLA_F8_SCRATCH);
    }
    return excess > kSlack;
  };
#pragma clang diagnostic pop

  // Second-pass flags live in tile buffer 0, free once every wave is past the barrier.
  MLA_LDS int* xflag = reinterpret_cast<MLA_LDS int*>(tiles);
  const bool flagged = run_pass();
  wait_vmcnt<0>();
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  {
    const int f = __builtin_amdgcn_ballot_w64(flagged) != 0;
    if (lane == 0) xflag[wave] = f;
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  const bool second_pass = (xflag[0] | xflag[1] | xflag[2] | xflag[3]) != 0;
  if (second_pass) {
    __builtin_amdgcn_s_barrier();  // every wave has read the flags
    m_ref = m_seen;
    if (n_tiles > 0) issue_tile(0);
    if (n_tiles > 1) issue_tile(1);
    run_pass();
  }

  // Epilogue.  Lane-derived values are recomputed here from an opaque lane
  // id rather than kept live across the tile loop, where every register
  // outside the streams' scratch range holds an operand.  The wave's 32
  // normalised rows are staged through LDS (16-byte chunk q of head h at
  // chunk q ^ (h & 15) of a 1 KB row) and stored as whole 1 KB rows.
  int lane_e;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
  const int he = lane_e & 31, hfe = lane_e >> 5;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();  // every wave is done with the tile buffers
  MLA_LDS char* stage = tiles + wave * kTileBytes;
#pragma unroll
  for (int ct = 0; ct < 16; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4_t v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = f32_to_bf16(oacc[ct][4 * j + i] * inv);
      *reinterpret_cast<MLA_LDS bf16x4_t*>(stage + he * 1024 + (((4 * ct + j) ^ (he & 15)) * 16) + 8 * hfe) = v;
    }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's rows staged
  int64_t row_base;                     // output row of head h0 (+ h for head h0 + h)
  if (direct) {
    row_base = static_cast<int64_t>(n_tok) * p.n_h + h0;
  } else {
    row_base = static_cast<int64_t>(u.part) * rows_per_req + row0;
  }
  __bf16* obase = direct ? p.o_lat : p.o_part;
#pragma unroll 4
  for (int h = 0; h < 32; ++h) {
    const bf16x8_t v = *reinterpret_cast<MLA_LDS const bf16x8_t*>(stage + h * 1024 + ((lane_e ^ (h & 15)) * 16));
    *reinterpret_cast<bf16x8_t*>(obase + (row_base + h) * kDc + 8 * lane_e) = v;
  }
  float* lbase = direct ? p.lse : p.lse_part;
  if (lbase != nullptr && hfe == 0) lbase[row_base + he] = lse_v;
}

}  // namespace

hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t st) {
  Fp8Params p;
  p.q_lat = static_cast<const uint8_t*>(a.q_lat);
  p.q_scale = a.q_scale;
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
  p.xcd_pack = a.items == nullptr && a.num_splits > 1 && p.row_groups > 1;
  const int grid_splits = p.xcd_pack ? (a.num_splits + 7) / 8 * 8 : a.num_splits;
  const dim3 grid = a.items != nullptr ? dim3(a.num_slots) : dim3(grid_splits * p.row_groups, a.batch);
  if (a.items != nullptr && a.num_slots == 0) return hipSuccess;
  if (waves == 4 && a.q_len <= 32)
    hipLaunchKernelGGL(decode_fp8_pipe_kernel, grid, dim3(256), 0, st, p);
  else if (waves == 4)
    hipLaunchKernelGGL((decode_fp8_kernel<4, 3>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((decode_fp8_kernel<2, 2>), grid, dim3(128), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || rows == 0) return e;
  return launch_combine(a, st);
}

}  // namespace mla
