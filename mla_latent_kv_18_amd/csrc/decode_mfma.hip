// Latent-cache decode for MI355X (gfx950): absorbed MLA attention as an
// MQA with one shared 576-wide key row per token whose first 512 elements
// are also the value ([MLA explainer, trade-offs section]).
//
// Work decomposition
//   workgroup = (request b, context chunk, row group); rows of a request are
//   (query t, head h) pairs, r = t * n_h + h.  Each 64-lane wave owns 32
//   consecutive rows (one query position, 32 heads) for the whole chunk.
//   A workgroup of WAVES waves owns 32*WAVES rows and streams its chunk of
//   cache rows through LDS once; every wave reuses each staged tile.
//
// Per 32-token tile, per wave (bf16 MFMA 32x32x16, fp32 accumulate):
//   S^T[t, h]  = sum_d K[t, d] Q[h, d]      A = K tile from LDS (ds_read_b128),
//                                           B = Q^T, register resident (144 VGPR)
//   online softmax over t (per lane: one head, 16 tokens; the other 16 tokens
//   of that head sit in lane ^ 32)
//   O^T[c, h] += sum_t V^T[c, t] P^T[t, h]  A = V^T read with ds_read_b64_tr_b16
//                                           from the same LDS tile, B = P^T taken
//                                           straight from the S^T registers
// The token order inside each 16-token MFMA k-step is permuted identically on
// both operands so P never leaves registers.
//
// LDS tile: 32 rows x 72 sixteen-byte chunks, chunk c of row t stored at
// t*72 + (c ^ f(t)), f(t) = u ^ ((u & 1) << 2), u = (t >> 1) & 7; this keeps
// both the 16-lane b128 key reads and the 32-lane transposed value reads free
// of bank conflicts.  Tiles arrive by direct global->LDS 16-byte loads
// (global_load_lds_dwordx4), NBUF tiles in flight.
#include <type_traits>

#include "decode_unit.h"
#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"
#include "merge_row.h"

namespace mla {
namespace {

constexpr int kDc = 512;
constexpr int kD = 576;
constexpr int kTileT = 32;
constexpr int kChunks = kD * 2 / 16;                 // 72
constexpr int kTileBytes = kTileT * kD * 2;          // 36864
constexpr int kLoadsPerTile = kTileBytes / (64 * 16);  // 36 wave-wide 16-byte loads

struct DecodeParams {
  const __bf16* q_lat;
  const __bf16* cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  __bf16* o_part;
  float* lse_part;
  __bf16* o_lat;
  float* lse;
  int max_blocks, num_blocks, block_size, q_len, n_h, max_seq_len;
  int split_tokens, num_splits, row_groups;
  int xcd_group;  // 1: the workgroups of one request share an XCD (see xcd_slot)
  float scale_log2;
  const int32_t* items;  // planned launch list, or null for the uniform split
  const float* cache_scale;  // e4m3 latent rows: one fp32 scale per cache slot
};

__device__ __forceinline__ int swz(int t) {
  const int u = (t >> 1) & 7;
  return u ^ ((u & 1) << 2);
}

template <int WAVES>
__device__ __forceinline__ void load_tile(const __bf16* rows, int valid_rows, uint32_t buf, int wave,
                                          int lane) {
#pragma unroll
  for (int ii = 0; ii < kLoadsPerTile / WAVES; ++ii) {
    const int i = wave + ii * WAVES;
    const int slot = 64 * i + lane;
    const int t = slot / kChunks;
    const int c = (slot - t * kChunks) ^ swz(t);
    const int tr = t < valid_rows ? t : valid_rows - 1;  // rows past the end: repeat a valid row
    const char* g = reinterpret_cast<const char*>(rows) + static_cast<size_t>(tr) * (kD * 2) + c * 16;
    dma16(g, buf + i * 1024);
  }
}

template <int WAVES, int NBUF>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_bf16_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char tiles_raw[NBUF * kTileBytes];
  __shared__ int second_pass;
  MLA_LDS char* tiles = (MLA_LDS char*)tiles_raw;
  const uint32_t tiles_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tiles));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5;          // which 4-token half of each 8-token group
  DecodeUnit u;
  if (p.items != nullptr) {
    if (!unit_from_list(p.items, p.seq_lens, p.max_seq_len, blockIdx.x, u)) return;
  } else if (!unit_uniform(p.seq_lens, p.max_seq_len, p.split_tokens, p.num_splits, blockIdx.y,
                           blockIdx.x % p.row_groups, blockIdx.x / p.row_groups, u)) {
    return;  // empty chunk: the combine step skips it
  }
  const int b = u.b, rg = u.rg, T = u.T, j0 = u.j0, j1 = u.j1;
  const bool direct = u.part < 0;

  // block table and lengths are read through the scalar path (uniform per workgroup)
  const MLA_CONST int32_t* block_table = (const MLA_CONST int32_t*)(p.block_table);
  const int n_tiles = j1 > j0 ? (j1 - j0 + kTileT - 1) / kTileT : 0;

  const int rows_per_req = p.q_len * p.n_h;
  const int row0 = rg * (32 * WAVES) + wave * 32;  // first row of this wave
  const int t_q = row0 / p.n_h;                     // query index of this wave
  const int h0 = row0 % p.n_h;
  const int n_tok = b * p.q_len + t_q;
  const int vis_end = T - p.q_len + t_q + 1;         // keys < vis_end are visible
  const int my_h = h0 + (lane & 31);
  if (threadIdx.x == 0) second_pass = 0;

  // latent query rows of this wave's heads, register resident: Q[h, 16s + 8hf .. +8]
  bf16x8_t qf[36];
  {
    const __bf16* qrow = p.q_lat + (static_cast<int64_t>(n_tok) * p.n_h + my_h) * kD + 8 * hf;
#pragma unroll
    for (int s = 0; s < 36; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * s);
    wait_vmcnt<0>();  // complete before the tile copies start counting
  }

  // per-lane LDS byte offsets (tile independent)
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
  auto issue_tile = [&](int k, int bi) {
    const int tok0 = j0 + k * kTileT;
    const int valid = min(kTileT, T - tok0);
    int blk = block_table[bt_row + tok0 / p.block_size];
    blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
    const __bf16* rows = p.cache + (static_cast<int64_t>(blk) * p.block_size + tok0 % p.block_size) * kD;
    load_tile<WAVES>(rows, valid, tiles_addr + bi * kTileBytes, wave, lane);
  };

  // Softmax reference point m_ref (log2 domain, per lane = per head).  It is
  // fixed at the first tile with a visible key and never moved inside the
  // loop, so the accumulators are only ever touched by MFMA there: P =
  // 2^(s - m_ref) may grow up to 2^kSlack (exact in fp32/bf16).  If some tile
  // exceeds m_ref + kSlack, the chunk is processed again with m_ref = the
  // exact chunk maximum found by the first pass (no third pass is needed).
  constexpr float kSlack = 64.f;
  f32x16_t oacc[16];
  float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f;

  auto run_pass = [&]() -> bool {
    bool flagged = false;
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) oacc[ct] = f32x16_t{};
    l_run = 0.f;
    // prologue: tiles 0 .. NBUF-2 in flight
#pragma unroll
    for (int k = 0; k < NBUF - 1; ++k)
      if (k < n_tiles) issue_tile(k, k);
    int bcur = 0;
    for (int k = 0; k < n_tiles; ++k) {
      if constexpr (NBUF >= 3) {
        if (k + 1 < n_tiles) wait_vmcnt<kLoadsPerTile / WAVES>();
        else wait_vmcnt<0>();
      } else {
        wait_vmcnt<0>();
      }
      __builtin_amdgcn_s_barrier();  // tile k visible to all; tile k-1 released by all
      if (k + NBUF - 1 < n_tiles) issue_tile(k + NBUF - 1, bcur == 0 ? NBUF - 1 : bcur - 1);
      MLA_LDS char* buf = tiles + bcur * kTileBytes;
      bcur = bcur == NBUF - 1 ? 0 : bcur + 1;

      // scores S^T for 32 tokens x 32 heads, key fragments prefetched 4 ahead
      f32x16_t sacc = f32x16_t{};
      bf16x8_t kf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kf[s] = *reinterpret_cast<MLA_LDS const bf16x8_t*>(buf + qk_off[s & 3] + (2 * s & ~7) * 16);
#pragma unroll
      for (int s = 0; s < 36; ++s) {
        const bf16x8_t cur = kf[s & 3];
        if (s + 4 < 36)
          kf[s & 3] = *reinterpret_cast<MLA_LDS const bf16x8_t*>(buf + qk_off[(s + 4) & 3] + (2 * (s + 4) & ~7) * 16);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[s], sacc, 0, 0, 0);
      }

      // softmax numerators; register r holds token 8(r/4) + 4hf + r%4
      const int tok_base = j0 + k * kTileT + 4 * hf;
      float sv[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = tok_base + 8 * (r >> 2) + (r & 3);
        sv[r] = tok < vis_end ? sacc[r] * p.scale_log2 : -INFINITY;
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
        pf[r >> 3][r & 7] = f32_to_bf16(pr);
      }
      l_run += psum;

      // O^T += V^T P^T over the tile's two 16-token k-steps
      i16x4_t vlo[2], vhi[2];
      auto vread = [&](int ks, int ct, int slot) {
        const int hi_off = (ct >> 1) * 128;
        vlo[slot] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<MLA_LDS i16x4_t*>(buf + pv_off[ks][0][ct & 1] + hi_off));
        vhi[slot] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
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
    }
    return flagged;
  };

  const bool flagged = run_pass();
  // workgroup-wide decision on the second pass
  if (__builtin_amdgcn_ballot_w64(flagged) != 0 && lane == 0) second_pass = 1;
  wait_vmcnt<0>();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  if (second_pass) {
    __builtin_amdgcn_s_barrier();
    m_ref = m_seen;
    run_pass();
  }

  // epilogue: normalise, write o (rows of this wave) and lse
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
  const int my_row = row0 + (lane & 31);
  if (direct) {
    __bf16* orow = p.o_lat + (static_cast<int64_t>(n_tok) * p.n_h + my_h) * kDc;
#pragma unroll
    for (int ct = 0; ct < 16; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4_t v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = f32_to_bf16(oacc[ct][4 * j + i] * inv);
        *reinterpret_cast<bf16x4_t*>(orow + 32 * ct + 8 * j + 4 * hf) = v;
      }
    if (p.lse != nullptr && hf == 0) p.lse[static_cast<int64_t>(n_tok) * p.n_h + my_h] = lse_v;
  } else {
    const int64_t pr = static_cast<int64_t>(u.part) * rows_per_req + my_row;
    __bf16* orow = p.o_part + pr * kDc;
#pragma unroll
    for (int ct = 0; ct < 16; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4_t v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = f32_to_bf16(oacc[ct][4 * j + i] * inv);
        *reinterpret_cast<bf16x4_t*>(orow + 32 * ct + 8 * j + 4 * hf) = v;
      }
    if (hf == 0) p.lse_part[pr] = lse_v;
  }
}

// Software-pipelined form of the kernel above for workgroups of four waves
// (128 rows, one query position).  Step k scores tile k+1, turns the scores
// into softmax numerators and adds tile k's weighted value rows, as one
// instruction stream per wave: two independent score chains and the
// weighted-sum MFMAs alternate so the matrix pipe never waits on a chain,
// the softmax VALU work runs between the last weighted-sum MFMAs, and the
// wave's nine tile copies are spread over the stream.  The weighted sum is
// split by latent columns: wave w accumulates O^T for columns
// 128w..128w+127 of all 128 heads, reading each transposed value fragment
// once and reusing it for four head groups; the numerators P^T of all heads
// go through LDS.  Per tile and CU this reads 184 KB of LDS (keys 147 KB,
// values 16 KB, P 24 KB with the writes) where per-head value reads would
// take 275 KB.  The streams are written out instruction by instruction
// (decode_bf16_asm.inc, generated by gen_decode_bf16_asm.py) because the
// register budget (Q: 144 VGPRs, O: 256 AGPRs, one wave per SIMD) leaves the
// compiler's scheduler no room for this overlap.  LDS: four tile buffers
// (tile k values, tile k+1 keys, tile k+2 landing, tile k+3 being copied)
// and two P^T buffers.  The softmax is that of the kernel above; the scores
// are summed in a different order (two chains), so results agree to fp32
// rounding of the scores rather than bit for bit.
// The same stream serves two more row formats (PipeFmt):
//   kPipeNope  512-wide bf16 rows (MLA without the decoupled RoPE part):
//              32 query fragments, 32 KB tiles, eight copies per wave;
//   kPipeFp4   576 E2M1 codes + 18 E8M0 block scales per row (320 bytes):
//              each wave copies its eight stored rows of tile k+4 into a
//              staging slot, and step k's stream expands its rows of tile
//              k+2 into the bf16 tile layout between the weighted-sum MFMAs
//              (E2M1 times a power of two is exact in bf16).  LDS: three tile
//              buffers, two P^T buffers, three staging slots.
//   kPipeFp8Kr 512 e4m3 latent codes with one power-of-two scale per row
//              (fp32, beside the pool) and a 64-wide bf16 RoPE key (640 bytes): each wave
//              copies the codes and scales of its eight rows of tile k+3 into
//              a staging slot, and its rows' RoPE keys straight into their
//              place in bf16 tile k+3 (that buffer still holds tile k, whose
//              keys were scored a step earlier; the weighted sum reads only
//              the latent columns).  Step k's stream expands its rows of tile
//              k+2 between the weighted-sum MFMAs (the row scale is a power
//              of two, so code * scale is exact in bf16).  LDS: three tile
//              buffers, two P^T buffers, two staging slots.
enum { kPipeBf16 = 0, kPipeNope = 1, kPipeFp4 = 2, kPipeFp8Kr = 3 };
constexpr int kPBytes = kTileT * 128 * 2;  // P^T of one tile, all heads, bf16

template <int PF>
struct PipeGeo {
  static constexpr int D = PF == kPipeNope ? 512 : 576;
  static constexpr int kNk = D / 16;                    // query fragments
  static constexpr int kChunks = D / 8;                 // 16-byte chunks of a tile row
  static constexpr int kTileBytes = kTileT * D * 2;
  static constexpr int kCopies = kTileBytes / 1024 / 4;  // direct copies per wave and tile
  static constexpr bool kExpand = PF == kPipeFp4;
  static constexpr bool kFp8 = PF == kPipeFp8Kr;
  static constexpr bool kStaged = kExpand || kFp8;
  // stored bytes per cache row
  static constexpr int kRowBytes = kExpand ? 320 : (kFp8 ? 640 : D * 2);
  static constexpr int kBufs = kStaged ? 3 : 4;
  // a wave's staged rows: FP4 8 x 320 B (+ pad); FP8-KR 8 x 512 B of codes, then
  // 256 B whose first 32 hold the rows' scales
  static constexpr int kStageWave = kFp8 ? 4096 + 256 : 3072;
  static constexpr int kStageBytes = 4 * kStageWave;
  static constexpr int kSlots = kFp8 ? 2 : 3;
  static constexpr int kRawCopies = 3;
  static constexpr int kTiles = kBufs * kTileBytes;
  static constexpr int kLds = kTiles + 2 * kPBytes + (kStaged ? kSlots * kStageBytes : 0);
  static_assert(kLds <= 160 * 1024, "LDS");
  static_assert(4 * kTileBytes <= kLds, "query staging");
};

#define MLA_ASM_ACC                                                                          \
  [o0] "+a"(oacc[0]), [o1] "+a"(oacc[1]), [o2] "+a"(oacc[2]), [o3] "+a"(oacc[3]),            \
      [o4] "+a"(oacc[4]), [o5] "+a"(oacc[5]), [o6] "+a"(oacc[6]), [o7] "+a"(oacc[7]),        \
      [o8] "+a"(oacc[8]), [o9] "+a"(oacc[9]), [o10] "+a"(oacc[10]), [o11] "+a"(oacc[11]),    \
      [o12] "+a"(oacc[12]), [o13] "+a"(oacc[13]), [o14] "+a"(oacc[14]), [o15] "+a"(oacc[15])
#define MLA_ASM_Q32                                                                          \
  [q0] "v"(qf[0]), [q1] "v"(qf[1]), [q2] "v"(qf[2]), [q3] "v"(qf[3]), [q4] "v"(qf[4]),       \
      [q5] "v"(qf[5]), [q6] "v"(qf[6]), [q7] "v"(qf[7]), [q8] "v"(qf[8]), [q9] "v"(qf[9]),   \
      [q10] "v"(qf[10]), [q11] "v"(qf[11]), [q12] "v"(qf[12]), [q13] "v"(qf[13]),            \
      [q14] "v"(qf[14]), [q15] "v"(qf[15]), [q16] "v"(qf[16]), [q17] "v"(qf[17]),            \
      [q18] "v"(qf[18]), [q19] "v"(qf[19]), [q20] "v"(qf[20]), [q21] "v"(qf[21]),            \
      [q22] "v"(qf[22]), [q23] "v"(qf[23]), [q24] "v"(qf[24]), [q25] "v"(qf[25]),            \
      [q26] "v"(qf[26]), [q27] "v"(qf[27]), [q28] "v"(qf[28]), [q29] "v"(qf[29]),            \
      [q30] "v"(qf[30]), [q31] "v"(qf[31])
#define MLA_ASM_Q MLA_ASM_Q32, [q32] "v"(qf[32]), [q33] "v"(qf[33]), [q34] "v"(qf[34]), [q35] "v"(qf[35])
#define MLA_ASM_KEYS [ka0] "v"(ka[0]), [ka1] "v"(ka[1]), [ka2] "v"(ka[2]), [ka3] "v"(ka[3]), [bk] "s"(bk)
#define MLA_ASM_VALUES \
  [va0] "v"(va[0]), [va1] "v"(va[1]), [va2] "v"(va[2]), [va3] "v"(va[3]), [bv] "s"(bv), [bp] "s"(bp)
#define MLA_ASM_SOFTMAX_STATE [mref] "+v"(m_ref), [mseen] "+v"(m_seen), [lrun] "+v"(l_run), [exc] "+v"(excess)
#define MLA_ASM_SOFTMAX_IN [scale] "s"(p.scale_log2), [bpw] "s"(bpw), [vlim] "v"(vlim), [tok] "s"(tok), [pa] "v"(pa)
#define MLA_ASM_COPY                                                                     \
  [cb] "s"(cb), [cd] "s"(cd), [cl] "s"(cl), [k1152] "s"(G::D * 2), [c0] "v"(cpk[0]),          \
      [c1] "v"(cpk[1]), [c2] "v"(cpk[2]), [c3] "v"(cpk[3]), [c4] "v"(cpk[4])
#define MLA_ASM_EXPAND [xs] "s"(xs), [xt] "s"(xt), [xw] "s"(xw), [xtl0] "v"(xtl0), [xtl1] "v"(xtl1)
#define MLA_ASM_EXPAND8 [xs] "s"(xs), [xt] "s"(xt), [xw] "s"(xw)
#define MLA_ASM_SCRATCH MLA_BF16_ASM_SCRATCH, "memory", "m0", "scc", "vcc"

#include "decode_bf16_asm.inc"

// Workgroups are dispatched to the eight XCDs round-robin by linear id.
// Remap so that all gridDim.x workgroups of request b run on one XCD: they
// read the same latent query rows, which that XCD's L2 then fetches once.
// Requires gridDim.y (the batch) to be a multiple of 8.
__device__ __forceinline__ void xcd_slot(int& b, int& unit) {
  const int lin = blockIdx.x + gridDim.x * blockIdx.y;
  const int xcd = lin & 7, pos = lin >> 3;
  b = xcd + 8 * (pos / gridDim.x);
  unit = pos % gridDim.x;
}

// Eight E2M1 codes (element 2i in the low nibble of byte i) times 2^(e - 127).
__device__ __forceinline__ bf16x8_t fp4_word_to_bf16(uint32_t w, uint32_t e) {
  const float sc = __uint_as_float(e << 23);
  const bf16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
  const bf16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
  const bf16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
  const bf16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
  return bf16x8_t{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

template <int PF>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_pipe_kernel(DecodeParams p) {
  using G = PipeGeo<PF>;
  __shared__ __attribute__((aligned(1024))) char lds_raw[G::kLds];
  MLA_LDS char* tiles = (MLA_LDS char*)lds_raw;
  MLA_LDS char* pbuf = tiles + G::kTiles;
  const uint32_t tiles_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tiles));
  const uint32_t pbuf_addr = tiles_addr + G::kTiles;
  const uint32_t stage_addr = pbuf_addr + 2 * kPBytes;
  (void)pbuf;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5;
  DecodeUnit u;
  if (p.items != nullptr) {
    if (!unit_from_list(p.items, p.seq_lens, p.max_seq_len, blockIdx.x, u)) return;
  } else {
    int bu = blockIdx.y, unit = blockIdx.x;
    if (p.xcd_group) xcd_slot(bu, unit);
    if (!unit_uniform(p.seq_lens, p.max_seq_len, p.split_tokens, p.num_splits, bu, unit % p.row_groups,
                      unit / p.row_groups, u))
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

  // per-lane LDS byte offsets of the key fragments (chunk 2s + hf of row
  // tq, four offsets cycling with s) and of the transposed value fragments
  // of column tile 4*wave ([h2][column parity]; column tile 4*wave + j adds
  // (j >> 1) * 128 B and the second 16-token k-step 16 rows = 16 * D * 2 B)
  const int tq = lane & 31;
  const int fq = swz(tq);
  int ka[4], va[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) ka[q] = (tq * G::kChunks + (((2 * q) | hf) ^ fq)) * 16;
  {
    const int L = lane & 15, cg = (lane >> 4) & 1;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int row = 8 * h2 + 4 * hf + (L >> 2);
      const int f = swz(row);
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int x = 4 * par + 2 * cg + ((L & 3) >> 1);
        va[2 * h2 + par] = (row * G::kChunks + (x ^ f)) * 16 + 8 * (L & 1) + 256 * wave;
      }
    }
  }

  // Copy ii of this wave moves wave-wide load i = wave + 4*ii of a bf16
  // tile: lane -> (row t, swizzled 16-byte chunk c), packed as c*16 | t << 11
  // in the low (even ii) or high (odd ii) half of cpk[ii / 2].  The query
  // rows are copied this way in every format.
  uint32_t cpk[5] = {};
#pragma unroll
  for (int ii = 0; ii < G::kCopies; ++ii) {
    const int slot = 64 * (wave + 4 * ii) + lane;
    const int t = slot / G::kChunks;
    const int c = (slot - t * G::kChunks) ^ swz(t);
    cpk[ii / 2] |= (static_cast<uint32_t>(c * 16) | (static_cast<uint32_t>(t) << 11)) << (16 * (ii & 1));
  }
  const int64_t bt_row = static_cast<int64_t>(b) * p.max_blocks;
  // block-table entry of tile k, and the first stored cache row of tile k given it
  auto block_of = [&](int k) { return block_table[bt_row + (j0 + k * kTileT) / p.block_size]; };
  auto base_from = [&](int blk, int k) -> const char* {
    const int tok0 = j0 + k * kTileT;
    blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
    return reinterpret_cast<const char*>(p.cache) +
           (static_cast<int64_t>(blk) * p.block_size + tok0 % p.block_size) * G::kRowBytes;
  };
  auto tile_base = [&](int k) { return base_from(block_of(k), k); };
  auto last_row = [&](int k) { return min(kTileT, T - (j0 + k * kTileT)) - 1; };
  auto buf_addr = [&](int k) { return tiles_addr + (static_cast<uint32_t>(k) % G::kBufs) * G::kTileBytes; };
  auto pbuf_addr_of = [&](int k) { return pbuf_addr + (k & 1) * kPBytes; };
  // bf16 formats: the wave's copies of tile k straight into its tile buffer
  auto issue_tile = [&](int k) {
    const char* base = tile_base(k);
    const uint32_t last = static_cast<uint32_t>(last_row(k));
    const uint32_t dst = buf_addr(k);
#pragma unroll
    for (int ii = 0; ii < G::kCopies; ++ii) {
      const uint32_t pk = cpk[ii / 2] >> (16 * (ii & 1));
      const uint32_t t = min((pk >> 11) & 31u, last);  // rows past the end repeat a valid row
      dma16_sv(base, t * (G::D * 2) + (pk & 2047u), dst + (wave + 4 * ii) * 1024);
    }
  };
  // FP4: the wave's stored rows 8w..8w+7 of tile k (2560 bytes) into its
  // part of staging slot k % 3; byte offsets past them repeat the last chunk
  auto issue_raw_at = [&](const char* base, int k) {
    const int last = last_row(k);
    const uint32_t dst = stage_addr + (k % 3) * G::kStageBytes + wave * G::kStageWave;
#pragma unroll
    for (int i = 0; i < G::kRawCopies; ++i) {
      const int o = min(1024 * i + 16 * lane, 8 * 320 - 16);
      const int r = o / 320;
      const int t = min(8 * wave + r, last);
      dma16_sv(base, static_cast<uint32_t>(t * 320 + (o - 320 * r)), dst + 1024 * i);
    }
  };
  // FP4: expand the wave's rows of staged tile k into bf16 tile k (C++ form,
  // for the first two tiles of a pass; the step stream does the rest)
  auto expand_cpp = [&](int k) {
    MLA_LDS const char* sw = tiles + (stage_addr - tiles_addr) + (k % 3) * G::kStageBytes + wave * G::kStageWave;
    MLA_LDS char* tw = tiles + (static_cast<uint32_t>(k) % G::kBufs) * G::kTileBytes + 8 * wave * G::kChunks * 16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w = *reinterpret_cast<const MLA_LDS uint32_t*>(sw + 320 * j + 4 * lane);
      const uint32_t e = *reinterpret_cast<const MLA_LDS uint8_t*>(sw + 320 * j + 288 + (lane >> 2));
      *reinterpret_cast<MLA_LDS bf16x8_t*>(tw + j * 1152 + 16 * (lane ^ swz(8 * wave + j))) =
          fp4_word_to_bf16(w, e);
    }
    const int r = lane >> 3, c = 64 + (lane & 7);
    const uint32_t w = *reinterpret_cast<const MLA_LDS uint32_t*>(sw + 320 * r + 4 * c);
    const uint32_t e = *reinterpret_cast<const MLA_LDS uint8_t*>(sw + 320 * r + 288 + (c >> 2));
    *reinterpret_cast<MLA_LDS bf16x8_t*>(tw + r * 1152 + 16 * (c ^ swz(8 * wave + r))) = fp4_word_to_bf16(w, e);
  };
  // FP8-KR: first cache slot of tile k given its block-table entry
  auto slot_from = [&](int blk, int k) -> int64_t {
    const int tok0 = j0 + k * kTileT;
    blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
    return static_cast<int64_t>(blk) * p.block_size + tok0 % p.block_size;
  };
  // FP8-KR: the codes of the wave's rows 8w..8w+7 of tile k (4 KB: copy i
  // moves rows 2i, 2i+1) and their scales (lanes 0-7; the rest repeat them)
  // into its part of staging slot k % 2
  auto issue_stage8 = [&](int64_t slot0, int k) {
    const int last = last_row(k);
    const char* base = reinterpret_cast<const char*>(p.cache) + slot0 * G::kRowBytes;
    const uint32_t dst = stage_addr + (k & 1) * G::kStageBytes + wave * G::kStageWave;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = min(8 * wave + 2 * i + (lane >> 5), last);
      dma16_sv(base, static_cast<uint32_t>(t * G::kRowBytes + ((16 * lane) & 511)), dst + 1024 * i);
    }
    const int ts = min(8 * wave + (lane & 7), last);
    dma4_sv(p.cache_scale + slot0, static_cast<uint32_t>(4 * ts), dst + 4096);
  };
  // FP8-KR: the RoPE keys of the wave's rows of tile k (128 B each, already
  // bf16) straight into chunks 64..71 of their rows in bf16 tile k, one
  // eight-lane copy per row (position c holds chunk c ^ swz(row))
  auto issue_rope8 = [&](int64_t slot0, int k) {
    const int last = last_row(k);
    const char* base = reinterpret_cast<const char*>(p.cache) + slot0 * G::kRowBytes;
    const uint32_t dst = buf_addr(k);
    if (lane < 8) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int t = 8 * wave + jj;
        const int ts = min(t, last);
        dma16_sv(base, static_cast<uint32_t>(ts * G::kRowBytes + kDc + 16 * (lane ^ swz(t))),
                 dst + t * (G::D * 2) + 2 * kDc);
      }
    }
  };
  // FP8-KR: expand the wave's staged rows of tile k into bf16 tile k (C++
  // form, for the first two tiles of a pass; the step stream does the rest).
  // The conversion applies the row's power-of-two scale exactly.
  auto expand8_cpp = [&](int k) {
    MLA_LDS const char* sw = tiles + (stage_addr - tiles_addr) + (k & 1) * G::kStageBytes + wave * G::kStageWave;
    MLA_LDS char* tw = tiles + (static_cast<uint32_t>(k) % G::kBufs) * G::kTileBytes + 8 * wave * G::kChunks * 16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const i32x2_t c = *reinterpret_cast<MLA_LDS const i32x2_t*>(sw + 512 * j + 8 * lane);
      const float sc = *reinterpret_cast<MLA_LDS const float*>(sw + 4096 + 4 * j);
      const bf16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], sc, false);
      const bf16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], sc, true);
      const bf16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], sc, false);
      const bf16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], sc, true);
      *reinterpret_cast<MLA_LDS bf16x8_t*>(tw + j * 1152 + 16 * (lane ^ swz(8 * wave + j))) =
          bf16x8_t{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
    }
  };
  // FP4 stream inputs: the rows' last eight chunks (code word | scale byte <<
  // 16 in the staged rows; destination in the bf16 tile) and the swizzle term
  // 64 * (wave & 1) that the wave's rows share
  const uint32_t xtl0 = (320 * (lane >> 3) + 4 * (lane & 7)) | ((320 * (lane >> 3) + ((lane & 7) >> 2)) << 16);
  const uint32_t xtl1 = 1152 * (lane >> 3) + 16 * ((64 + (lane & 7)) ^ swz(8 * wave + (lane >> 3)));
  const uint32_t xw = 64 * (wave & 1);
  (void)xtl0;
  (void)xtl1;
  (void)xw;
  const uint32_t pa = 16 * lane;

  constexpr float kSlack = 64.f;
  f32x16_t oacc[16];
  float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f;
  float excess = -INFINITY;  // largest tile maximum minus m_ref seen in this pass
  // token t of tile k is visible iff 8(r/4) + r%4 < vlim - 32k (register r)
  const int vlim = vis_end - j0 - 4 * hf;

  // Latent queries.  The workgroup's 128 rows are contiguous in q_lat; they
  // are copied with whole-kilobyte loads into the first four tile-sized
  // areas of LDS (32 rows each, in the tile layout) and each wave then reads
  // its fragments with the key-fragment addressing.  Loading them straight
  // into registers would take one 32-byte piece from each of 32 rows per
  // load instruction.
  bf16x8_t qf[G::kNk];
  {
    const char* qblk =
        reinterpret_cast<const char*>(p.q_lat + (static_cast<int64_t>(b) * rows_per_req + rg * 128) * G::D);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const char* base = qblk + w * G::kTileBytes;
      const uint32_t dst = tiles_addr + w * G::kTileBytes;
#pragma unroll
      for (int ii = 0; ii < G::kCopies; ++ii) {
        const uint32_t pk = cpk[ii / 2] >> (16 * (ii & 1));
        dma16_sv(base, ((pk >> 11) & 31u) * (G::D * 2) + (pk & 2047u), dst + (wave + 4 * ii) * 1024);
      }
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    MLA_LDS const char* qb = tiles + wave * G::kTileBytes;
#pragma unroll
    for (int s = 0; s < G::kNk; ++s)
      qf[s] = *reinterpret_cast<MLA_LDS const bf16x8_t*>(qb + ka[s & 3] + 128 * (s >> 2));
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): fragments in registers
    __builtin_amdgcn_s_barrier();        // every wave done with the buffers
  }
  auto issue_first = [&]() {  // the first tiles of a pass
    if constexpr (G::kFp8) {
      // copy order: RoPE 0, staged 0, RoPE 1, staged 1, RoPE 2 (the waits
      // below count on it)
#pragma unroll
      for (int k = 0; k < 3; ++k)
        if (k < n_tiles) {
          const int64_t s0 = slot_from(block_of(k), k);
          issue_rope8(s0, k);
          if (k < 2) issue_stage8(s0, k);
        }
    } else if constexpr (G::kExpand) {
#pragma unroll
      for (int k = 0; k < 3; ++k)
        if (k < n_tiles) issue_raw_at(tile_base(k), k);
    } else {
      if (n_tiles > 0) issue_tile(0);
      if (n_tiles > 1) issue_tile(1);
      wait_vmcnt<0>();
    }
  };
  issue_first();

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  auto run_pass = [&]() -> bool {
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) oacc[ct] = f32x16_t{};
    l_run = 0.f;
    excess = -INFINITY;
    if (n_tiles == 0) return false;
    if constexpr (G::kFp8) {
      // each copy group: RoPE 8 copies, staged rows 5 copies
      if (n_tiles >= 3) wait_vmcnt<21>();  // staged 0 landed (RoPE 1, staged 1, RoPE 2 may not have)
      else if (n_tiles == 2) wait_vmcnt<13>();
      else wait_vmcnt<0>();
      expand8_cpp(0);
      if (n_tiles > 1) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): staging slot 0 read
        if (n_tiles > 2) {
          issue_stage8(slot_from(block_of(2), 2), 2);
          wait_vmcnt<13>();  // staged 1 landed (RoPE 2, staged 2 may not have)
        } else {
          wait_vmcnt<0>();
        }
        expand8_cpp(1);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    } else if constexpr (G::kExpand) {
      // staged tiles 0..2 are in flight; tiles 0 and 1 into bf16 buffers 0, 1
      if (n_tiles >= 3) wait_vmcnt<2 * G::kRawCopies>();
      else if (n_tiles == 2) wait_vmcnt<G::kRawCopies>();
      else wait_vmcnt<0>();
      expand_cpp(0);
      if (n_tiles > 1) {
        if (n_tiles >= 3) wait_vmcnt<G::kRawCopies>();
        else wait_vmcnt<0>();
        expand_cpp(1);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): staging slot 0 read
      if (n_tiles > 3) issue_raw_at(tile_base(3), 3);
    } else {
      if (n_tiles > 2) issue_tile(2);
    }
    __builtin_amdgcn_s_barrier();  // tiles 0 and 1 visible to all waves
    {  // scores and numerators of tile 0
      const uint32_t bk = buf_addr(0);
      const uint32_t bpw = pbuf_addr_of(0) + wave * 2048;
      const int tok = 0;
      if constexpr (PF == kPipeNope)
        asm volatile(MLA_NOPE_FIRST
                     : MLA_ASM_SOFTMAX_STATE
                     : MLA_ASM_Q32, MLA_ASM_KEYS, MLA_ASM_SOFTMAX_IN
                     : MLA_ASM_SCRATCH);
      else
        asm volatile(MLA_BF16_FIRST
                     : MLA_ASM_SOFTMAX_STATE
                     : MLA_ASM_Q, MLA_ASM_KEYS, MLA_ASM_SOFTMAX_IN
                     : MLA_ASM_SCRATCH);
    }
    int k = 0;
    if constexpr (G::kFp8) {
      // Step k expands tile k+2 (staged in step k-1, slot k % 2) and copies
      // the RoPE keys and staged rows of tile k+3.  Its scored tile k+1 is
      // not the chunk's last, so the stream skips the mask.  Copy sources
      // are looked up a step ahead.
      int64_t s_next = n_tiles > 3 ? slot_from(block_of(3), 3) : 0;
      int blk_next = n_tiles > 4 ? block_of(4) : 0;
      for (; k + 2 < n_tiles; ++k) {
        wait_vmcnt<18>();  // this wave's RoPE keys of tile k+1 (staged k+1, RoPE k+2, staged k+2 after them)
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): tile k+1 rows and P^T of tile k written
        __builtin_amdgcn_s_barrier();  // tile k+1 and P^T of tile k visible; tile k-1 released
        if (k + 3 < n_tiles) {
          issue_rope8(s_next, k + 3);
          issue_stage8(s_next, k + 3);
        } else {
          wait_vmcnt<0>();  // no copies behind tile k+2's staged rows for the stream's count
        }
        const uint32_t bk = buf_addr(k + 1), bv = buf_addr(k), bp = pbuf_addr_of(k);
        const uint32_t bpw = pbuf_addr_of(k + 1) + wave * 2048;
        const uint32_t xs = stage_addr + (k & 1) * G::kStageBytes + wave * G::kStageWave;
        const uint32_t xt = buf_addr(k + 2) + 8 * wave * G::kChunks * 16;
        const uint32_t xw = 64 * (wave & 1);
        const int tok = 32 * (k + 1);
        asm volatile(MLA_FP8KR_STEP_EXPAND
                     : MLA_ASM_ACC, MLA_ASM_SOFTMAX_STATE
                     : MLA_ASM_Q, MLA_ASM_KEYS, MLA_ASM_VALUES, MLA_ASM_SOFTMAX_IN, MLA_ASM_EXPAND8
                     : MLA_ASM_SCRATCH);
        if (k + 4 < n_tiles) s_next = slot_from(blk_next, k + 4);
        if (k + 5 < n_tiles) blk_next = block_of(k + 5);
      }
    } else if constexpr (G::kExpand) {
      // Step k expands tile k+2 and copies the stored rows of tile k+4 (into
      // the staging slot that tile k+1 left in step k-1).  Its scored tile
      // k+1 is not the chunk's last, so with q_len <= 32 all of it is
      // visible and the stream skips the mask.  Copy sources are looked up
      // a step ahead.
      const char* cb_next = n_tiles > 4 ? tile_base(4) : nullptr;
      int blk_next = n_tiles > 5 ? block_of(5) : 0;
      for (; k + 2 < n_tiles; ++k) {
        if (k + 3 < n_tiles) wait_vmcnt<G::kRawCopies>();  // this wave's stored rows of tile k+2
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's tile k+1 rows and P^T of tile k written
        __builtin_amdgcn_s_barrier();  // tile k+1 and P^T of tile k visible; tile k-1 released
        if (k + 4 < n_tiles) issue_raw_at(cb_next, k + 4);
        const uint32_t bk = buf_addr(k + 1), bv = buf_addr(k), bp = pbuf_addr_of(k);
        const uint32_t bpw = pbuf_addr_of(k + 1) + wave * 2048;
        const uint32_t xs = stage_addr + ((k + 2) % 3) * G::kStageBytes + wave * G::kStageWave;
        const uint32_t xt = buf_addr(k + 2) + 8 * wave * G::kChunks * 16;
        const int tok = 32 * (k + 1);
        asm volatile(MLA_FP4_STEP_EXPAND
                     : MLA_ASM_ACC, MLA_ASM_SOFTMAX_STATE
                     : MLA_ASM_Q, MLA_ASM_KEYS, MLA_ASM_VALUES, MLA_ASM_SOFTMAX_IN, MLA_ASM_EXPAND
                     : MLA_ASM_SCRATCH);
        if (k + 5 < n_tiles) cb_next = base_from(blk_next, k + 5);
        if (k + 6 < n_tiles) blk_next = block_of(k + 6);
      }
    } else {
      // Steps that also copy tile k+3.  Their scored tile k+1 ends at least 32
      // tokens before the sequence end, so with q_len <= 32 all of it is
      // visible and the stream skips the mask.
      // Copy sources are looked up ahead: the block-table entry of tile k+5 is
      // read in step k and turned into an address in step k+1, so no step
      // waits for a table read.
      const char* cb_next = n_tiles > 3 ? tile_base(3) : nullptr;
      int blk_next = n_tiles > 4 ? block_of(4) : 0;
      for (; k + 3 < n_tiles; ++k) {
        const char* cb = cb_next;
        wait_vmcnt<G::kCopies>();
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's P^T of tile k written
        __builtin_amdgcn_s_barrier();  // tile k+1 and P^T of tile k visible; tile k-1 released
        const int cl = last_row(k + 3);
        const uint32_t cd = buf_addr(k + 3) + wave * 1024;
        const uint32_t bk = buf_addr(k + 1), bv = buf_addr(k), bp = pbuf_addr_of(k);
        const uint32_t bpw = pbuf_addr_of(k + 1) + wave * 2048;
        const int tok = 32 * (k + 1);
        if constexpr (PF == kPipeNope)
          asm volatile(MLA_NOPE_STEP_COPY
                       : MLA_ASM_ACC, MLA_ASM_SOFTMAX_STATE
                       : MLA_ASM_Q32, MLA_ASM_KEYS, MLA_ASM_VALUES, MLA_ASM_SOFTMAX_IN, MLA_ASM_COPY
                       : MLA_ASM_SCRATCH);
        else
          asm volatile(MLA_BF16_STEP_COPY
                       : MLA_ASM_ACC, MLA_ASM_SOFTMAX_STATE
                       : MLA_ASM_Q, MLA_ASM_KEYS, MLA_ASM_VALUES, MLA_ASM_SOFTMAX_IN, MLA_ASM_COPY
                       : MLA_ASM_SCRATCH);
        if (k + 4 < n_tiles) cb_next = base_from(blk_next, k + 4);
        if (k + 5 < n_tiles) blk_next = block_of(k + 5);
      }
    }
    for (; k + 1 < n_tiles; ++k) {
      if (!G::kStaged && k + 2 < n_tiles) wait_vmcnt<G::kCopies>();
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_s_barrier();
      const uint32_t bk = buf_addr(k + 1), bv = buf_addr(k), bp = pbuf_addr_of(k);
      const uint32_t bpw = pbuf_addr_of(k + 1) + wave * 2048;
      const int tok = 32 * (k + 1);
      if constexpr (PF == kPipeNope)
        asm volatile(MLA_NOPE_STEP_MASKED
                     : MLA_ASM_ACC, MLA_ASM_SOFTMAX_STATE
                     : MLA_ASM_Q32, MLA_ASM_KEYS, MLA_ASM_VALUES, MLA_ASM_SOFTMAX_IN
                     : MLA_ASM_SCRATCH);
      else
        asm volatile(MLA_BF16_STEP_MASKED
                     : MLA_ASM_ACC, MLA_ASM_SOFTMAX_STATE
                     : MLA_ASM_Q, MLA_ASM_KEYS, MLA_ASM_VALUES, MLA_ASM_SOFTMAX_IN
                     : MLA_ASM_SCRATCH);
    }
    {  // weighted sum of the last tile (its keys were scored in the last step)
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_s_barrier();  // P^T of the last tile visible
      const uint32_t bv = buf_addr(k), bp = pbuf_addr_of(k);
      if constexpr (PF == kPipeNope)
        asm volatile(MLA_NOPE_PV_ONLY : MLA_ASM_ACC : MLA_ASM_VALUES, [pa] "v"(pa) : MLA_ASM_SCRATCH);
      else
        asm volatile(MLA_BF16_PV_ONLY : MLA_ASM_ACC : MLA_ASM_VALUES, [pa] "v"(pa) : MLA_ASM_SCRATCH);
    }
    return excess > kSlack;
  };
#pragma clang diagnostic pop
  // Cross-wave words (second-pass flag, per-head 1/l) live in tile buffer 0,
  // which no wave reads once every wave has passed the barrier below.
  MLA_LDS int* xflag = reinterpret_cast<MLA_LDS int*>(tiles);
  MLA_LDS float* xinv = reinterpret_cast<MLA_LDS float*>(tiles) + 64;
  const bool flagged = run_pass();
  wait_vmcnt<0>();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
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
    issue_first();
    run_pass();
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
  }

  // the softmax wave of each head publishes 1/l; lse is written by it too
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
  if (hf == 0) xinv[wave * 32 + lane] = inv;
  const int my_row = row0 + (lane & 31);
  if (direct) {
    if (p.lse != nullptr && hf == 0) p.lse[static_cast<int64_t>(n_tok) * p.n_h + my_h] = lse_v;
  } else {
    const int64_t pr = static_cast<int64_t>(u.part) * rows_per_req + my_row;
    if (hf == 0) p.lse_part[pr] = lse_v;
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  // This wave holds O^T for columns 128*wave.. of head group g in oacc[4j + g].
  // The normalised rows are staged in LDS (32 KB per wave, 256 B per head,
  // 16-byte chunk c of head h at c ^ (h & 15)) and then stored as whole
  // 256-byte row segments, four heads per store instruction.
  MLA_LDS char* stage = tiles + 1024 + wave * 32768;  // clear of the exchange words
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float ginv = xinv[g * 32 + (lane & 31)];
    const int h = g * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16x4_t v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = f32_to_bf16(oacc[4 * j + g][4 * jj + i] * ginv);
        *reinterpret_cast<MLA_LDS bf16x4_t*>(stage + h * 256 + (((4 * j + jj) ^ (h & 15)) * 16) + 8 * hf) = v;
      }
  }
  const int hrow0 = rg * 128;  // first row (query t_q, head h0 of wave 0) of this row group
#pragma unroll 4
  for (int it = 0; it < 32; ++it) {
    const int h = 4 * it + (lane >> 4), c = lane & 15;
    const bf16x8_t v = *reinterpret_cast<MLA_LDS const bf16x8_t*>(stage + h * 256 + ((c ^ (h & 15)) * 16));
    const int row = hrow0 + h;
    __bf16* orow;
    if (direct) {
      orow = p.o_lat + (static_cast<int64_t>(b * p.q_len + row / p.n_h) * p.n_h + row % p.n_h) * kDc;
    } else {
      orow = p.o_part + (static_cast<int64_t>(u.part) * rows_per_req + row) * kDc;
    }
    *reinterpret_cast<bf16x8_t*>(orow + 128 * wave + 8 * c) = v;
  }
}

// Merge the chunk partials of one row (merge_row): one wave per (row,
// request).  The lse of the first 64 splits (one per lane) and the partial
// rows of the first 8 splits are requested together, before the request's
// length is known: slots of splits past that length hold stale workspace
// contents and are never used, so the common case costs one memory round
// trip.  With xcd_group the rows of request b run on XCD b % 8, where the
// pipelined kernel wrote the request's partials, so that their reads can hit
// that XCD's L2.
template <typename OutT>
__global__ void __launch_bounds__(64) combine_kernel(const __bf16* __restrict__ o_part,
                                                     const float* __restrict__ lse_part,
                                                     const int32_t* __restrict__ seq_lens,
                                                     const int32_t* __restrict__ part_ptr,
                                                     int num_splits, int split_tokens, int q_len,
                                                     int n_h, int max_seq_len, OutT* __restrict__ o_lat,
                                                     float* __restrict__ lse, int xcd_group) {
  int row = blockIdx.x, b = blockIdx.y;
  if (xcd_group) xcd_slot(b, row);  // the XCD whose L2 took the request's partials
  const int lane = threadIdx.x;
  const int rows = q_len * n_h;
  // Planned launch: the request's partial blocks are part_ptr[b] .. part_ptr[b+1]-1
  // (none: its one chunk wrote o_lat).  Uniform split: b * num_splits + s for
  // the chunks that start before the request's end.
  int64_t first = static_cast<int64_t>(b) * num_splits;
  int last = num_splits - 1, ns_planned = 0;
  if (part_ptr != nullptr) {
    const int p0 = part_ptr[b];
    ns_planned = part_ptr[b + 1] - p0;
    if (ns_planned <= 0) return;
    first = p0;
    last = ns_planned - 1;
  }
  const int64_t base = first * rows + row;
  auto part_of = [&](int s) {
    return *reinterpret_cast<const bf16x8_t*>(o_part + (base + static_cast<int64_t>(s) * rows) * kDc + lane * 8);
  };
  // Indices are clamped rather than branched on, so that every load issues
  // before the first wait.
  int T = seq_lens[b];
  const float lv = lse_part[base + static_cast<int64_t>(min(lane, last)) * rows];
  bf16x8_t x0[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x0[j] = part_of(min(j, last));
  T = T < 0 ? 0 : (T > max_seq_len ? max_seq_len : T);
  const int ns = part_ptr != nullptr ? ns_planned : (T + split_tokens - 1) / split_tokens;
  float acc[8];
  const float L = merge_row<8>(ns, lv, lse_part + base, rows, x0, part_of, acc);
  const int n = b * q_len + row / n_h, h = row % n_h;
  OutT* dst = o_lat + (static_cast<int64_t>(n) * n_h + h) * kDc + lane * 8;
  if constexpr (sizeof(OutT) == 2) {
    bf16x8_t v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = f32_to_bf16(acc[i]);
    *reinterpret_cast<bf16x8_t*>(dst) = v;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = acc[i];
  }
  if (lse != nullptr && lane == 0) lse[static_cast<int64_t>(n) * n_h + h] = L;
}

}  // namespace

int decode_waves_per_group(int n_h, int q_len) {
  const int rows = n_h * q_len;
  return rows % 128 == 0 ? 4 : 2;
}

size_t decode_mfma_workspace(int batch, int q_len, int n_h, int num_splits) {
  if (num_splits <= 1) return 0;
  const size_t rows = static_cast<size_t>(batch) * num_splits * q_len * n_h;
  return rows * kDc * sizeof(__bf16) + rows * sizeof(float);  // bf16 partials, fp32 lse
}

// Partial rows: bf16 [units, q_len * n_h, 512] at the start of a.workspace,
// then fp32 lse [units, q_len * n_h]; units = planned partial blocks, or
// batch * num_splits for the uniform split
// (0: every request has one chunk and no combine runs).
int64_t partial_units(const DecodeArgs& a) {
  if (a.items != nullptr) return a.num_partials;
  return a.num_splits > 1 ? static_cast<int64_t>(a.batch) * a.num_splits : 0;
}

namespace {

DecodeParams decode_params(const DecodeArgs& a) {
  DecodeParams p;
  p.q_lat = static_cast<const __bf16*>(a.q_lat);
  p.cache = static_cast<const __bf16*>(a.cache);
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
  p.cache_scale = a.cache_scale;
  const int waves = decode_waves_per_group(a.n_h, a.q_len);
  p.row_groups = a.q_len * a.n_h / (32 * waves);
  p.xcd_group = 0;
  return p;
}

}  // namespace

bool decode_pipe_supported(int n_h, int q_len) { return decode_waves_per_group(n_h, q_len) == 4 && q_len <= 32; }

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t st) {
  DecodeParams p = decode_params(a);
  const int waves = decode_waves_per_group(a.n_h, a.q_len);
  const bool pipe = decode_pipe_supported(a.n_h, a.q_len);
  p.xcd_group = a.items == nullptr && pipe && a.batch % 8 == 0;
  const dim3 grid = a.items != nullptr ? dim3(a.num_slots) : dim3(a.num_splits * p.row_groups, a.batch);
  if (a.items != nullptr && a.num_slots == 0) return hipSuccess;
  if (pipe)
    hipLaunchKernelGGL(decode_pipe_kernel<kPipeBf16>, grid, dim3(256), 0, st, p);
  else if (waves == 4)
    hipLaunchKernelGGL((decode_bf16_kernel<4, 3>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((decode_bf16_kernel<2, 2>), grid, dim3(128), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || partial_units(a) == 0) return e;
  return launch_combine(a, st, p.xcd_group != 0);
}

// The pipelined stream over the NoPE (512-wide bf16) and FP4 cache rows.
hipError_t launch_decode_pipe(const DecodeArgs& a, int fmt, hipStream_t st) {
  DecodeParams p = decode_params(a);
  p.xcd_group = a.items == nullptr && a.batch % 8 == 0;
  const dim3 grid = a.items != nullptr ? dim3(a.num_slots) : dim3(a.num_splits * p.row_groups, a.batch);
  if (a.items != nullptr && a.num_slots == 0) return hipSuccess;
  if (fmt == kDqFp4Mx)
    hipLaunchKernelGGL(decode_pipe_kernel<kPipeFp4>, grid, dim3(256), 0, st, p);
  else if (fmt == kDqFp8Kr)
    hipLaunchKernelGGL(decode_pipe_kernel<kPipeFp8Kr>, grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(decode_pipe_kernel<kPipeNope>, grid, dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || partial_units(a) == 0) return e;
  return launch_combine(a, st, p.xcd_group != 0);
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t st, bool xcd_group) {
  const int64_t rows = partial_units(a) * a.q_len * a.n_h;
  const __bf16* o_part = static_cast<const __bf16*>(a.workspace);
  const float* lse_part = reinterpret_cast<const float*>(o_part + rows * kDc);
  const dim3 cgrid(a.q_len * a.n_h, a.batch);
  hipLaunchKernelGGL((combine_kernel<__bf16>), cgrid, dim3(64), 0, st, o_part, lse_part, a.seq_lens,
                     a.items != nullptr ? a.part_ptr : nullptr, a.num_splits, a.split_tokens, a.q_len,
                     a.n_h, a.max_seq_len, static_cast<__bf16*>(a.o_lat), a.lse,
                     xcd_group && a.batch % 8 == 0 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace mla
