// Prefill attention, the non-absorbed side of MLA: keys and values are
// materialised per head (k^C_i = W^UK_i c, v_i = W^UV_i c, by mla_linear
// over the latent rows) and each head runs causal attention with query and
// key width d_h + d_R = 192 and value width d_v = 128 [MLA explainer,
// decoupled RoPE eq.(14) (q and k of a head are [content ; RoPE part]) and
// eq.(16) (the score is the sum of both blocks); trade-offs section (the
// prompt is processed without absorption)].
//
// Sequences: sequence s has Tk_s keys (its cached context followed by its
// new tokens) and Tq_s <= Tk_s new tokens, the queries; query t sits at
// position ctx_s + t with ctx_s = Tk_s - Tq_s and sees keys 0..ctx_s + t
// (chunked prefill continues a prompt after ctx_s cached tokens; ctx_s = 0 is
// a whole prompt).  Queries and outputs of sequence s are rows cu_q[s] ..
// cu_q[s+1]-1, its keys and values rows cu_k[s] .. cu_k[s+1]-1.
//
// Work decomposition: workgroup = (block of 256 queries, head), 8 waves; wave
// w owns queries 32w..32w+31 of the block.  The keys and values of each
// 64-token tile are staged once in LDS and shared by the eight waves (a
// workgroup of 128 queries fetched twice the bytes per flop and was bound by
// them), three tiles ahead of the one computed.  One step of a wave is one
// hand-ordered instruction stream over one tile (prefill_asm.inc, written by
// gen_prefill_asm.py; bf16 MFMA 32x32x16, fp32 accumulate), the tile split
// into 32-key halves A and B:
//   S^T[key, q] = sum_d K[key, d] Q[q, d]     A = K tile (ds_read_b128),
//                                             B = Q^T, register resident
//   softmax numerators p = 2^(s * scale - m_ref) (per lane: one query, 16
//   keys of a half; the other 16 keys of that query sit in lane ^ 32)
//   O^T[v, q] += sum_key V^T[v, key] P^T[key, q]   A = V^T read with
//                                             ds_read_b64_tr_b16, B = P^T
//                                             straight from the S^T registers
// in the order scores A, scores B with the softmax of A between them, sum A
// with the softmax of B between them, sum B.  The token order inside each
// 16-key MFMA k-step is the same permutation on both operands (register r of
// the scores holds key 8(r/4) + 4hf + r%4), so P never leaves registers.
// The reference m_ref is fixed per query at its first tile (key 0 is
// visible to every query), so the accumulators are never rescaled; if a
// later score exceeds it by more than 64 (log2 units), past which the
// numerators could overflow, the workgroup redoes its pass with the largest
// score as reference.  The query's RoPE part is rotated as it is loaded
// (pair k of the 64-wide part: dims k and k + 32, angle pos / theta^(2k/64))
// and rounded to bf16 like the rest of the query.  Query blocks run longest
// first.
#include <cmath>

#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"
#include "prefill_asm.inc"

namespace mla {
namespace {

constexpr int kPH = 128;        // d_h (content part of q and k)
constexpr int kPR = 64;         // d_R
constexpr int kPD = kPH + kPR;  // 192
constexpr int kPV = 128;        // d_v
constexpr int kKC = kPD * 2 / 16;   // 24 sixteen-byte chunks per key row
constexpr int kVS = 16;             // chunks per staged value row
constexpr int kWaves = 8;               // 32 queries each: 256 queries per workgroup
constexpr int kQB = 32 * kWaves;
constexpr int kTK = 64;                 // keys per staged tile (two 32-key MFMA sub-tiles)
constexpr int kKTile = kTK * kKC * 16;  // 24,576 B
constexpr int kVTile = kTK * kVS * 16;  // 16,384 B
constexpr int kBuf = kKTile + kVTile;   // one tile: 40 wave-wide 1 KB copies
constexpr int kNBuf = 4;                // tiles in LDS (160 KB): keys and values of one tile each
constexpr int kCopies = kBuf / 1024 / kWaves;  // copies per wave per tile

struct PrefillParams {
  const __bf16* q_nope;  // [T, n_h, 128]
  const __bf16* q_pe;    // [T, n_h, 64], before RoPE
  const __bf16* k_nope;  // [T, n_h, 128]
  const __bf16* k_rope;  // row t at k_rope + t * k_rope_stride: 64 values, RoPE applied
  const __bf16* v;       // [T, n_h, 128]
  __bf16* out;           // [T, n_h, 128]
  float* lse;            // [T, n_h] natural log, or null
  int T, n_h, k_rope_stride;
  float scale_log2;
  const int32_t* cu_q;   // [num_seqs + 1] query row offsets, or null: one sequence of T queries and T keys
  const int32_t* cu_k;   // [num_seqs + 1] key row offsets
  int max_q;             // most queries of one sequence (sizes the grid)
};

__device__ __forceinline__ bf16x8_t ld8(const __bf16* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// K tile: chunk c of key row r at r * 24 + (c ^ ((r >> 1) & 7)): the XOR stays
// inside the chunk's group of eight, and 16 consecutive rows of one logical
// chunk land on 16 distinct bank groups.  V tile: chunk c of row r at
// r * 16 + (c ^ 2(r & 3)), so the four rows of a transposed read hit four
// different 32-byte spans.  Tiles arrive by direct global->LDS copies (lane l of copy i fills
// slot 64i + l, so the layout is chosen by which chunk each lane fetches),
// three tiles ahead of the one being computed (four tile buffers).
__device__ __forceinline__ int k_slot(int r, int c) { return r * kKC + (c ^ ((r >> 1) & 7)); }

__global__ void __launch_bounds__(64 * kWaves) prefill_attention_kernel(PrefillParams p, RopeTable64 rope) {
  __shared__ __attribute__((aligned(1024))) char tiles_raw[kNBuf * kBuf];
  MLA_LDS char* tiles = (MLA_LDS char*)tiles_raw;
  const uint32_t tiles_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tiles));
  const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups reach the eight XCDs round-robin by linear id.  The n-th
  // workgroup on XCD x takes head x + 8(n / nqb) and query block n % nqb
  // (longest first), so the query blocks of one head run together on one XCD
  // and read that head's keys and values through its L2.
  const int nqb = (p.max_q + kQB - 1) / kQB;
  const int id = blockIdx.x + gridDim.x * blockIdx.y;   // gridDim.y is a multiple of 8
  const int xcd = id & 7, n = id >> 3;
  const int head = xcd + 8 * (n / nqb);
  const int qb = nqb - 1 - n % nqb;
  if (head >= p.n_h) return;
  // this workgroup's sequence: query rows q_row0 + [0, Tq), key rows k_row0 + [0, Tk)
  int Tq = p.T, Tk = p.T, q_row0 = 0, k_row0 = 0;
  if (p.cu_q != nullptr) {
    const MLA_CONST int32_t* cq = (const MLA_CONST int32_t*)(p.cu_q);
    const MLA_CONST int32_t* ck = (const MLA_CONST int32_t*)(p.cu_k);
    q_row0 = cq[blockIdx.z];
    Tq = cq[blockIdx.z + 1] - q_row0;
    k_row0 = ck[blockIdx.z];
    Tk = ck[blockIdx.z + 1] - k_row0;
  }
  if (qb * kQB >= Tq || Tk <= 0) return;
  const int ctx = max(Tk - Tq, 0);                        // cached keys before the first query
  const int q0 = qb * kQB + 32 * wave;                   // this wave's first query
  const int my_q = q0 + l32;
  const int qc = min(my_q, Tq - 1);
  const int vis = min(ctx + my_q, Tk - 1);               // last key this query sees
  const int last_key = min(ctx + qb * kQB + kQB - 1, Tk - 1);
  const int n_tiles = last_key / kTK + 1;              // tiles the workgroup reads

  // Q^T fragments: qf[s] = Q[q][16s + 8hf .. +7]; s < 8 content, s >= 8 RoPE
  // part.  The RoPE part is rotated once the loads have landed and the
  // first tile copies are on their way (further down); its angles are taken
  // here, while the loads are in flight: the angle is reduced to a fraction
  // of a turn in double precision and its sine and cosine taken by the
  // hardware's turn-based v_sin / v_cos (about 1e-6 absolute, far below the
  // bf16 rounding of the rotated values).
  bf16x8_t qf[kPD / 16];
  bf16x8_t x[4];
  float rc[16], rs[16];
  {
    const int64_t qrow = q_row0 + qc;
    const int qpos = ctx + qc;
    const __bf16* qn = p.q_nope + (qrow * p.n_h + head) * kPH + 8 * hf;
#pragma unroll
    for (int s = 0; s < kPH / 16; ++s) qf[s] = ld8(qn + 16 * s);
    const __bf16* qr = p.q_pe + (qrow * p.n_h + head) * kPR + 8 * hf;
#pragma unroll
    for (int s = 0; s < 4; ++s) x[s] = ld8(qr + 16 * s);
    // dims d = 16s + 8hf + e; s = 0, 1 hold pair members k = d, s = 2, 3 their partners k + 32
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const double turns = static_cast<double>(qpos) * rope.inv[16 * (i >> 3) + 8 * hf + (i & 7)] * 0.15915494309189533577;
      const float f = static_cast<float>(turns - rint(turns));
      rc[i] = __builtin_amdgcn_cosf(f);
      rs[i] = __builtin_amdgcn_sinf(f);
    }
    wait_vmcnt<0>();  // complete before the tile copies start counting
  }
  // per-lane LDS offsets.  Key fragment s of lane (row l32, chunk 2s + hf) is
  // at kq_off[s & 3] + 128 (s >> 2): the row's XOR swizzle touches only the
  // low three chunk bits.  Value fragment (k-step ks, half h2, column tile
  // ct) is at pv_off[h2][ct & 1] + 4096 ks + 128 (ct >> 1), for the same
  // reason (16 rows further keep the row's swizzle).
  int kq_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) kq_off[s] = k_slot(l32, 2 * s + hf) * 16;
  const int L = lane & 15, cg = (lane >> 4) & 1;
  int pv_off[2][2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int row = 8 * h2 + 4 * hf + (L >> 2);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int chunk = 4 * par + 2 * cg + ((L & 3) >> 1);
      pv_off[h2][par] = (row * kVS + (chunk ^ (2 * (row & 3)))) * 16 + 8 * (L & 1);
    }
  }

  // Copies of tile k into buffer k % kNBuf: copy i = wave + 8j of the
  // tile's 40 lands at buffer offset 1024 i; lane l fills slot 64 i + l.
  // Copies 0-2 of a wave fill key rows, copies 3, 4 value rows.  A key lane's
  // source is its chunk of key row 0 of the sequence (cp) plus the row times
  // the stride of the array the chunk comes from (cs); a value lane's is the
  // tile's first value row (a uniform base) plus row * n_h * 256 B plus its
  // column.  The rows (0..63) and value columns are packed into d0, d1.
  const char* cp[3];
  uint32_t cs[3];
  uint32_t d0 = 0, d1 = 0;
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int i = wave + kWaves * j, slot = 64 * i + lane;
    if (j < 3) {
      const int r = slot / kKC, c = (slot - r * kKC) ^ ((r >> 1) & 7);
      d0 |= static_cast<uint32_t>(r) << (8 * j);
      if (c < 16) {
        cp[j] = reinterpret_cast<const char*>(p.k_nope + (static_cast<int64_t>(k_row0) * p.n_h + head) * kPH + 8 * c);
        cs[j] = p.n_h * kPH * 2;
      } else {
        cp[j] = reinterpret_cast<const char*>(p.k_rope + static_cast<int64_t>(k_row0) * p.k_rope_stride + 8 * (c - 16));
        cs[j] = p.k_rope_stride * 2;
      }
    } else {
      const int s2 = slot - kKTile / 16, r = s2 / kVS, c = (s2 - r * kVS) ^ (2 * (r & 3));
      if (j == 3) d0 |= static_cast<uint32_t>(r) << 24, d1 |= static_cast<uint32_t>(16 * c) << 8;
      else d1 |= static_cast<uint32_t>(r) | static_cast<uint32_t>(16 * c) << 16;
    }
  }
  const uint32_t vs = p.n_h * kPV * 2;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  auto issue = [&](int k) {
    const int row0 = kTK * k;
    const int rlast = min(kTK - 1, Tk - 1 - row0);
    const char* vbase = reinterpret_cast<const char*>(p.v + ((static_cast<int64_t>(k_row0) + row0) * p.n_h + head) * kPV);
    const uint32_t cd = __builtin_amdgcn_readfirstlane(tiles_addr + (k % kNBuf) * kBuf + wave * 1024);
    asm volatile(MLA_PF_COPY
                 :
                 : [d0] "v"(d0), [d1] "v"(d1), [cp0] "v"(cp[0]), [cp1] "v"(cp[1]), [cp2] "v"(cp[2]),
                   [cs0] "v"(cs[0]), [cs1] "v"(cs[1]), [cs2] "v"(cs[2]), [rlast] "s"(rlast), [row0] "s"(row0),
                   [vbase] "s"(vbase), [vs] "s"(vs), [cd] "s"(cd)
                 : MLA_PF_ASM_SCRATCH, "vcc", "m0", "memory");
  };
#pragma clang diagnostic pop

  // the first tiles' copies go out before the query's RoPE part is rotated
  for (int k = 0; k < 3 && k < n_tiles; ++k) issue(k);
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float cs = rc[8 * s + e], sn = rs[8 * s + e];
      const float a = static_cast<float>(x[s][e]), b = static_cast<float>(x[s + 2][e]);
      qf[8 + s][e] = f32_to_bf16(a * cs - b * sn);
      qf[10 + s][e] = f32_to_bf16(a * sn + b * cs);
    }

  f32x16_t oacc[kPV / 32];
  float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f;
  // the wave's queries see keys up to ctx + q0 + 31 (its last query), and
  // every key of a tile up to min(ctx + q0, Tk - 1) (its first query's last)
  const int wave_last = ctx + q0 + 31;
  const int wave_full = min(ctx + q0, Tk - 1);
  const int vis_lim = vis - 4 * hf;
  const float scale = p.scale_log2;

#define MLA_PF_OUT                                                                             \
  [o0] "+v"(oacc[0]), [o1] "+v"(oacc[1]), [o2] "+v"(oacc[2]), [o3] "+v"(oacc[3]),             \
      [mref] "+v"(m_ref), [mseen] "+v"(m_seen), [lrun] "+v"(l_run)
#define MLA_PF_IN                                                                              \
  [q0] "v"(qf[0]), [q1] "v"(qf[1]), [q2] "v"(qf[2]), [q3] "v"(qf[3]), [q4] "v"(qf[4]),         \
      [q5] "v"(qf[5]), [q6] "v"(qf[6]), [q7] "v"(qf[7]), [q8] "v"(qf[8]), [q9] "v"(qf[9]),     \
      [q10] "v"(qf[10]), [q11] "v"(qf[11]), [kq0] "v"(kq_off[0]), [kq1] "v"(kq_off[1]),        \
      [kq2] "v"(kq_off[2]), [kq3] "v"(kq_off[3]), [va0] "v"(pv_off[0][0]),                     \
      [va1] "v"(pv_off[0][1]), [va2] "v"(pv_off[1][0]), [va3] "v"(pv_off[1][1]), [kb] "s"(kb),  \
      [vb] "s"(vb), [scale] "s"(scale), [lim] "v"(lim), [msk] "s"(msk)
#define MLA_PF_CLOBBER MLA_PF_ASM_SCRATCH, "vcc", "scc", "memory"

  // One pass over the wave's tiles.  Step k waits for tile k (each wave its
  // own copies, then a barrier), issues the copies of tile k+3 into the
  // buffer of tile k-1 (which every wave finished in step k-1), and runs one
  // stream over tile k.  The numerators are taken against a reference fixed
  // at the first tile (key 0 is visible to every query); the pass reports
  // whether a later tile's largest score exceeded it by more than kSlack
  // (log2 units), past which the numerators could overflow.
  constexpr float kSlack = 64.f;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  auto run_pass = [&](bool set_ref) -> bool {
#pragma unroll
    for (int ct = 0; ct < kPV / 32; ++ct) oacc[ct] = f32x16_t{};
    l_run = 0.f;
    if (!set_ref)  // the first pass finds its first tiles issued
      for (int k = 0; k < 3 && k < n_tiles; ++k) issue(k);
    for (int k = 0; k < n_tiles; ++k) {
      const int ahead = min(n_tiles - 1 - k, 2);  // tiles issued after tile k
      if (ahead == 2) wait_vmcnt<2 * kCopies>();
      else if (ahead == 1) wait_vmcnt<kCopies>();
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      if (k + 3 < n_tiles) issue(k + 3);
      if (kTK * k > wave_last) continue;
      const uint32_t kb = __builtin_amdgcn_readfirstlane(tiles_addr + (k % kNBuf) * kBuf);
      const uint32_t vb = kb + kKTile;
      const int lim = vis_lim - kTK * k;
      const int msk = __builtin_amdgcn_readfirstlane(kTK * k + kTK - 1 > wave_full);
      if (k == 0 && set_ref)
        asm volatile(MLA_PF_FIRST : MLA_PF_OUT : MLA_PF_IN : MLA_PF_CLOBBER);
      else
        asm volatile(MLA_PF_STEP : MLA_PF_OUT : MLA_PF_IN : MLA_PF_CLOBBER);
    }
    return m_seen * scale > m_ref + kSlack;
  };
#pragma clang diagnostic pop
  const bool flagged = run_pass(true);
  // workgroup-wide decision on a second pass, through words in tile buffer 0
  // (no wave reads the tiles once every wave has passed this barrier)
  MLA_LDS int* xflag = reinterpret_cast<MLA_LDS int*>(tiles);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  if (lane == 0) xflag[wave] = __builtin_amdgcn_ballot_w64(flagged) != 0;
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  int any = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) any |= xflag[w];
  if (any) {
    __builtin_amdgcn_s_barrier();  // every wave has read the flags
    // the reference becomes the largest scaled score of the query (both lanes)
    m_ref = fmaxf(m_seen, __shfl_xor(m_seen, 32)) * scale;
    run_pass(false);
  }

  // epilogue: normalise and store the rows of this wave's queries
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (my_q < Tq) {
    const int64_t out_row = q_row0 + my_q;
    __bf16* orow = p.out + (out_row * p.n_h + head) * kPV;
#pragma unroll
    for (int ct = 0; ct < kPV / 32; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4_t o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16(oacc[ct][4 * j + i] * inv);
        *reinterpret_cast<bf16x4_t*>(orow + 32 * ct + 8 * j + 4 * hf) = o;
      }
    if (p.lse != nullptr && hf == 0)
      p.lse[out_row * p.n_h + head] =
          (m_ref + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
}

}  // namespace

hipError_t launch_prefill_attention(const PrefillArgs& a, hipStream_t st) {
  PrefillParams p;
  p.q_nope = static_cast<const __bf16*>(a.q_nope);
  p.q_pe = static_cast<const __bf16*>(a.q_pe);
  p.k_nope = static_cast<const __bf16*>(a.k_nope);
  p.k_rope = static_cast<const __bf16*>(a.k_rope);
  p.v = static_cast<const __bf16*>(a.v);
  p.out = static_cast<__bf16*>(a.out);
  p.lse = a.lse;
  p.T = a.seq_len;
  p.n_h = a.n_h;
  p.k_rope_stride = a.k_rope_stride;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.max_q = a.cu_q != nullptr ? a.max_q : a.seq_len;
  RopeTable64 rope;
  for (int k = 0; k < 32; ++k) rope.inv[k] = std::pow(static_cast<double>(a.theta), -2.0 * k / kPR);
  // (nqb query blocks x n_h heads, padded to a multiple of 8 heads: the
  // extra workgroups exit at once) per sequence
  const int nqb = (p.max_q + kQB - 1) / kQB;
  const int heads8 = (a.n_h + 7) / 8 * 8;
  const int seqs = a.cu_q != nullptr ? a.num_seqs : 1;
  hipLaunchKernelGGL(prefill_attention_kernel, dim3(nqb, heads8, seqs), dim3(64 * kWaves), 0, st, p, rope);
  return hipGetLastError();
}

}  // namespace mla
