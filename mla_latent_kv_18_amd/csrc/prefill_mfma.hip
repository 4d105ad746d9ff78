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
// them).  Per 64-key tile, per wave (bf16 MFMA 32x32x16, fp32 accumulate), as
// two 32-key sub-tiles whose score chains run side by side:
//   S^T[key, q] = sum_d K[key, d] Q[q, d]     A = K tile (ds_read_b128),
//                                             B = Q^T, register resident
//   (two chains over the even and odd k-steps), online softmax over the keys
//   (per lane: one query, 16 keys; the other 16 keys of that query sit in
//   lane ^ 32), rescaling O only in the tiles where some query's maximum grows
//   O^T[v, q] += sum_key V^T[v, key] P^T[key, q]   A = V^T read with
//                                             ds_read_b64_tr_b16, B = P^T
//                                             straight from the S^T registers
// The token order inside each 16-key MFMA k-step is the same permutation on
// both operands (register r of the scores holds key 8(r/4) + 4hf + r%4), so
// P never leaves registers.  The query's RoPE part is rotated as it is
// loaded (pair k of the 64-wide part: dims k and k + 32, angle
// pos / theta^(2k/64)).  Query blocks run longest first.
#include <cmath>

#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"

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
// two tiles ahead of the one being computed (four tile buffers).
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

  // Q^T fragments: qf[s] = Q[q][16s + 8hf .. +7]; s < 8 content, s >= 8 RoPE part
  bf16x8_t qf[kPD / 16];
  {
    const int64_t qrow = q_row0 + qc;
    const int qpos = ctx + qc;
    const __bf16* qn = p.q_nope + (qrow * p.n_h + head) * kPH + 8 * hf;
#pragma unroll
    for (int s = 0; s < kPH / 16; ++s) qf[s] = ld8(qn + 16 * s);
    const __bf16* qr = p.q_pe + (qrow * p.n_h + head) * kPR + 8 * hf;
    bf16x8_t x[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) x[s] = ld8(qr + 16 * s);
    // dims d = 16s + 8hf + e; s = 0, 1 hold pair members k = d, s = 2, 3 their partners k + 32
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float cs, sn;
        rope_cos_sin_inv(qpos, rope.inv[16 * s + 8 * hf + e], &cs, &sn);
        const float a = static_cast<float>(x[s][e]), b = static_cast<float>(x[s + 2][e]);
        qf[8 + s][e] = f32_to_bf16(a * cs - b * sn);
        qf[10 + s][e] = f32_to_bf16(a * sn + b * cs);
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

  // copies of tile k into buffer bi: copy i = wave + 8j; the first 24 fill the
  // key rows, the last 16 the value rows
  auto issue = [&](int k) {
#pragma unroll
    for (int j = 0; j < kCopies; ++j) {
      const int i = wave + kWaves * j, slot = 64 * i + lane;
      const __bf16* g;
      if (i < kKTile / 1024) {
        const int r = slot / kKC, c = (slot - r * kKC) ^ ((r >> 1) & 7);
        const int64_t key = k_row0 + min(kTK * k + r, Tk - 1);
        g = c < 16 ? p.k_nope + (key * p.n_h + head) * kPH + 8 * c
                   : p.k_rope + key * p.k_rope_stride + 8 * (c - 16);
      } else {
        const int s2 = slot - kKTile / 16, r = s2 / kVS, c = (s2 - r * kVS) ^ (2 * (r & 3));
        const int64_t key = k_row0 + min(kTK * k + r, Tk - 1);
        g = p.v + (key * p.n_h + head) * kPV + 8 * c;
      }
      dma16(g, tiles_addr + (k % kNBuf) * kBuf + i * 1024);
    }
  };

  f32x16_t oacc[kPV / 32];
#pragma unroll
  for (int ct = 0; ct < kPV / 32; ++ct) oacc[ct] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  const int last_key = min(ctx + qb * kQB + kQB - 1, Tk - 1);
  const int n_tiles = last_key / kTK + 1;
  // the wave's queries see keys up to ctx + q0 + 31 (its last query), and
  // every key of a tile up to min(ctx + q0, Tk - 1) (its first query's last)
  const int wave_last = ctx + q0 + 31;
  const int wave_full = min(ctx + q0, Tk - 1);
  auto visible = [&](int k) { return kTK * k <= wave_last; };

  f32x16_t sc[2];
  bf16x8_t pf[4];
  // scores of tile k: S^T for the two 32-key sub-tiles, two independent
  // chains; key fragments are read two k-steps ahead
  auto scores = [&](int k) {
    MLA_LDS const char* ktile = tiles + (k % kNBuf) * kBuf;
    auto kread = [&](int s, int sub) {
      return *reinterpret_cast<MLA_LDS const bf16x8_t*>(ktile + sub * (32 * kKC * 16) + kq_off[s & 3] + 128 * (s >> 2));
    };
    constexpr int kAhead = 2;
    bf16x8_t kf[kAhead][2];
#pragma unroll
    for (int s = 0; s < kAhead; ++s)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) kf[s][sub] = kread(s, sub);
    sc[0] = f32x16_t{};
    sc[1] = f32x16_t{};
#pragma unroll
    for (int s = 0; s < kPD / 16; ++s)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const bf16x8_t cur = kf[s % kAhead][sub];
        if (s + kAhead < kPD / 16) kf[s % kAhead][sub] = kread(s + kAhead, sub);
        sc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[s], sc[sub], 0, 0, 0);
      }
  };
  // O^T += V^T P^T for tile k (k-steps 0, 1 sum the first sub-tile's
  // values, 2, 3 the second's); value fragments are read one MFMA ahead
  auto weighted_sum = [&](int k) {
    MLA_LDS char* vtile = tiles + (k % kNBuf) * kBuf + kKTile;
    auto vread = [&](int i) {
      const int ks = i >> 2, ct = i & 3;
      MLA_LDS char* vb = vtile + (ks >> 1) * (32 * kVS * 16) + (ks & 1) * 4096 + 128 * (ct >> 1);
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<MLA_LDS i16x4_t*>(vb + pv_off[0][ct & 1]));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<MLA_LDS i16x4_t*>(vb + pv_off[1][ct & 1]));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8_t vf[2];
    vf[0] = vread(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 1 < 16) vf[(i + 1) & 1] = vread(i + 1);
      oacc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i & 1], pf[i >> 2], oacc[i & 3], 0, 0, 0);
    }
  };
  // online softmax of tile k's scores: numerators P (bf16) for the next
  // weighted sum, running maximum and sum, O rescaled where a maximum grew.
  // The scale goes into the exponent's fma (the maximum is taken on the raw
  // scores; the scale is positive); keys are masked only in tiles that reach
  // past some query's last visible key.
  auto softmax = [&](int k) {
    const int key0 = kTK * k;
    if (key0 + kTK - 1 > wave_full) {
      // register r of sub-tile u holds key key0 + 32u + 8(r/4) + 4hf + r%4
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * sub + 8 * (r >> 2) + 4 * hf + (r & 3);
          sc[sub][r] = key <= vis ? sc[sub][r] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[sub][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // key 0 is visible to every query, so m_new is finite from the first tile on
    const float m_new = fmaxf(m_run, mx * p.scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(sc[sub][r], p.scale_log2, -m_new));
        psum += pr;
        pf[2 * sub + (r >> 3)][r & 7] = f32_to_bf16(pr);
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // the accumulators are rescaled only when some query's maximum grew
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int ct = 0; ct < kPV / 32; ++ct) oacc[ct] *= alpha;
    }
  };

  // Two groups of four waves (waves w and w + 4 share a SIMD) run the same
  // phase sequence -- matrix phase k (scores of tile k, weighted sum of tile
  // k-1, copies of tile k+2), softmax phase k -- with the second group one
  // phase behind, so that on every SIMD one wave's softmax runs beside the
  // other wave's MFMAs.  Barriers separate the phases.  Tile k+2 goes into
  // the buffer of tile k-2, whose values both groups summed in their matrix
  // phase k-1; each wave's copies of tile k+1 have landed by the end of its
  // matrix phase k.
  if (n_tiles > 0) issue(0);
  if (n_tiles > 1) issue(1);
  if (n_tiles > 1) wait_vmcnt<kCopies>();
  else wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();  // tile 0 visible to all
  const bool late = wave >= kWaves / 2;
  if (late) __builtin_amdgcn_s_barrier();
  for (int k = 0;; ++k) {
    __builtin_amdgcn_s_setprio(1);
    if (k + 2 < n_tiles) issue(k + 2);
    if (k < n_tiles && visible(k)) scores(k);
    if (k >= 1 && visible(k - 1)) weighted_sum(k - 1);
    if (k + 2 < n_tiles) wait_vmcnt<kCopies>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_barrier();
    if (k == n_tiles) break;
    if (visible(k)) softmax(k);
    __builtin_amdgcn_s_barrier();
  }
  if (!late) __builtin_amdgcn_s_barrier();

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
          (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
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
