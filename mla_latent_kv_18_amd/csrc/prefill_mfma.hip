// Prefill attention, the non-absorbed side of MLA: keys and values are
// materialised per head (k^C_i = W^UK_i c, v_i = W^UV_i c, by mla_linear
// over the latent rows) and each head runs causal attention with query and
// key width d_h + d_R = 192 and value width d_v = 128 [MLA explainer,
// decoupled RoPE eq.(14) (q and k of a head are [content ; RoPE part]) and
// eq.(16) (the score is the sum of both blocks); trade-offs section (the
// prompt is processed without absorption)].
//
// One sequence of T tokens at positions 0..T-1; query t sees keys 0..t.
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
constexpr int kNBuf = 4;                // tiles in LDS (160 KB): the one computed and three landing
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
};

__device__ __forceinline__ bf16x8_t ld8(const __bf16* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// K tile: chunk c of key row r at r * 24 + (c ^ ((r >> 1) & 7)): the XOR stays
// inside the chunk's group of eight, and 16 consecutive rows of one logical
// chunk land on 16 distinct bank groups.  V tile: chunk c of row r at
// r * 16 + (c ^ 2(r & 3)), so the four rows of a transposed read hit four
// different 32-byte spans.  Tiles arrive by direct global->LDS copies (lane l of copy i fills
// slot 64i + l, so the layout is chosen by which chunk each lane fetches),
// up to three tiles ahead of the one being computed.
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
  const int nqb = (p.T + kQB - 1) / kQB;
  const int id = blockIdx.x + gridDim.x * blockIdx.y;
  const int xcd = id & 7, n = id >> 3;
  const int head = xcd + 8 * (n / nqb);
  const int qb = nqb - 1 - n % nqb;
  if (head >= p.n_h) return;
  const int q0 = qb * kQB + 32 * wave;                   // this wave's first query
  const int my_q = q0 + l32;
  const int qc = min(my_q, p.T - 1);

  // Q^T fragments: qf[s] = Q[q][16s + 8hf .. +7]; s < 8 content, s >= 8 RoPE part
  bf16x8_t qf[kPD / 16];
  {
    const __bf16* qn = p.q_nope + (static_cast<int64_t>(qc) * p.n_h + head) * kPH + 8 * hf;
#pragma unroll
    for (int s = 0; s < kPH / 16; ++s) qf[s] = ld8(qn + 16 * s);
    const __bf16* qr = p.q_pe + (static_cast<int64_t>(qc) * p.n_h + head) * kPR + 8 * hf;
    bf16x8_t x[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) x[s] = ld8(qr + 16 * s);
    // dims d = 16s + 8hf + e; s = 0, 1 hold pair members k = d, s = 2, 3 their partners k + 32
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float cs, sn;
        rope_cos_sin_inv(qc, rope.inv[16 * s + 8 * hf + e], &cs, &sn);
        const float a = static_cast<float>(x[s][e]), b = static_cast<float>(x[s + 2][e]);
        qf[8 + s][e] = f32_to_bf16(a * cs - b * sn);
        qf[10 + s][e] = f32_to_bf16(a * sn + b * cs);
      }
    wait_vmcnt<0>();  // complete before the tile copies start counting
  }

  // per-lane LDS offsets
  int kq_off[kPD / 16];
#pragma unroll
  for (int s = 0; s < kPD / 16; ++s) kq_off[s] = k_slot(l32, 2 * s + hf) * 16;
  const int L = lane & 15, cg = (lane >> 4) & 1;
  int pv_off[2][2][4];  // [k-step][h2][value column tile]
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int row = 16 * ks + 8 * h2 + 4 * hf + (L >> 2);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int chunk = 8 * (ct >> 1) + 4 * (ct & 1) + 2 * cg + ((L & 3) >> 1);
        pv_off[ks][h2][ct] = (row * kVS + (chunk ^ (2 * (row & 3)))) * 16 + 8 * (L & 1);
      }
    }

  // copies of tile k into buffer bi: copy i = wave + 8j; the first 24 fill the
  // key rows, the last 16 the value rows
  auto issue = [&](int k, int bi) {
#pragma unroll
    for (int j = 0; j < kCopies; ++j) {
      const int i = wave + kWaves * j, slot = 64 * i + lane;
      const __bf16* g;
      if (i < kKTile / 1024) {
        const int r = slot / kKC, c = (slot - r * kKC) ^ ((r >> 1) & 7);
        const int key = min(kTK * k + r, p.T - 1);
        g = c < 16 ? p.k_nope + (static_cast<int64_t>(key) * p.n_h + head) * kPH + 8 * c
                   : p.k_rope + static_cast<int64_t>(key) * p.k_rope_stride + 8 * (c - 16);
      } else {
        const int s2 = slot - kKTile / 16, r = s2 / kVS, c = (s2 - r * kVS) ^ (2 * (r & 3));
        const int key = min(kTK * k + r, p.T - 1);
        g = p.v + (static_cast<int64_t>(key) * p.n_h + head) * kPV + 8 * c;
      }
      dma16(g, tiles_addr + bi * kBuf + i * 1024);
    }
  };

  f32x16_t oacc[kPV / 32];
#pragma unroll
  for (int ct = 0; ct < kPV / 32; ++ct) oacc[ct] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  const int last_key = min(qb * kQB + kQB - 1, p.T - 1);
  const int n_tiles = last_key / kTK + 1;
#pragma unroll
  for (int k = 0; k < kNBuf - 1; ++k)
    if (k < n_tiles) issue(k, k);
  for (int k = 0; k < n_tiles; ++k) {
    // copies still allowed in flight: those of the tiles issued after tile k
    switch (min(n_tiles - 1 - k, kNBuf - 2)) {  // copies of the tiles issued after tile k may be in flight
      case 2: wait_vmcnt<2 * kCopies>(); break;
      case 1: wait_vmcnt<kCopies>(); break;
      default: wait_vmcnt<0>(); break;
    }
    __builtin_amdgcn_s_barrier();  // tile k visible to all; tile k-1 released by all
    if (k + kNBuf - 1 < n_tiles) issue(k + kNBuf - 1, (k + kNBuf - 1) % kNBuf);
    MLA_LDS char* ktile = tiles + (k % kNBuf) * kBuf;
    MLA_LDS char* vtile = ktile + kKTile;
    const int key0 = kTK * k;
    if (key0 <= q0 + 31) {  // some key of the tile is visible to this wave
      // scores of the two 32-key sub-tiles: two independent MFMA chains
      f32x16_t sc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
      for (int s = 0; s < kPD / 16; ++s)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const bf16x8_t kf = *reinterpret_cast<MLA_LDS const bf16x8_t*>(ktile + sub * (32 * kKC * 16) + kq_off[s]);
          sc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sc[sub], 0, 0, 0);
        }
      // register r of sub-tile u holds key key0 + 32u + 8(r/4) + 4hf + r%4
      float mx = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * sub + 8 * (r >> 2) + 4 * hf + (r & 3);
          sc[sub][r] = key <= my_q ? sc[sub][r] * p.scale_log2 : -INFINITY;
          mx = fmaxf(mx, sc[sub][r]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      // key 0 is visible to every query, so m_new is finite from the first tile on
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      bf16x8_t pf[4];
      float psum = 0.f;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = __builtin_amdgcn_exp2f(sc[sub][r] - m_new);
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
      // k-steps 0, 1 sum the first sub-tile's values, 2, 3 the second's
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int ct = 0; ct < kPV / 32; ++ct) {
          MLA_LDS char* vb = vtile + (ks >> 1) * (32 * kVS * 16);
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<MLA_LDS i16x4_t*>(vb + pv_off[ks & 1][0][ct]));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<MLA_LDS i16x4_t*>(vb + pv_off[ks & 1][1][ct]));
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], oacc[ct], 0, 0, 0);
        }
    }
  }

  // epilogue: normalise and store the rows of this wave's queries
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (my_q < p.T) {
    __bf16* orow = p.out + (static_cast<int64_t>(my_q) * p.n_h + head) * kPV;
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
      p.lse[static_cast<int64_t>(my_q) * p.n_h + head] =
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
  RopeTable64 rope;
  for (int k = 0; k < 32; ++k) rope.inv[k] = std::pow(static_cast<double>(a.theta), -2.0 * k / kPR);
  // n_h heads x nqb query blocks, padded to a multiple of 8 heads (the extra workgroups exit at once)
  const int nqb = (a.seq_len + kQB - 1) / kQB;
  const int heads8 = (a.n_h + 7) / 8 * 8;
  hipLaunchKernelGGL(prefill_attention_kernel, dim3(nqb, heads8), dim3(64 * kWaves), 0, st, p, rope);
  return hipGetLastError();
}

}  // namespace mla
