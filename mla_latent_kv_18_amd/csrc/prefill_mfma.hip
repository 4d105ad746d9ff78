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
// Work decomposition: workgroup = (block of 128 queries, head), 4 waves; wave
// w owns queries 32w..32w+31 of the block.  The keys and values of each
// 32-token tile are staged once in LDS and shared by the four waves.  Per
// tile, per wave (bf16 MFMA 32x32x16, fp32 accumulate):
//   S^T[key, q] = sum_d K[key, d] Q[q, d]     A = K tile (ds_read_b128),
//                                             B = Q^T, register resident
//   online softmax over the keys (per lane: one query, 16 keys; the other 16
//   keys of that query sit in lane ^ 32), rescaling O when the maximum grows
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

namespace mla {
namespace {

constexpr int kPH = 128;        // d_h (content part of q and k)
constexpr int kPR = 64;         // d_R
constexpr int kPD = kPH + kPR;  // 192
constexpr int kPV = 128;        // d_v
constexpr int kKC = kPD * 2 / 16;   // 24 sixteen-byte chunks per key row
constexpr int kVS = 18;             // chunks per staged value row (16 used; 2 of padding)
constexpr int kKTile = 32 * kKC * 16;   // 12,288 B
constexpr int kVTile = 32 * kVS * 16;   //  9,216 B

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
// chunk land on 16 distinct bank groups.  V tile: rows of 18 chunks.
__device__ __forceinline__ int k_slot(int r, int c) { return r * kKC + (c ^ ((r >> 1) & 7)); }

__global__ void __launch_bounds__(256) prefill_attention_kernel(PrefillParams p, RopeTable64 rope) {
  __shared__ __attribute__((aligned(16))) char ktile[kKTile];
  __shared__ __attribute__((aligned(16))) char vtile[kVTile];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5, l32 = lane & 31;
  const int head = blockIdx.y;
  const int nqb = (p.T + 127) / 128;
  const int qb = nqb - 1 - static_cast<int>(blockIdx.x);  // longest blocks first
  const int q0 = qb * 128 + 32 * wave;                   // this wave's first query
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
        pv_off[ks][h2][ct] = (row * kVS + chunk) * 16 + 8 * (L & 1);
      }
    }

  // staging: thread t copies key chunks t + 256m (m < 3) and value chunks t + 256m (m < 2)
  bf16x8_t kr[3], vr[2];
  auto fetch = [&](int k) {
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      const int i = tid + 256 * m, r = i / kKC, c = i - r * kKC;
      const int key = min(32 * k + r, p.T - 1);
      kr[m] = c < 16 ? ld8(p.k_nope + (static_cast<int64_t>(key) * p.n_h + head) * kPH + 8 * c)
                     : ld8(p.k_rope + static_cast<int64_t>(key) * p.k_rope_stride + 8 * (c - 16));
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int i = tid + 256 * m, r = i >> 4, c = i & 15;
      const int key = min(32 * k + r, p.T - 1);
      vr[m] = ld8(p.v + (static_cast<int64_t>(key) * p.n_h + head) * kPV + 8 * c);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      const int i = tid + 256 * m, r = i / kKC, c = i - r * kKC;
      *reinterpret_cast<bf16x8_t*>(ktile + k_slot(r, c) * 16) = kr[m];
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int i = tid + 256 * m, r = i >> 4, c = i & 15;
      *reinterpret_cast<bf16x8_t*>(vtile + (r * kVS + c) * 16) = vr[m];
    }
  };

  f32x16_t oacc[kPV / 32];
#pragma unroll
  for (int ct = 0; ct < kPV / 32; ++ct) oacc[ct] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  const int last_key = min(qb * 128 + 127, p.T - 1);
  const int n_tiles = last_key / 32 + 1;
  fetch(0);
  for (int k = 0; k < n_tiles; ++k) {
    stage();
    __syncthreads();
    if (k + 1 < n_tiles) fetch(k + 1);
    if (32 * k <= q0 + 31) {  // some key of the tile is visible to this wave
      f32x16_t sacc = f32x16_t{};
#pragma unroll
      for (int s = 0; s < kPD / 16; ++s) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(ktile + kq_off[s]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc, 0, 0, 0);
      }
      // register r holds key 32k + 8(r/4) + 4hf + r%4
      float sv[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * k + 8 * (r >> 2) + 4 * hf + (r & 3);
        sv[r] = key <= my_q ? sacc[r] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      // key 0 is visible to every query, so m_new is finite from the first tile on
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      bf16x8_t pf[2];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(sv[r] - m_new);
        psum += pr;
        pf[r >> 3][r & 7] = f32_to_bf16(pr);
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int ct = 0; ct < kPV / 32; ++ct) oacc[ct] *= alpha;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int ct = 0; ct < kPV / 32; ++ct) {
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<MLA_LDS i16x4_t*>((MLA_LDS char*)vtile + pv_off[ks][0][ct]));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<MLA_LDS i16x4_t*>((MLA_LDS char*)vtile + pv_off[ks][1][ct]));
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], oacc[ct], 0, 0, 0);
        }
    }
    __syncthreads();  // every wave is done with the tile before the next is staged
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
  hipLaunchKernelGGL(prefill_attention_kernel, dim3((a.seq_len + 127) / 128, a.n_h), dim3(256), 0, st, p, rope);
  return hipGetLastError();
}

}  // namespace mla
