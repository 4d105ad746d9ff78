// Launch interfaces between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

struct AppendArgs {
  const void* hidden;
  const void* w;  // null: hidden holds the projection [n, d_c + d_r] fp32
  const float* gamma;
  const int32_t* positions;
  const int64_t* slots;
  int n_tokens, d_model, d_c, d_r;
  int64_t cache_slots;
  float eps, theta;
  void* cache;
  float* cache_scale;
  void* workspace;
  int cache_dtype;
};

struct AbsorbArgs {
  const void* q_nope;
  const void* q_pe;
  const void* w_uk;
  const int32_t* positions;
  int n_tokens, n_h, d_h, d_c, d_r;
  float theta;
  void* q_lat;
  float* q_scale;
  void* workspace;
  int cache_dtype;
};

struct DecodeArgs {
  const void* q_lat;
  const float* q_scale;
  const void* cache;
  const float* cache_scale;
  const int32_t* block_table;
  int max_blocks, num_blocks;
  const int32_t* seq_lens;
  int batch, q_len, n_h, d_c, d_r, block_size, max_seq_len;
  int split_tokens, num_splits;
  float scale;
  void* workspace;  // partials: bf16 [units, rows, 512] then fp32 lse [units, rows]
  void* o_lat;
  float* lse;
  int cache_dtype;
  // planned launch (null items: uniform split): launch list of num_slots
  // int32 x 4 entries and the partial blocks of request b, part_ptr[b] ..
  // part_ptr[b + 1] - 1, out of num_partials
  const int32_t* items;
  const int32_t* part_ptr;
  int num_slots, num_partials;
};

struct OutProjArgs {
  const void* o_lat;
  const void* w_uv;
  int n_tokens, n_h, d_c, d_v;
  void* out;
};

// y [m, n] = x [m, k] w [n, k]^T, bf16 (n % 128 == 0, k % 16 == 0, x rows ldx apart)
struct LinearArgs {
  const void* x;
  const void* w;
  int m, n, k, ldx;
  void* y;
  void* workspace;
};

// C_i = X_i Y_i for i < batch: C_i[r, c] = sum_k X_i[r, k] Y_i[k, c] with
// every operand addressed through element strides (absorbed weights)
struct FoldArgs {
  const void* x;
  const void* y;
  void* out;
  int batch, rows, cols, k;
  int64_t xs_i, xs_r, xs_k, ys_i, ys_k, ys_c, os_i, os_r, os_c;
};
hipError_t launch_fold(const FoldArgs&, bool bf16, hipStream_t);

// fp32, any dims
hipError_t launch_append_f32(const AppendArgs&, hipStream_t);
hipError_t launch_absorb_q_f32(const AbsorbArgs&, hipStream_t);
hipError_t launch_decode_f32(const DecodeArgs&, hipStream_t);
hipError_t launch_out_proj_f32(const OutProjArgs&, hipStream_t);

// bf16 activations, d_c = 512, d_r = 64, d_h = d_v = 128 (MFMA)
size_t append_mfma_workspace(int n_tokens);
hipError_t launch_append_mfma(const AppendArgs&, hipStream_t);
size_t absorb_mfma_workspace(int n_tokens, int n_h, int cache_dtype);
hipError_t launch_absorb_q_mfma(const AbsorbArgs&, hipStream_t);
hipError_t launch_out_proj_mfma(const OutProjArgs&, hipStream_t);
// append (with its down-projection) and absorb q in one launch, then the finish
hipError_t launch_append_absorb_mfma(const AppendArgs&, const AbsorbArgs&, hipStream_t);

// latent decode, bf16 or fp8 cache (d_c = 512, d_r = 64)
int decode_waves_per_group(int n_h, int q_len);
size_t decode_mfma_workspace(int batch, int q_len, int n_h, int num_splits);
hipError_t launch_decode_mfma(const DecodeArgs&, hipStream_t);
hipError_t launch_decode_fp8(const DecodeArgs&, hipStream_t);
// decode over the cache variants, rows expanded to bf16 in LDS
enum { kDqFp4Mx = 0, kDqFp8Kr = 1, kDqBf16Nope = 2 };
hipError_t launch_decode_dq(const DecodeArgs&, int fmt, hipStream_t);
// the pipelined decode stream (workgroups of 128 rows, q_len <= 32) over
// bf16 576-wide rows (launch_decode_mfma), NoPE rows and FP4 rows
bool decode_pipe_supported(int n_h, int q_len);
// streaming read of a buffer (achievable HBM read rate); mode 0: loads into
// registers, grid kProbeRegsGrid, one XOR word per workgroup into sink;
// mode 1: direct global->LDS copies of 36 KB tiles, 256 workgroups
constexpr int kProbeRegsGrid = 2048;
hipError_t launch_hbm_read_probe(const void* buf, size_t bytes, int mode, uint32_t* sink, hipStream_t st);
hipError_t launch_decode_pipe(const DecodeArgs&, int fmt, hipStream_t);
// causal prefill attention of one sequence with per-head keys and values
// (q, k: [d_h content ; d_R RoPE part] = 192 wide, v: 128 wide)
struct PrefillArgs {
  const void* q_nope;
  const void* q_pe;
  const void* k_nope;
  const void* k_rope;
  int k_rope_stride;
  const void* v;
  int seq_len, n_h;
  float scale, theta;
  void* out;
  float* lse;
  // several sequences (null cu_q: one sequence of seq_len queries and keys)
  const int32_t* cu_q;
  const int32_t* cu_k;
  int num_seqs, max_q;
};
hipError_t launch_prefill_attention(const PrefillArgs&, hipStream_t);

// skinny GEMM of the projections around the attention block
int linear_chunks(int m, int n, int k);
size_t linear_workspace(int m, int n, int k);
hipError_t launch_linear(const LinearArgs&, hipStream_t);
// y [m, n] = x w^T and y2 [m, n2] = x w2^T in one launch (n2 % 128 == 0;
// workspace sized by linear_workspace(m, n + n2, k))
hipError_t launch_linear_pair(const LinearArgs&, const void* w2, int n2, void* y2, hipStream_t);

// merge of the chunk partials that a split decode left in the workspace
// (xcd_group: the partials of request b were written on XCD b % 8, batch % 8 == 0)
hipError_t launch_combine(const DecodeArgs&, hipStream_t, bool xcd_group = false);
// partial row blocks the decode of `a` writes (0: no combine)
int64_t partial_units(const DecodeArgs& a);

}  // namespace mla
