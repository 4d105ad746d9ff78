// C-ABI entry points of libmla: argument checks on the host, kernel
// selection, launch, HIP error mapping.  No device memory is allocated here.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/mla.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

mla_status_t fail(mla_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

mla_status_t hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) {
    g_err[0] = '\0';
    return MLA_OK;
  }
  return fail(MLA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

struct Resolved {
  int n_h, d_c, d_h, d_r, d_v, d_model, bs, cache_dtype, act_dtype;
  float scale, theta, eps;
  bool mfma;  // bf16 / fp8 path with the fixed MFMA dims
};

int elem_size(int dt) { return dt == MLA_F32 ? 4 : (dt == MLA_BF16 ? 2 : 1); }

mla_status_t resolve(const mla_dims_t* d, Resolved* r) {
  if (d == nullptr) return fail(MLA_ERR_INVALID_ARGUMENT, "dims is NULL");
  r->n_h = d->num_heads;
  r->d_c = d->kv_lora_rank;
  r->d_h = d->qk_nope_head_dim;
  r->d_r = d->qk_rope_head_dim;
  r->d_v = d->v_head_dim;
  r->d_model = d->hidden_size;
  r->bs = d->block_size;
  r->cache_dtype = d->cache_dtype;
  r->act_dtype = d->act_dtype;
  if (r->n_h <= 0 || r->d_c <= 0 || r->d_h <= 0 || r->d_r < 0 || r->d_v <= 0 || r->d_model <= 0 || r->bs <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "dims must be positive (d_R may be 0)");
  if (r->d_r % 2 != 0) return fail(MLA_ERR_INVALID_ARGUMENT, "qk_rope_head_dim must be even");
  r->scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.f / sqrtf(static_cast<float>(r->d_h + r->d_r));
  r->theta = d->rope_theta > 0.f ? d->rope_theta : 10000.f;
  r->eps = d->rms_eps > 0.f ? d->rms_eps : 1e-6f;
  if (r->cache_dtype == MLA_F32 && r->act_dtype == MLA_F32) {
    r->mfma = false;
    return MLA_OK;
  }
  if ((r->cache_dtype == MLA_BF16 || r->cache_dtype == MLA_FP8_E4M3) && r->act_dtype == MLA_BF16) {
    if (r->d_c != 512 || r->d_r != 64 || r->d_h != 128 || r->d_v != 128)
      return fail(MLA_ERR_UNSUPPORTED, "bf16/fp8 kernels need d_c=512, d_R=64, d_h=d_v=128 (got %d,%d,%d,%d)",
                  r->d_c, r->d_r, r->d_h, r->d_v);
    if (r->n_h % 64 != 0) return fail(MLA_ERR_UNSUPPORTED, "bf16/fp8 kernels need num_heads %% 64 == 0");
    if (r->bs % 64 != 0) return fail(MLA_ERR_UNSUPPORTED, "bf16/fp8 kernels need block_size %% 64 == 0");
    if (r->d_model % 64 != 0) return fail(MLA_ERR_UNSUPPORTED, "hidden_size must be a multiple of 64");
    r->mfma = true;
    return MLA_OK;
  }
  return fail(MLA_ERR_UNSUPPORTED, "unsupported dtype pair cache=%d act=%d", r->cache_dtype, r->act_dtype);
}

int32_t default_split(const Resolved& r, int32_t batch, int32_t q_len, int32_t max_seq_len) {
  if (!r.mfma) return max_seq_len > 0 ? max_seq_len : 1;  // the fp32 kernel makes one pass
  const int waves = mla::decode_waves_per_group(r.n_h, q_len);
  const int groups = q_len * r.n_h / (32 * waves);
  const int slots = 256 * (4 / waves);  // workgroups resident at once (1 wave per SIMD)
  const int64_t units = static_cast<int64_t>(batch) * groups;
  int64_t splits = (slots + units - 1) / units;
  if (splits < 1) splits = 1;
  int64_t len = (max_seq_len + splits - 1) / splits;
  if (len < 256) len = 256;
  len = (len + 63) / 64 * 64;
  return static_cast<int32_t>(len);
}

}  // namespace

extern "C" {

size_t mla_cache_row_bytes(const mla_dims_t* dims) {
  // a pure size helper: defined for any positive dims, kernel support aside
  if (dims == nullptr || dims->kv_lora_rank <= 0 || dims->qk_rope_head_dim < 0) return 0;
  if (dims->cache_dtype < MLA_F32 || dims->cache_dtype > MLA_FP8_E4M3) return 0;
  return static_cast<size_t>(dims->kv_lora_rank + dims->qk_rope_head_dim) * elem_size(dims->cache_dtype);
}

size_t mla_q_lat_row_bytes(const mla_dims_t* dims) {
  const size_t row = mla_cache_row_bytes(dims);
  return dims != nullptr && dims->cache_dtype == MLA_FP8_E4M3 ? 2 * row : row;
}

size_t mla_append_workspace_size(const mla_dims_t* dims, int32_t n_tokens) {
  Resolved r;
  if (resolve(dims, &r) != MLA_OK || n_tokens <= 0) return 0;
  return r.mfma ? mla::append_mfma_workspace(n_tokens) : 0;
}

mla_status_t mla_append_latent(const mla_dims_t* dims, const void* hidden, const void* w_dkv_kr,
                               const float* rms_gamma, const int32_t* positions,
                               const int64_t* slot_mapping, int32_t n_tokens, int64_t cache_slots,
                               void* cache, float* cache_scale, void* workspace,
                               size_t workspace_bytes, mla_stream_t stream) {
  Resolved r;
  mla_status_t st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  if (n_tokens < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "n_tokens < 0");
  if (n_tokens == 0) return hip_status(hipSuccess, "");
  if (!hidden || !rms_gamma || !positions || !slot_mapping || !cache)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (cache_slots <= 0) return fail(MLA_ERR_INVALID_ARGUMENT, "cache_slots must be positive");
  if (r.cache_dtype == MLA_FP8_E4M3 && !cache_scale)
    return fail(MLA_ERR_INVALID_ARGUMENT, "fp8 cache needs cache_scale");
  const size_t need = mla_append_workspace_size(dims, n_tokens);
  if (r.mfma && w_dkv_kr != nullptr && (workspace == nullptr || workspace_bytes < need))
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "append needs %zu workspace bytes, got %zu", need, workspace_bytes);
  mla::AppendArgs a{hidden, w_dkv_kr, rms_gamma, positions, slot_mapping, n_tokens, r.d_model, r.d_c,
                    r.d_r, cache_slots, r.eps, r.theta, cache, cache_scale, workspace, r.cache_dtype};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(r.mfma ? mla::launch_append_mfma(a, s) : mla::launch_append_f32(a, s), "mla_append_latent");
}

size_t mla_absorb_workspace_size(const mla_dims_t* dims, int32_t n_tokens) {
  Resolved r;
  if (resolve(dims, &r) != MLA_OK || n_tokens <= 0 || !r.mfma) return 0;
  return mla::absorb_mfma_workspace(n_tokens, r.n_h, r.cache_dtype);
}

mla_status_t mla_absorb_q(const mla_dims_t* dims, const void* q_nope, const void* q_pe,
                          const void* w_uk, const int32_t* positions, int32_t n_tokens, void* q_lat,
                          float* q_scale, void* workspace, size_t workspace_bytes,
                          mla_stream_t stream) {
  Resolved r;
  mla_status_t st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  if (n_tokens < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "n_tokens < 0");
  if (n_tokens == 0) return hip_status(hipSuccess, "");
  if (!q_nope || !w_uk || !positions || !q_lat || (r.d_r > 0 && !q_pe))
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (r.cache_dtype == MLA_FP8_E4M3 && !q_scale) return fail(MLA_ERR_INVALID_ARGUMENT, "fp8 needs q_scale");
  const size_t need = mla_absorb_workspace_size(dims, n_tokens);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "absorb needs %zu workspace bytes, got %zu", need, workspace_bytes);
  mla::AbsorbArgs a{q_nope, q_pe, w_uk, positions, n_tokens, r.n_h, r.d_h, r.d_c, r.d_r, r.theta,
                    q_lat, q_scale, workspace, r.cache_dtype};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(r.mfma ? mla::launch_absorb_q_mfma(a, s) : mla::launch_absorb_q_f32(a, s), "mla_absorb_q");
}

size_t mla_decode_workspace_size(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                 int32_t max_seq_len, int32_t split_tokens) {
  Resolved r;
  if (resolve(dims, &r) != MLA_OK || batch <= 0 || q_len <= 0 || max_seq_len < 0) return 0;
  if (!r.mfma) return 0;
  const int32_t L = split_tokens > 0 ? split_tokens : default_split(r, batch, q_len, max_seq_len);
  const int32_t splits = max_seq_len > 0 ? (max_seq_len + L - 1) / L : 1;
  return mla::decode_mfma_workspace(batch, q_len, r.n_h, splits);
}

int32_t mla_decode_default_split(const mla_dims_t* dims, int32_t batch, int32_t q_len, int32_t max_seq_len) {
  Resolved r;
  if (resolve(dims, &r) != MLA_OK || batch <= 0 || q_len <= 0 || max_seq_len < 0) return 0;
  return default_split(r, batch, q_len, max_seq_len);
}

mla_status_t mla_decode(const mla_dims_t* dims, const void* q_lat, const float* q_scale,
                        const void* cache, const float* cache_scale, const int32_t* block_table,
                        int32_t max_blocks_per_seq, int32_t num_blocks, const int32_t* seq_lens,
                        int32_t batch, int32_t q_len, int32_t max_seq_len, int32_t split_tokens,
                        void* workspace, size_t workspace_bytes, void* o_lat, float* lse,
                        mla_stream_t stream) {
  Resolved r;
  mla_status_t st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  if (batch < 0 || q_len <= 0 || max_seq_len < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "bad sizes (batch %d q_len %d max_seq_len %d max_blocks %d num_blocks %d)",
                batch, q_len, max_seq_len, max_blocks_per_seq, num_blocks);
  if (batch == 0) return hip_status(hipSuccess, "");
  if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_blocks_per_seq) * r.bs)
    return fail(MLA_ERR_INVALID_ARGUMENT, "max_seq_len %d exceeds max_blocks_per_seq*block_size", max_seq_len);
  if (!q_lat || !cache || !block_table || !seq_lens || !o_lat)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (r.cache_dtype == MLA_FP8_E4M3 && (!q_scale || !cache_scale))
    return fail(MLA_ERR_INVALID_ARGUMENT, "fp8 decode needs q_scale and cache_scale");
  if (r.mfma && q_len > 2) return fail(MLA_ERR_UNSUPPORTED, "bf16/fp8 decode supports q_len <= 2");
  if (split_tokens < 0 || (r.mfma && split_tokens % 64 != 0))
    return fail(MLA_ERR_INVALID_ARGUMENT, "split_tokens must be 0 or a positive multiple of 64");
  hipStream_t s = static_cast<hipStream_t>(stream);
  mla::DecodeArgs a{};
  a.q_lat = q_lat;
  a.q_scale = q_scale;
  a.cache = cache;
  a.cache_scale = cache_scale;
  a.block_table = block_table;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.q_len = q_len;
  a.n_h = r.n_h;
  a.d_c = r.d_c;
  a.d_r = r.d_r;
  a.block_size = r.bs;
  a.max_seq_len = max_seq_len;
  a.scale = r.scale;
  a.o_lat = o_lat;
  a.lse = lse;
  a.cache_dtype = r.cache_dtype;
  if (!r.mfma) return hip_status(mla::launch_decode_f32(a, s), "mla_decode");
  a.split_tokens = split_tokens > 0 ? split_tokens : default_split(r, batch, q_len, max_seq_len);
  a.num_splits = max_seq_len > 0 ? (max_seq_len + a.split_tokens - 1) / a.split_tokens : 1;
  const size_t need = mla::decode_mfma_workspace(batch, q_len, r.n_h, a.num_splits);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "decode needs %zu workspace bytes, got %zu", need, workspace_bytes);
  a.workspace = workspace;
  return hip_status(r.cache_dtype == MLA_FP8_E4M3 ? mla::launch_decode_fp8(a, s) : mla::launch_decode_mfma(a, s),
                    "mla_decode");
}

mla_status_t mla_out_proj(const mla_dims_t* dims, const void* o_lat, const void* w_uv,
                          int32_t n_tokens, void* out, mla_stream_t stream) {
  Resolved r;
  mla_status_t st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  if (n_tokens < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "n_tokens < 0");
  if (n_tokens == 0) return hip_status(hipSuccess, "");
  if (!o_lat || !w_uv || !out) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  mla::OutProjArgs a{o_lat, w_uv, n_tokens, r.n_h, r.d_c, r.d_v, out};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(r.mfma ? mla::launch_out_proj_mfma(a, s) : mla::launch_out_proj_f32(a, s), "mla_out_proj");
}

mla_status_t mla_prefill_attention(const mla_dims_t* dims, const void* q_nope, const void* q_pe,
                                   const void* k_nope, const void* k_rope, int32_t k_rope_stride,
                                   const void* v, int32_t seq_len, void* out, float* lse, mla_stream_t stream) {
  Resolved r;
  mla_status_t st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  if (!r.mfma || r.act_dtype != MLA_BF16 || r.cache_dtype != MLA_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "prefill attention needs the bf16 MFMA dims (d_h = d_v = 128, d_R = 64)");
  if (seq_len < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "seq_len < 0");
  if (seq_len == 0) return hip_status(hipSuccess, "");
  if (!q_nope || !q_pe || !k_nope || !k_rope || !v || !out)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (k_rope_stride < r.d_r || k_rope_stride % 8 != 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "k_rope_stride must be >= d_R and a multiple of 8 (got %d)", k_rope_stride);
  mla::PrefillArgs a{q_nope, q_pe, k_nope, k_rope, k_rope_stride, v, seq_len, r.n_h, r.scale, r.theta, out, lse};
  return hip_status(mla::launch_prefill_attention(a, static_cast<hipStream_t>(stream)), "mla_prefill_attention");
}

size_t mla_linear_workspace_size(int32_t m, int32_t n, int32_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || n % 128 != 0 || k % 16 != 0) return 0;
  return mla::linear_workspace(m, n, k);
}

mla_status_t mla_linear(const void* x, int32_t ldx, const void* w, int32_t m, int32_t n, int32_t k, void* y,
                        void* workspace, size_t workspace_bytes, mla_stream_t stream) {
  if (m < 0 || n <= 0 || k <= 0) return fail(MLA_ERR_INVALID_ARGUMENT, "m < 0 or n, k <= 0");
  if (ldx < k || ldx % 8 != 0) return fail(MLA_ERR_INVALID_ARGUMENT, "ldx must be >= k and a multiple of 8 (got %d)", ldx);
  if (n % 128 != 0 || k % 16 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "linear needs n %% 128 == 0 and k %% 16 == 0 (got n=%d, k=%d)", n, k);
  if (m == 0) return hip_status(hipSuccess, "");
  if (!x || !w || !y) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  const size_t need = mla_linear_workspace_size(m, n, k);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "linear needs %zu workspace bytes, got %zu", need, workspace_bytes);
  mla::LinearArgs a{x, w, m, n, k, ldx, y, workspace};
  return hip_status(mla::launch_linear(a, static_cast<hipStream_t>(stream)), "mla_linear");
}

const char* mla_status_string(mla_status_t status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARGUMENT: return "MLA_ERR_INVALID_ARGUMENT";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error_message(void) { return g_err; }

int32_t mla_version(void) { return 200; }

}  // extern "C"
