// C-ABI entry points of libmla: argument checks on the host, kernel
// selection, launch, HIP error mapping.  No device memory is allocated here.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/mla.h"
#include "kernels.h"
#include "plan.h"

// Scratch of mla_decode_uniform_noalloc: the split partials of a decode,
// for callers that cannot allocate.  One copy per GPU, held until the
// process ends.  Host code never uses the array's name as an address (it is
// a host-side stand-in); it uses the per-device address from
// hipGetSymbolAddress below.
constexpr size_t kStaticScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

thread_local char g_err[512] = "";

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_addr[dev] = ptr;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

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

// Stored bytes of one cache row of D = d_c + d_R elements.
size_t row_bytes(int dt, int d_c, int d_r) {
  const size_t D = static_cast<size_t>(d_c) + d_r;
  switch (dt) {
    case MLA_F32: return 4 * D;
    case MLA_BF16: return 2 * D;
    case MLA_FP8_E4M3: return D;
    case MLA_FP4_E2M1: return (D / 2 + D / 32 + 15) / 16 * 16;  // codes, E8M0 scales, padding
    case MLA_FP8_E4M3_KR_BF16: return static_cast<size_t>(d_c) + 2 * static_cast<size_t>(d_r);
  }
  return 0;
}

// Decode kernels for the cache format.
hipError_t launch_decode_for(const Resolved& r, const mla::DecodeArgs& a, hipStream_t s) {
  switch (r.cache_dtype) {
    case MLA_FP8_E4M3: return mla::launch_decode_fp8(a, s);
    case MLA_FP4_E2M1: return mla::launch_decode_dq(a, mla::kDqFp4Mx, s);
    case MLA_FP8_E4M3_KR_BF16: return mla::launch_decode_dq(a, mla::kDqFp8Kr, s);
  }
  return r.d_r == 0 ? mla::launch_decode_dq(a, mla::kDqBf16Nope, s) : mla::launch_decode_mfma(a, s);
}

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
  const bool known = r->cache_dtype == MLA_BF16 || r->cache_dtype == MLA_FP8_E4M3 ||
                     r->cache_dtype == MLA_FP4_E2M1 || r->cache_dtype == MLA_FP8_E4M3_KR_BF16;
  if (known && r->act_dtype == MLA_BF16) {
    // d_R = 0 (no decoupled RoPE part) on the bf16 cache only
    const bool rope_ok = r->d_r == 64 || (r->d_r == 0 && r->cache_dtype == MLA_BF16);
    if (r->d_c != 512 || !rope_ok || r->d_h != 128 || r->d_v != 128)
      return fail(MLA_ERR_UNSUPPORTED,
                  "MFMA kernels need d_c=512, d_h=d_v=128 and d_R=64 (or d_R=0 with a bf16 cache) (got %d,%d,%d,%d)",
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

mla::PlanShape plan_shape(const Resolved& r, int32_t q_len) {
  mla::PlanShape sh;
  if (!r.mfma) {
    sh.row_groups = 1;
    sh.resident_per_xcd = 32;
    return sh;
  }
  const int waves = mla::decode_waves_per_group(r.n_h, q_len);
  sh.row_groups = q_len * r.n_h / (32 * waves);
  sh.resident_per_xcd = 32 * (4 / waves);  // one wave per SIMD: 1 or 2 workgroups per CU
  return sh;
}

int64_t partial_bytes(const Resolved& r, int32_t q_len, int64_t num_partials) {
  if (!r.mfma) return 0;
  const int64_t rows = num_partials * q_len * r.n_h;
  return rows * 512 * 2 + rows * 4;  // bf16 partial rows, fp32 lse
}

// Everything a plan stands for, except the hash itself.
uint64_t plan_hash(const mla_dims_t* d, const mla_plan_t* p) {
  uint64_t h = 0xcbf29ce484222325ull;
  h = mla::fnv1a(h, d, sizeof(*d));
  const int32_t f[] = {p->batch, p->q_len, p->num_items, p->max_splits, p->split_tokens, p->max_seq_len,
                       p->num_slots, p->num_partials};
  h = mla::fnv1a(h, f, sizeof(f));
  const uint64_t g[] = {static_cast<uint64_t>(p->workspace_bytes), static_cast<uint64_t>(p->image_bytes),
                        p->seq_digest, p->workspace};
  return mla::fnv1a(h, g, sizeof(g));
}

// Validates a plan request and builds it on the host.
mla_status_t make_plan(const mla_dims_t* dims, const int32_t* seq_lens_host, int32_t batch, int32_t q_len,
                       int32_t hint, Resolved* r, mla::PlanResult* res, mla::PlanLayout* lay) {
  mla_status_t st = resolve(dims, r);
  if (st != MLA_OK) return st;
  if (batch < 0 || q_len <= 0) return fail(MLA_ERR_INVALID_ARGUMENT, "bad sizes (batch %d q_len %d)", batch, q_len);
  if (batch > 0 && seq_lens_host == nullptr) return fail(MLA_ERR_INVALID_ARGUMENT, "seq_lens_host is NULL");
  if (batch >= (1 << 24)) return fail(MLA_ERR_UNSUPPORTED, "batch must be below 2^24");
  if (r->mfma && q_len > 2) return fail(MLA_ERR_UNSUPPORTED, "bf16/fp8 decode supports q_len <= 2");
  if (hint < 0 || (hint > 0 && hint % 64 != 0))
    return fail(MLA_ERR_INVALID_ARGUMENT, "split_tokens_hint must be 0 or a positive multiple of 64");
  for (int32_t b = 0; b < batch; ++b)
    if (seq_lens_host[b] < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "seq_lens_host[%d] = %d < 0", b, seq_lens_host[b]);
  const mla::PlanShape sh = plan_shape(*r, q_len);
  int32_t L = hint;
  if (!r->mfma) {  // the fp32 kernel makes one pass per request
    int32_t mx = 64;
    for (int32_t b = 0; b < batch; ++b) mx = seq_lens_host[b] > mx ? seq_lens_host[b] : mx;
    L = (mx + 63) / 64 * 64;
  } else if (L == 0) {
    L = mla::choose_split(seq_lens_host, batch, sh);
  }
  if (!mla::build_plan(seq_lens_host, batch, sh, L, res)) return fail(MLA_ERR_INVALID_ARGUMENT, "planning failed");
  *lay = mla::plan_layout(batch, res->num_slots, partial_bytes(*r, q_len, res->num_partials));
  return MLA_OK;
}

}  // namespace

extern "C" {

size_t mla_cache_row_bytes(const mla_dims_t* dims) {
  // a pure size helper: defined for any positive dims, kernel support aside
  if (dims == nullptr || dims->kv_lora_rank <= 0 || dims->qk_rope_head_dim < 0) return 0;
  return row_bytes(dims->cache_dtype, dims->kv_lora_rank, dims->qk_rope_head_dim);
}

size_t mla_cache_bytes_per_token(const mla_dims_t* dims) {
  const size_t row = mla_cache_row_bytes(dims);
  const bool scaled = dims != nullptr && (dims->cache_dtype == MLA_FP8_E4M3 || dims->cache_dtype == MLA_FP8_E4M3_KR_BF16);
  return row > 0 && scaled ? row + sizeof(float) : row;
}

size_t mla_q_lat_row_bytes(const mla_dims_t* dims) {
  if (mla_cache_row_bytes(dims) == 0) return 0;
  const size_t D = static_cast<size_t>(dims->kv_lora_rank) + dims->qk_rope_head_dim;
  switch (dims->cache_dtype) {
    case MLA_F32: return 4 * D;
    case MLA_FP8_E4M3: return 2 * D;  // two e4m3 planes
    default: return 2 * D;            // bf16 (also for the FP4 and FP8-KR caches)
  }
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
  if ((r.cache_dtype == MLA_FP8_E4M3 || r.cache_dtype == MLA_FP8_E4M3_KR_BF16) && !cache_scale)
    return fail(MLA_ERR_INVALID_ARGUMENT, "fp8 cache needs cache_scale");
  const size_t need = mla_append_workspace_size(dims, n_tokens);
  if (r.mfma && w_dkv_kr != nullptr && (workspace == nullptr || workspace_bytes < need))
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "append needs %zu workspace bytes, got %zu", need, workspace_bytes);
  mla::AppendArgs a{hidden, w_dkv_kr, rms_gamma, positions, slot_mapping, n_tokens, r.d_model, r.d_c,
                    r.d_r, cache_slots, r.eps, r.theta, cache, cache_scale, workspace, r.cache_dtype};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(r.mfma ? mla::launch_append_mfma(a, s) : mla::launch_append_f32(a, s), "mla_append_latent");
}

size_t mla_append_absorb_workspace_size(const mla_dims_t* dims, int32_t n_tokens, int32_t n_q_tokens) {
  const size_t a = (mla_append_workspace_size(dims, n_tokens) + 255) / 256 * 256;
  return a + mla_absorb_workspace_size(dims, n_q_tokens);
}

mla_status_t mla_append_absorb(const mla_dims_t* dims, const void* hidden, const void* w_dkv_kr,
                               const float* rms_gamma, const int32_t* positions, const int64_t* slot_mapping,
                               int32_t n_tokens, int64_t cache_slots, void* cache, float* cache_scale,
                               const void* q_nope, const void* q_pe, const void* w_uk,
                               const int32_t* q_positions, int32_t n_q_tokens, void* q_lat, float* q_scale,
                               void* workspace, size_t workspace_bytes, mla_stream_t stream) {
  Resolved r;
  mla_status_t st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  const size_t need = mla_append_absorb_workspace_size(dims, n_tokens, n_q_tokens);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "append + absorb needs %zu workspace bytes, got %zu", need,
                workspace_bytes);
  const size_t a_bytes = (mla_append_workspace_size(dims, n_tokens) + 255) / 256 * 256;
  char* ws = static_cast<char*>(workspace);
  void* q_ws = mla_absorb_workspace_size(dims, n_q_tokens) > 0 ? ws + a_bytes : nullptr;
  // one fused launch on the MFMA path with both calls doing work; otherwise the two calls in order
  if (!r.mfma || w_dkv_kr == nullptr || n_tokens <= 0 || n_q_tokens <= 0) {
    st = mla_append_latent(dims, hidden, w_dkv_kr, rms_gamma, positions, slot_mapping, n_tokens, cache_slots, cache,
                           cache_scale, workspace, a_bytes, stream);
    if (st != MLA_OK) return st;
    return mla_absorb_q(dims, q_nope, q_pe, w_uk, q_positions, n_q_tokens, q_lat, q_scale, q_ws,
                        mla_absorb_workspace_size(dims, n_q_tokens), stream);
  }
  if (!hidden || !rms_gamma || !positions || !slot_mapping || !cache || !q_nope || !w_uk || !q_positions ||
      !q_lat || (r.d_r > 0 && !q_pe))
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (cache_slots <= 0) return fail(MLA_ERR_INVALID_ARGUMENT, "cache_slots must be positive");
  if ((r.cache_dtype == MLA_FP8_E4M3 || r.cache_dtype == MLA_FP8_E4M3_KR_BF16) && !cache_scale)
    return fail(MLA_ERR_INVALID_ARGUMENT, "fp8 cache needs cache_scale");
  if (r.cache_dtype == MLA_FP8_E4M3 && !q_scale) return fail(MLA_ERR_INVALID_ARGUMENT, "fp8 needs q_scale");
  mla::AppendArgs a{hidden, w_dkv_kr, rms_gamma, positions, slot_mapping, n_tokens, r.d_model, r.d_c,
                    r.d_r, cache_slots, r.eps, r.theta, cache, cache_scale, workspace, r.cache_dtype};
  mla::AbsorbArgs q{q_nope, q_pe, w_uk, q_positions, n_q_tokens, r.n_h, r.d_h, r.d_c, r.d_r, r.theta,
                    q_lat, q_scale, q_ws, r.cache_dtype};
  return hip_status(mla::launch_append_absorb_mfma(a, q, static_cast<hipStream_t>(stream)), "mla_append_absorb");
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

size_t mla_decode_uniform_workspace_size(const mla_dims_t* dims, int32_t batch, int32_t q_len,
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

mla_status_t mla_decode_uniform(const mla_dims_t* dims, const void* q_lat, const float* q_scale,
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
  if (r.cache_dtype == MLA_FP8_E4M3_KR_BF16 && !cache_scale)
    return fail(MLA_ERR_INVALID_ARGUMENT, "the fp8 latent needs cache_scale");
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
  return hip_status(launch_decode_for(r, a, s), "mla_decode_uniform");
}

mla_status_t mla_decode_uniform_noalloc(const mla_dims_t* dims, const void* q_lat, const float* q_scale,
                                        const void* cache, const float* cache_scale, const int32_t* block_table,
                                        int32_t max_blocks_per_seq, int32_t num_blocks, const int32_t* seq_lens,
                                        int32_t batch, int32_t q_len, int32_t max_seq_len, int32_t split_tokens,
                                        void* o_lat, float* lse, mla_stream_t stream) {
  // the sizes first, so that an oversized call fails before any HIP call
  Resolved r;
  mla_status_t st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  const size_t need = mla_decode_uniform_workspace_size(dims, batch, q_len, max_seq_len, split_tokens);
  if (need > kStaticScratchBytes)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                "the decode needs %zu bytes of split partials; the static scratch of "
                "mla_decode_uniform_noalloc holds %zu (use mla_decode_uniform with a workspace)",
                need, kStaticScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    st = hip_status(static_scratch(&ws), "mla_decode_uniform_noalloc (scratch address)");
    if (st != MLA_OK) return st;
  }
  return mla_decode_uniform(dims, q_lat, q_scale, cache, cache_scale, block_table, max_blocks_per_seq, num_blocks,
                            seq_lens, batch, q_len, max_seq_len, split_tokens, ws, need, o_lat, lse, stream);
}

size_t mla_decode_plan_workspace_size(const mla_dims_t* dims, const int32_t* seq_lens_host, int32_t batch,
                                      int32_t q_len, int32_t split_tokens_hint) {
  Resolved r;
  mla::PlanResult res;
  mla::PlanLayout lay;
  if (make_plan(dims, seq_lens_host, batch, q_len, split_tokens_hint, &r, &res, &lay) != MLA_OK) return 0;
  return lay.total;
}

mla_status_t mla_decode_plan_host(const mla_dims_t* dims, const int32_t* seq_lens_host, int32_t batch,
                                  int32_t q_len, int32_t split_tokens_hint, const void* workspace,
                                  mla_plan_t* plan, void* host_image, size_t host_image_bytes) {
  if (plan == nullptr) return fail(MLA_ERR_INVALID_ARGUMENT, "plan is NULL");
  Resolved r;
  mla::PlanResult res;
  mla::PlanLayout lay;
  mla_status_t st = make_plan(dims, seq_lens_host, batch, q_len, split_tokens_hint, &r, &res, &lay);
  if (st != MLA_OK) return st;
  mla_plan_t p{};
  p.batch = batch;
  p.q_len = q_len;
  p.num_items = res.num_items;
  p.max_splits = res.max_splits;
  p.workspace_bytes = lay.total;
  p.image_bytes = lay.partials;
  p.split_tokens = res.split_tokens;
  p.max_seq_len = res.max_seq_len;
  p.num_slots = res.num_slots;
  p.num_partials = res.num_partials;
  p.seq_digest = mla::fnv1a(0xcbf29ce484222325ull, seq_lens_host, sizeof(int32_t) * static_cast<size_t>(batch));
  p.workspace = static_cast<uint64_t>(reinterpret_cast<uintptr_t>(workspace));
  p.hash = plan_hash(dims, &p);
  if (host_image != nullptr) {
    if (host_image_bytes < lay.partials)
      return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "the work-list image needs %zu bytes, got %zu", lay.partials,
                  host_image_bytes);
    unsigned char* img = static_cast<unsigned char*>(host_image);
    memset(img, 0, lay.partials);
    memcpy(img, "MLAPLAN1", 8);
    memcpy(img + 8, &p.hash, 8);
    if (!res.list.empty()) memcpy(img + lay.list, res.list.data(), res.list.size() * 4);
    memcpy(img + lay.part_ptr, res.part_ptr.data(), res.part_ptr.size() * 4);
  }
  *plan = p;
  g_err[0] = '\0';
  return MLA_OK;
}

mla_status_t mla_decode_plan(const mla_dims_t* dims, const int32_t* seq_lens_host, int32_t batch, int32_t q_len,
                             int32_t split_tokens_hint, mla_plan_t* plan, void* workspace, size_t workspace_bytes,
                             mla_stream_t stream) {
  if (plan == nullptr) return fail(MLA_ERR_INVALID_ARGUMENT, "plan is NULL");
  mla_plan_t p{};
  mla_status_t st = mla_decode_plan_host(dims, seq_lens_host, batch, q_len, split_tokens_hint, workspace, &p,
                                         nullptr, 0);
  if (st != MLA_OK) return st;
  if (workspace == nullptr || workspace_bytes < p.workspace_bytes)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "decode plan needs %zu workspace bytes, got %zu", p.workspace_bytes,
                workspace_bytes);
  std::vector<unsigned char> host(p.image_bytes);
  st = mla_decode_plan_host(dims, seq_lens_host, batch, q_len, split_tokens_hint, workspace, &p, host.data(),
                            host.size());
  if (st != MLA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(workspace, host.data(), host.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // the host image is freed on return
  st = hip_status(e, "mla_decode_plan");
  if (st == MLA_OK) *plan = p;
  return st;
}

mla_status_t mla_decode(const mla_dims_t* dims, const mla_plan_t* plan, const void* q_lat, const float* q_scale,
                        const void* cache, const float* cache_scale, const int32_t* block_table,
                        int32_t max_blocks_per_seq, int32_t num_blocks, const int32_t* seq_lens, void* workspace,
                        size_t workspace_bytes, void* o_lat, float* lse, mla_stream_t stream) {
  Resolved r;
  mla_status_t st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  if (plan == nullptr) return fail(MLA_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (plan_hash(dims, plan) != plan->hash)
    return fail(MLA_ERR_PLAN_MISMATCH, "the plan was made for other dims or has been modified");
  if (static_cast<uint64_t>(reinterpret_cast<uintptr_t>(workspace)) != plan->workspace)
    return fail(MLA_ERR_PLAN_MISMATCH, "the plan's work list is in another workspace");
  if (workspace_bytes < plan->workspace_bytes)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "decode needs %zu workspace bytes, got %zu", plan->workspace_bytes,
                workspace_bytes);
  if (max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "bad sizes (max_blocks %d num_blocks %d)", max_blocks_per_seq, num_blocks);
  if (plan->batch == 0) return hip_status(hipSuccess, "");
  if (static_cast<int64_t>(plan->max_seq_len) > static_cast<int64_t>(max_blocks_per_seq) * r.bs)
    return fail(MLA_ERR_INVALID_ARGUMENT, "planned length %d exceeds max_blocks_per_seq*block_size", plan->max_seq_len);
  if (!q_lat || !cache || !block_table || !seq_lens || !o_lat)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (r.cache_dtype == MLA_FP8_E4M3 && (!q_scale || !cache_scale))
    return fail(MLA_ERR_INVALID_ARGUMENT, "fp8 decode needs q_scale and cache_scale");
  if (r.cache_dtype == MLA_FP8_E4M3_KR_BF16 && !cache_scale)
    return fail(MLA_ERR_INVALID_ARGUMENT, "the fp8 latent needs cache_scale");
  const mla::PlanLayout lay = mla::plan_layout(plan->batch, plan->num_slots,
                                               partial_bytes(r, plan->q_len, plan->num_partials));
  char* ws = static_cast<char*>(workspace);
  mla::DecodeArgs a{};
  a.q_lat = q_lat;
  a.q_scale = q_scale;
  a.cache = cache;
  a.cache_scale = cache_scale;
  a.block_table = block_table;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.seq_lens = seq_lens;
  a.batch = plan->batch;
  a.q_len = plan->q_len;
  a.n_h = r.n_h;
  a.d_c = r.d_c;
  a.d_r = r.d_r;
  a.block_size = r.bs;
  a.max_seq_len = plan->max_seq_len;
  a.scale = r.scale;
  a.o_lat = o_lat;
  a.lse = lse;
  a.cache_dtype = r.cache_dtype;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!r.mfma) return hip_status(mla::launch_decode_f32(a, s), "mla_decode");
  a.split_tokens = plan->split_tokens;
  a.num_splits = plan->max_splits;
  a.items = reinterpret_cast<const int32_t*>(ws + lay.list);
  a.part_ptr = reinterpret_cast<const int32_t*>(ws + lay.part_ptr);
  a.num_slots = plan->num_slots;
  a.num_partials = plan->num_partials;
  a.workspace = ws + lay.partials;
  return hip_status(launch_decode_for(r, a, s), "mla_decode");
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
  mla::PrefillArgs a{q_nope, q_pe, k_nope, k_rope, k_rope_stride, v, seq_len, r.n_h, r.scale, r.theta, out, lse,
                     nullptr, nullptr, 1, seq_len};
  return hip_status(mla::launch_prefill_attention(a, static_cast<hipStream_t>(stream)), "mla_prefill_attention");
}

mla_status_t mla_prefill_attention_varlen(const mla_dims_t* dims, const void* q_nope, const void* q_pe,
                                          const void* k_nope, const void* k_rope, int32_t k_rope_stride,
                                          const void* v, const int32_t* cu_q, const int32_t* cu_k,
                                          int32_t num_seqs, int32_t max_q, int32_t total_q, void* out,
                                          float* lse, mla_stream_t stream) {
  Resolved r;
  mla_status_t st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  if (!r.mfma || r.act_dtype != MLA_BF16 || r.cache_dtype != MLA_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "prefill attention needs the bf16 MFMA dims (d_h = d_v = 128, d_R = 64)");
  if (num_seqs < 0 || max_q < 0 || total_q < 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "num_seqs, max_q and total_q must be >= 0");
  if (num_seqs >= 65536) return fail(MLA_ERR_UNSUPPORTED, "num_seqs must be below 65536");
  if (num_seqs == 0 || max_q == 0) return hip_status(hipSuccess, "");
  if (!q_nope || !q_pe || !k_nope || !k_rope || !v || !out || !cu_q || !cu_k)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (k_rope_stride < r.d_r || k_rope_stride % 8 != 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "k_rope_stride must be >= d_R and a multiple of 8 (got %d)", k_rope_stride);
  mla::PrefillArgs a{q_nope, q_pe, k_nope, k_rope, k_rope_stride, v, total_q, r.n_h, r.scale, r.theta, out, lse,
                     cu_q, cu_k, num_seqs, max_q};
  return hip_status(mla::launch_prefill_attention(a, static_cast<hipStream_t>(stream)),
                    "mla_prefill_attention_varlen");
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

mla_status_t mla_linear_pair(const void* x, int32_t ldx, int32_t m, int32_t k, const void* w1, int32_t n1, void* y1,
                             const void* w2, int32_t n2, void* y2, void* workspace, size_t workspace_bytes,
                             mla_stream_t stream) {
  if (m < 0 || n1 <= 0 || n2 <= 0 || k <= 0) return fail(MLA_ERR_INVALID_ARGUMENT, "m < 0 or n1, n2, k <= 0");
  if (ldx < k || ldx % 8 != 0) return fail(MLA_ERR_INVALID_ARGUMENT, "ldx must be >= k and a multiple of 8 (got %d)", ldx);
  if (n1 % 128 != 0 || n2 % 128 != 0 || k % 16 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "linear pair needs n1, n2 %% 128 == 0 and k %% 16 == 0 (got %d, %d, %d)", n1, n2, k);
  if (m == 0) return hip_status(hipSuccess, "");
  if (!x || !w1 || !y1 || !w2 || !y2) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  const size_t need = mla_linear_workspace_size(m, n1 + n2, k);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "linear pair needs %zu workspace bytes, got %zu", need, workspace_bytes);
  mla::LinearArgs a{x, w1, m, n1, k, ldx, y1, workspace};
  return hip_status(mla::launch_linear_pair(a, w2, n2, y2, static_cast<hipStream_t>(stream)), "mla_linear_pair");
}

mla_status_t mla_absorb_output_weights(const mla_dims_t* dims, const void* w_o, const void* w_uv, void* b,
                                       mla_stream_t stream) {
  Resolved r;
  mla_status_t st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  if (!w_o || !w_uv || !b) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  // B_i[m, c] = sum_k W^O[m, i*d_v + k] W^UV[i, k, c]
  mla::FoldArgs a{w_o, w_uv, b, r.n_h, r.d_model, r.d_c, r.d_v,
                  r.d_v, static_cast<int64_t>(r.n_h) * r.d_v, 1,
                  static_cast<int64_t>(r.d_v) * r.d_c, r.d_c, 1,
                  r.d_c, static_cast<int64_t>(r.n_h) * r.d_c, 1};
  return hip_status(mla::launch_fold(a, r.act_dtype == MLA_BF16, static_cast<hipStream_t>(stream)),
                    "mla_absorb_output_weights");
}

mla_status_t mla_absorb_query_weights(const mla_dims_t* dims, int32_t d_cq, const void* w_uq, const void* w_uk,
                                      void* a_out, mla_stream_t stream) {
  Resolved r;
  mla_status_t st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  if (d_cq <= 0) return fail(MLA_ERR_INVALID_ARGUMENT, "d_cq must be positive");
  if (!w_uq || !w_uk || !a_out) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  // A_i[c, m] = sum_k W^UK[i, k, c] W^UQ[i*d_h + k, m]
  mla::FoldArgs a{w_uk, w_uq, a_out, r.n_h, r.d_c, d_cq, r.d_h,
                  static_cast<int64_t>(r.d_h) * r.d_c, 1, r.d_c,
                  static_cast<int64_t>(r.d_h) * d_cq, d_cq, 1,
                  static_cast<int64_t>(r.d_c) * d_cq, d_cq, 1};
  return hip_status(mla::launch_fold(a, r.act_dtype == MLA_BF16, static_cast<hipStream_t>(stream)),
                    "mla_absorb_query_weights");
}

mla_status_t mla_hbm_read_probe(const void* buf, size_t bytes, int32_t mode, uint32_t* sink, size_t sink_words,
                                mla_stream_t stream) {
  if (!buf) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL buffer");
  if (mode == 0) {
    if (bytes % 16 != 0) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes must be a multiple of 16 (mode 0)");
    if (!sink || sink_words < static_cast<size_t>(mla::kProbeRegsGrid))
      return fail(MLA_ERR_INVALID_ARGUMENT, "mode 0 needs a sink of at least %d words", mla::kProbeRegsGrid);
  } else if (mode == 1) {
    if (bytes % 36864 != 0) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes must be a multiple of 36864 (mode 1)");
  } else {
    return fail(MLA_ERR_INVALID_ARGUMENT, "mode must be 0 or 1");
  }
  if (bytes == 0) return hip_status(hipSuccess, "");
  return hip_status(mla::launch_hbm_read_probe(buf, bytes, mode, sink, static_cast<hipStream_t>(stream)),
                    "mla_hbm_read_probe");
}

const char* mla_status_string(mla_status_t status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARGUMENT: return "MLA_ERR_INVALID_ARGUMENT";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
    case MLA_ERR_PLAN_MISMATCH: return "MLA_ERR_PLAN_MISMATCH";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error_message(void) { return g_err; }

int32_t mla_version(void) { return 300; }

}  // extern "C"
