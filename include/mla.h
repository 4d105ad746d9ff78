/*
 * libmla -- Multi-head Latent Attention (MLA) decode over a compressed
 * latent KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The method (pages on MLA; cited by page and section):
 *   [MLA explainer]  disassemble-channel.com, "Multi-head Latent Attention
 *                    （MLA）とは？KVキャッシュを圧縮するDeepSeekの注意機構を完全解説"
 *   [V2 summary]     abeam.tech, DeepSeek-V2 paper summary (MLA / KV cache)
 *   [variants]       youngju.dev, model internals: attention variants (ja)
 *
 * One decode step of one layer is four calls, in the order of the inference
 * flow of [V2 summary, "推論方法" (inference) section]:
 *
 *   mla_append_latent  h -> [W^DKV h ; W^KR h] -> RMSNorm on the latent,
 *                      RoPE on k^R -> write the row into a paged cache
 *   mla_absorb_q       q~_i = W^UK_i^T q^C_i (latent query), RoPE on q^R
 *   mla_decode         scores over [c^KV ; k^R], softmax, latent-weighted sum
 *                      (split over the context, then a combine kernel)
 *   mla_out_proj       o_i = W^UV_i o_lat_i
 *   mla_linear         the dense projections around them (query path
 *                      W^DQ, W^UQ, W^QR; output W^O or the absorbed B_i;
 *                      prefill keys and values W^UK c, W^UV c)
 *   mla_prefill_attention  the prompt's causal attention with per-head
 *                      keys and values (no absorption)
 *
 * Conventions
 *   - All tensors are dense row-major; every pointer argument except those
 *     marked "host" is a device pointer.  The caller owns all memory,
 *     including the workspaces; libmla never allocates or frees device
 *     memory and keeps no mutable global state.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronise the host.
 *   - Errors: every entry point checks its arguments on the host before any
 *     launch and returns a status; nothing is thrown across the ABI.  The
 *     text of the last error of the calling thread is returned by
 *     mla_last_error_message().  Device faults surface at the caller's next
 *     synchronisation.  Values inside device arrays (positions, slots,
 *     sequence lengths, block-table entries) cannot be checked on the host;
 *     their contracts are stated per call, and kernels clamp or skip
 *     out-of-range values so that no access leaves the arrays given.
 *   - Token order: new token n of a step is request b = n / q_len, query
 *     t = n % q_len; query t of a request with T cached rows (rows appended
 *     this step included) is at position T - q_len + t and attends to keys
 *     0 .. T - q_len + t (causal within the step).
 *   - Cache row layout: d_c latent elements followed by d_R RoPE-key
 *     elements ([MLA explainer, decoupled RoPE section]: the cache holds
 *     c^KV and the RoPE'd shared key k^R).  The pool is
 *     [num_blocks, block_size, d_c + d_R]; slot s = block * block_size + offset.
 *   - Supported dtype combinations (cache_dtype / act_dtype):
 *       MLA_F32 / MLA_F32   any dims (portable fp32 kernels)
 *       MLA_BF16 / MLA_BF16 d_c = 512, d_R = 64, d_h = d_v = 128,
 *                           num_heads a multiple of 64, q_len in {1, 2},
 *                           block_size a multiple of 64 (MFMA kernels)
 *       MLA_FP8_E4M3 / MLA_BF16  same dims as bf16; the cache stores OCP
 *                           e4m3 codes with one fp32 scale per row (token)
 *     Anything else returns MLA_ERR_UNSUPPORTED.
 */
#ifndef LIBMLA_MLA_H
#define LIBMLA_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1,
  MLA_ERR_UNSUPPORTED = 2,
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,
  MLA_ERR_HIP = 4
} mla_status_t;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1, MLA_FP8_E4M3 = 2 } mla_dtype_t;

/* A hipStream_t (kept opaque so the header needs no HIP include). */
typedef void* mla_stream_t;

/* Model dimensions.  Field names follow the model-config vocabulary of
 * [variants, MLA section]: kv_lora_rank = d_c, qk_rope_head_dim = d_R. */
typedef struct {
  int32_t num_heads;         /* n_h */
  int32_t kv_lora_rank;      /* d_c, latent width [MLA explainer eq.(2)] */
  int32_t qk_nope_head_dim;  /* d_h, per-head content query/key width */
  int32_t qk_rope_head_dim;  /* d_R, decoupled RoPE width (even) */
  int32_t v_head_dim;        /* d_v */
  int32_t hidden_size;       /* d_model */
  int32_t block_size;        /* tokens per cache block */
  int32_t cache_dtype;       /* mla_dtype_t of the cache and of q_lat */
  int32_t act_dtype;         /* mla_dtype_t of hidden, weights, q_nope, q_pe,
                                o_lat and out */
  float softmax_scale;       /* <= 0 selects 1/sqrt(d_h + d_R)
                                [MLA explainer, decoupled RoPE section] */
  float rope_theta;          /* <= 0 selects 10000 */
  float rms_eps;             /* <= 0 selects 1e-6 */
} mla_dims_t;

/* Bytes of one cache row: (d_c + d_R) * element size.  fp8 caches keep the
 * per-row fp32 scale in a separate [num_blocks, block_size] array.
 * Returns 0 for invalid dims.  [MLA explainer, cache comparison section;
 * variants, MLA section: per-token elements = d_c + d_R per layer.] */
size_t mla_cache_row_bytes(const mla_dims_t* dims);

/* Bytes of one latent-query row q_lat[n, i] as mla_absorb_q writes it and
 * mla_decode reads it: (d_c + d_R) * element size for fp32 / bf16; for an
 * fp8 cache two e4m3 planes of d_c + d_R codes each (see mla_absorb_q).
 * Returns 0 for invalid dims. */
size_t mla_q_lat_row_bytes(const mla_dims_t* dims);

/* ---------------------------------------------------------------- append
 * New cache rows [MLA explainer: low-rank section eq.(2), decoupled RoPE
 * section eq.(15), trade-offs section (normalisation of the latent);
 * variants, trade-off section (RMSNorm after the compressed latent)]:
 *   kv  = [W^DKV ; W^KR] h                 (w_dkv_kr: [d_c + d_R, d_model])
 *   c   = kv[:d_c] / sqrt(mean(kv[:d_c]^2) + eps) * gamma
 *   k^R = RoPE(kv[d_c:], position)         (half-split pairs, angle
 *                                           pos / theta^(2k/d_R))
 *   cache[slot] = [c ; k^R] in cache_dtype (fp8: scale = max|row| / 448,
 *                 code = e4m3(row / scale), RNE, saturating)
 * hidden:   [n_tokens, d_model] act_dtype; or, when w_dkv_kr is NULL, the
 *           down-projection output itself, [n_tokens, d_c + d_R] fp32.
 * rms_gamma: [d_c] fp32.  positions: [n_tokens] int32 (>= 0).
 * slot_mapping: [n_tokens] int64; a slot < 0 or >= cache_slots is skipped
 *           (padding token).  cache_slots = num_blocks * block_size.
 * cache_scale: [cache_slots] fp32 for fp8 caches, else NULL.
 * workspace: at least mla_append_workspace_size() bytes (may be NULL if 0). */
size_t mla_append_workspace_size(const mla_dims_t* dims, int32_t n_tokens);
mla_status_t mla_append_latent(const mla_dims_t* dims, const void* hidden,
                               const void* w_dkv_kr, const float* rms_gamma,
                               const int32_t* positions, const int64_t* slot_mapping,
                               int32_t n_tokens, int64_t cache_slots, void* cache,
                               float* cache_scale, void* workspace, size_t workspace_bytes,
                               mla_stream_t stream);

/* ------------------------------------------------------------- absorb q
 * Latent query [MLA explainer, matrix absorption section eq.(8); decoupled
 * RoPE section eqs.(15)-(16)]:
 *   q_lat[n, i, :d_c] = W^UK_i^T q_nope[n, i]     (w_uk: [n_h, d_h, d_c],
 *                                                  W^UK_i is d_h x d_c)
 *   q_lat[n, i, d_c:] = RoPE(q_pe[n, i], positions[n])
 * q_nope: [n_tokens, n_h, d_h], q_pe: [n_tokens, n_h, d_R] act_dtype.
 * q_lat: [n_tokens, n_h, d_c + d_R] in cache_dtype for fp32 / bf16.  For an
 *          fp8 cache each row is two e4m3 planes [hi (d_c + d_R) | lo (d_c +
 *          d_R)] with x = row / q_scale, hi = e4m3(x), lo = e4m3((x - hi) * 16),
 *          so row ~= q_scale * (hi + lo / 16) to about 8 significant bits
 *          (mla_q_lat_row_bytes() gives the row size).
 * q_scale: [n_tokens, n_h] fp32 for fp8 (scale = max|q_lat row| / 448),
 *          else NULL.
 * workspace: at least mla_absorb_workspace_size() bytes (0 unless fp8: the
 *          fp32 rows are staged there before quantisation). */
size_t mla_absorb_workspace_size(const mla_dims_t* dims, int32_t n_tokens);
mla_status_t mla_absorb_q(const mla_dims_t* dims, const void* q_nope, const void* q_pe,
                          const void* w_uk, const int32_t* positions, int32_t n_tokens,
                          void* q_lat, float* q_scale, void* workspace, size_t workspace_bytes,
                          mla_stream_t stream);

/* --------------------------------------------------------------- decode
 * Attention over the latent cache with the absorbed query; all heads share
 * the rows (MQA with head width d_c + d_R whose value is the latent part,
 * [MLA explainer, trade-offs section]):
 *   s_j   = (q_lat . cache_j) * softmax_scale        j <= query position
 *   o_lat = sum_j softmax(s)_j cache_j[:d_c]         [eq.(9)-(10)]
 *   lse   = log sum_j exp(s_j)  (natural log)
 * The context of each request is cut into chunks of split_tokens rows;
 * each chunk writes a partial (o, lse) to the workspace and a combine kernel
 * merges them; with one chunk per request the partial step writes o_lat
 * directly.  split_tokens = 0 picks a size from the shapes; otherwise it
 * must be a positive multiple of 64 (bf16/fp8) and only changes rounding.
 * q_lat: [batch*q_len, n_h] rows as mla_absorb_q writes them; q_scale as
 *   above.
 * cache: pool [num_blocks, block_size, d_c + d_R]; cache_scale [num_blocks,
 *   block_size] for fp8 else NULL.
 * block_table: [batch, max_blocks_per_seq] int32 physical block ids, each
 *   in [0, num_blocks) (out-of-range ids are clamped into the pool).
 * seq_lens: [batch] int32 device, T_b = rows cached for request b including
 *   this step's q_len rows; values are clamped to [0, max_seq_len].  A query
 *   with no visible key gets o_lat = 0 and lse = -inf.
 * max_seq_len (host): upper bound of seq_lens, <= max_blocks_per_seq *
 *   block_size; it sizes the grid and the workspace.
 * o_lat: [batch*q_len, n_h, d_c] act_dtype.  lse: [batch*q_len, n_h] fp32
 *   (may be NULL). */
size_t mla_decode_workspace_size(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                 int32_t max_seq_len, int32_t split_tokens);
mla_status_t mla_decode(const mla_dims_t* dims, const void* q_lat, const float* q_scale,
                        const void* cache, const float* cache_scale,
                        const int32_t* block_table, int32_t max_blocks_per_seq,
                        int32_t num_blocks, const int32_t* seq_lens, int32_t batch, int32_t q_len,
                        int32_t max_seq_len, int32_t split_tokens, void* workspace,
                        size_t workspace_bytes, void* o_lat, float* lse, mla_stream_t stream);

/* The chunk length mla_decode uses for split_tokens = 0 (host helper). */
int32_t mla_decode_default_split(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                 int32_t max_seq_len);

/* ------------------------------------------------------------- out proj
 * Per-head output [MLA explainer, value-side absorption eq.(10)]:
 *   out[n, i] = W^UV_i o_lat[n, i]      (w_uv: [n_h, d_v, d_c], W^UV_i is
 *                                        d_v x d_c)
 * o_lat: [n_tokens, n_h, d_c], out: [n_tokens, n_h, d_v], act_dtype. */
mla_status_t mla_out_proj(const mla_dims_t* dims, const void* o_lat, const void* w_uv,
                          int32_t n_tokens, void* out, mla_stream_t stream);

/* -------------------------------------------------------------- prefill
 * Causal attention of one prompt of seq_len tokens, the non-absorbed way
 * the pages prescribe for prefill [MLA explainer, trade-offs section (no
 * absorption while the prompt is processed); decoupled RoPE eqs.(14)-(16)]:
 * per head i, q_t = [q^C_t ; RoPE(q^R_t, t)], k_j = [k^C_j ; k^R_j],
 * s = q_t . k_j * softmax_scale for j <= t, o_t = softmax(s) V.  Tokens sit
 * at positions 0..seq_len-1.
 * q_nope [seq_len, n_h, d_h], q_pe [seq_len, n_h, d_R] (before RoPE),
 * k_nope [seq_len, n_h, d_h] (= W^UK_i c_j, e.g. from mla_linear over the
 * latent rows), v [seq_len, n_h, d_v] (= W^UV_i c_j), out [seq_len, n_h, d_v]:
 * bf16.  k_rope: the RoPE'd shared key of token j at k_rope + j *
 * k_rope_stride (d_R bf16 values; k_rope = cache rows + d_c and stride
 * d_c + d_R reads them from contiguous cache rows).  lse [seq_len, n_h] fp32
 * natural log, or NULL.  Needs the bf16 dims (d_h = d_v = 128, d_R = 64,
 * bf16 cache and activations); others return MLA_ERR_UNSUPPORTED.
 * seq_len = 0 returns MLA_OK and launches nothing. */
mla_status_t mla_prefill_attention(const mla_dims_t* dims, const void* q_nope, const void* q_pe,
                                   const void* k_nope, const void* k_rope, int32_t k_rope_stride,
                                   const void* v, int32_t seq_len, void* out, float* lse,
                                   mla_stream_t stream);

/* --------------------------------------------------------------- linear
 * The dense projections on either side of the four calls above, as one
 * skinny bf16 GEMM (fp32 accumulation):
 *   y[m, :] = W x[m, :]        y = x W^T,  x: [m, k], w: [n, k], y: [m, n]
 * It serves the query path [MLA explainer, query-compression section
 * eq.(17): c^Q = W^DQ h, q^C = W^UQ c^Q; decoupled RoPE section eq.(15):
 * the RoPE query part is RoPE(W^QR c^Q), rotated by mla_absorb_q] and the
 * output projection [MLA explainer, value-side absorption eq.(11): u =
 * sum_i W^O_i o_i, i.e. x = out viewed as [m, n_h * d_v] and w = W^O; or,
 * absorbed, u = sum_i B_i o_lat_i with B_i = W^O_i W^UV_i, x = o_lat viewed
 * as [m, n_h * d_c] and w = [B_1 ... B_nh]].
 * x, w, y: row-major bf16 device buffers, owned by the caller; m >= 1,
 * n a multiple of 128, k a multiple of 16.  ldx: elements between rows of
 * x (>= k, a multiple of 8: 16-byte aligned rows), so that x can be the
 * latent part of cache rows (ldx = d_c + d_R).  m = 0 returns MLA_OK and
 * launches nothing.
 * workspace: at least mla_linear_workspace_size(m, n, k) bytes of device
 * memory (fp32 partial sums over slices of k; may be NULL if that is 0).
 * Other shapes return MLA_ERR_UNSUPPORTED, NULL buffers
 * MLA_ERR_INVALID_ARGUMENT, a short workspace MLA_ERR_WORKSPACE_TOO_SMALL;
 * nothing is launched then. */
size_t mla_linear_workspace_size(int32_t m, int32_t n, int32_t k);
mla_status_t mla_linear(const void* x, int32_t ldx, const void* w, int32_t m, int32_t n, int32_t k,
                        void* y, void* workspace, size_t workspace_bytes, mla_stream_t stream);

/* ------------------------------------------------------------ diagnostics */
const char* mla_status_string(mla_status_t status);
const char* mla_last_error_message(void); /* thread-local, never NULL */
int32_t mla_version(void);                /* major * 10000 + minor * 100 + patch */

#ifdef __cplusplus
}
#endif

#endif /* LIBMLA_MLA_H */
