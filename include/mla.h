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
 *                      (split over the context, then a combine kernel), after
 *                      mla_decode_plan has balanced the chunks; or
 *                      mla_decode_uniform with one chunk length for all
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
 *     stream) and never synchronise the host, except mla_decode_plan, which
 *     reads host lengths and waits for the copy of its work list.
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
 *     Cache variants [MLA wiki note, open questions (FP8 / FP4 caches) and
 *     adopting models (Kimi Linear: MLA without the RoPE part)]:
 *       MLA_FP4_E2M1 / MLA_BF16          MX FP4 rows (see mla_dtype_t); the
 *                           latent query is bf16 as for a bf16 cache
 *       MLA_FP8_E4M3_KR_BF16 / MLA_BF16  e4m3 latent with a per-row scale,
 *                           RoPE key kept in bf16; bf16 latent query
 *       MLA_BF16 / MLA_BF16 with qk_rope_head_dim = 0 (NoPE): 512-wide rows,
 *                           no RoPE key, latent query of d_c
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
  MLA_ERR_PLAN_MISMATCH = 4, /* a decode plan used with other dims, another
                                workspace, or a modified plan struct */
  MLA_ERR_HIP = 5
} mla_status_t;

typedef enum {
  MLA_F32 = 0,
  MLA_BF16 = 1,
  MLA_FP8_E4M3 = 2,
  /* cache only: MX FP4 rows, (d_c + d_R) E2M1 codes, two per byte
   * (element 2i in the low nibble), then one E8M0 scale byte per 32
   * elements (value 2^(b - 127)), then zero padding to a multiple of 16
   * bytes (320 B for d_c + d_R = 576) */
  MLA_FP4_E2M1 = 3,
  /* cache only: d_c e4m3 latent codes with one scale per row in
   * cache_scale, then the d_R RoPE-key values in bf16 (640 B for 512 + 64).
   * The scale is a power of two, stored as fp32: the smallest s with
   * max|latent| / s <= 448 (mla_append_latent writes it so; the 128-row
   * decode applies it inside its e4m3 -> bf16 conversion, which is exact
   * only for powers of two) */
  MLA_FP8_E4M3_KR_BF16 = 4
} mla_dtype_t;

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

/* Bytes of one stored cache row: (d_c + d_R) * element size for fp32, bf16
 * and fp8; the formats of mla_dtype_t for MLA_FP4_E2M1 and
 * MLA_FP8_E4M3_KR_BF16.  fp8 latents keep the per-row fp32 scale in a
 * separate [num_blocks, block_size] array.
 * Returns 0 for invalid dims.  [MLA explainer, cache comparison section;
 * variants, MLA section: per-token elements = d_c + d_R per layer.] */
size_t mla_cache_row_bytes(const mla_dims_t* dims);

/* HBM bytes one cached token occupies in one layer: the row plus, for an fp8
 * latent, its fp32 scale (mla_cache_row_bytes, + 4 for fp8).  Returns 0 for
 * invalid dims.  [MLA explainer, cache comparison section: per-token cache
 * of d_c + d_R elements per layer; variants, MLA section.] */
size_t mla_cache_bytes_per_token(const mla_dims_t* dims);

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

/* ------------------------------------------------------- append + absorb
 * mla_append_latent and mla_absorb_q in one call, for a step whose new
 * tokens are also its queries [V2 summary, "推論方法" (inference) section:
 * both read the step's new tokens].  On the MFMA path (with w_dkv_kr) the
 * append's down-projection and the latent query run as one launch, each
 * workgroup streaming one of the two weights; the append's finish (and for
 * an fp8 cache the query's quantisation) follows.  Otherwise the two calls
 * run in order.  Arguments as for the two calls (q_positions, n_q_tokens,
 * q_nope, q_pe, w_uk, q_lat, q_scale are mla_absorb_q's positions,
 * n_tokens, ...); one workspace of at least
 * mla_append_absorb_workspace_size() bytes serves both. */
size_t mla_append_absorb_workspace_size(const mla_dims_t* dims, int32_t n_tokens, int32_t n_q_tokens);
mla_status_t mla_append_absorb(const mla_dims_t* dims, const void* hidden, const void* w_dkv_kr,
                               const float* rms_gamma, const int32_t* positions,
                               const int64_t* slot_mapping, int32_t n_tokens, int64_t cache_slots,
                               void* cache, float* cache_scale, const void* q_nope, const void* q_pe,
                               const void* w_uk, const int32_t* q_positions, int32_t n_q_tokens,
                               void* q_lat, float* q_scale, void* workspace, size_t workspace_bytes,
                               mla_stream_t stream);

/* --------------------------------------------------------------- decode
 * Attention over the latent cache with the absorbed query; all heads share
 * the rows (MQA with head width d_c + d_R whose value is the latent part,
 * [MLA explainer, trade-offs section]):
 *   s_j   = (q_lat . cache_j) * softmax_scale        j <= query position
 *   o_lat = sum_j softmax(s)_j cache_j[:d_c]         [eq.(9)-(10)]
 *   lse   = log sum_j exp(s_j)  (natural log)
 * The context of a request is cut into chunks; each chunk writes a partial
 * (o, lse) to the workspace and a combine kernel merges them by the
 * log-sum-exp rule; a request with one chunk writes o_lat directly.  The
 * chunking only changes rounding.
 *
 * Two ways to launch it:
 *   planned  mla_decode_plan (host, once per batch composition) turns the
 *            host copy of the sequence lengths into a balanced work list in
 *            the workspace; mla_decode then runs it.  Ragged batches get
 *            chunks sized for the whole batch and placed across the eight
 *            XCDs by load, and no workgroup is launched for nothing.
 *   uniform  mla_decode_uniform cuts every request into chunks of one
 *            length sized from max_seq_len alone; it needs no host copy of
 *            the lengths, so a captured graph can replay it as they change.
 *
 * Common arguments:
 * q_lat: [batch*q_len, n_h] rows as mla_absorb_q writes them; q_scale as
 *   there (fp8 only, else NULL).
 * cache: pool [num_blocks, block_size, d_c + d_R]; cache_scale [num_blocks,
 *   block_size] for fp8 else NULL.
 * block_table: [batch, max_blocks_per_seq] int32 physical block ids, each
 *   in [0, num_blocks) (out-of-range ids are clamped into the pool).
 * seq_lens: [batch] int32 device, T_b = rows cached for request b including
 *   this step's q_len rows.  A query with no visible key gets o_lat = 0 and
 *   lse = -inf.
 * o_lat: [batch*q_len, n_h, d_c] act_dtype.  lse: [batch*q_len, n_h] fp32
 *   (may be NULL). */

/* Decode plan: filled by mla_decode_plan, read by mla_decode.  Plain data
 * owned by the caller; the work list it describes lives at the start of the
 * workspace given to mla_decode_plan, which must be passed unchanged to
 * mla_decode. */
typedef struct {
  int32_t batch;          /* requests */
  int32_t q_len;          /* queries per request */
  int32_t num_items;      /* context chunks over all requests */
  int32_t max_splits;     /* most chunks of one request */
  uint64_t hash;          /* digest of the dims, the fields below and the
                             lengths planned for */
  size_t workspace_bytes; /* workspace bytes mla_decode needs for this plan */
  size_t image_bytes;     /* bytes at the start of the workspace that hold
                             the work list (header, launch list, part_ptr) */
  int32_t split_tokens;   /* chunk length, a multiple of 64 */
  int32_t max_seq_len;    /* longest request planned for */
  int32_t num_slots;      /* workgroups mla_decode launches */
  int32_t num_partials;   /* chunks that write a partial (requests with >1 chunk) */
  uint64_t seq_digest;    /* digest of the lengths planned for */
  uint64_t workspace;     /* device address of the workspace planned into */
} mla_plan_t;

/* Workspace bytes a plan for these lengths needs (host seq_lens [batch]).
 * Returns 0 for invalid arguments. */
size_t mla_decode_plan_workspace_size(const mla_dims_t* dims, const int32_t* seq_lens_host,
                                      int32_t batch, int32_t q_len, int32_t split_tokens_hint);

/* Plans a decode over requests of the given lengths [V2 summary, "推論方法"
 * (inference) section: one step over a batch of cached requests; MLA
 * explainer, opening section: contexts up to 128k tokens].
 * seq_lens_host: [batch] int32 host memory, the lengths the device array
 *   passed to mla_decode will hold (each >= 0).
 * split_tokens_hint: 0 picks the chunk length from the lengths (balanced
 *   over the GPU's workgroup slots); otherwise a positive multiple of 64.
 * plan: filled on success.  workspace: device memory of at least
 *   mla_decode_plan_workspace_size() bytes; the work list is copied into it
 *   on `stream`, and this call waits for that copy (the one synchronising
 *   call of the library), so the plan can be reused for any number of
 *   mla_decode calls (e.g. every layer of a step) while the lengths stay
 *   the same. */
mla_status_t mla_decode_plan(const mla_dims_t* dims, const int32_t* seq_lens_host, int32_t batch,
                             int32_t q_len, int32_t split_tokens_hint, mla_plan_t* plan,
                             void* workspace, size_t workspace_bytes, mla_stream_t stream);

/* The host half of mla_decode_plan, for callers that copy the work list
 * themselves (e.g. asynchronously from pinned memory): fills `plan` and
 * writes the work-list image (plan->image_bytes bytes) to host memory.
 * workspace: the device address the image will be copied to (recorded in
 * the plan, never accessed).  host_image may be NULL to fill the plan only;
 * otherwise host_image_bytes >= plan->image_bytes.  Image layout (all
 * little-endian int32 unless noted): bytes 0-7 "MLAPLAN1", 8-15 the hash
 * (uint64); from byte 256 the launch list, num_slots entries of four:
 * {b | row_group << 24 (b = -1: idle slot), first row, end row, partial
 * block (-1: the request's only chunk, written to o_lat directly)}; then,
 * at the next multiple of 256, part_ptr [batch + 1] (the partial blocks of
 * request b are part_ptr[b] .. part_ptr[b+1] - 1).  Launch slot s runs on
 * XCD s % 8.  No device work. */
mla_status_t mla_decode_plan_host(const mla_dims_t* dims, const int32_t* seq_lens_host, int32_t batch,
                                  int32_t q_len, int32_t split_tokens_hint, const void* workspace,
                                  mla_plan_t* plan, void* host_image, size_t host_image_bytes);

/* Runs a plan.  Returns MLA_ERR_PLAN_MISMATCH if the plan was made for other
 * dims, was planned into another workspace, or was modified.  The device
 * seq_lens must hold the lengths planned for (kernels clamp each chunk to
 * the device value, so a shorter length stays in bounds). */
mla_status_t mla_decode(const mla_dims_t* dims, const mla_plan_t* plan, const void* q_lat,
                        const float* q_scale, const void* cache, const float* cache_scale,
                        const int32_t* block_table, int32_t max_blocks_per_seq, int32_t num_blocks,
                        const int32_t* seq_lens, void* workspace, size_t workspace_bytes,
                        void* o_lat, float* lse, mla_stream_t stream);

/* Uniform split.  max_seq_len (host): upper bound of seq_lens, <=
 * max_blocks_per_seq * block_size; device lengths are clamped to
 * [0, max_seq_len].  split_tokens = 0 picks a length from the shapes;
 * otherwise a positive multiple of 64 (bf16/fp8).  workspace: at least
 * mla_decode_uniform_workspace_size() bytes. */
size_t mla_decode_uniform_workspace_size(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                         int32_t max_seq_len, int32_t split_tokens);
mla_status_t mla_decode_uniform(const mla_dims_t* dims, const void* q_lat, const float* q_scale,
                                const void* cache, const float* cache_scale,
                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                int32_t num_blocks, const int32_t* seq_lens, int32_t batch,
                                int32_t q_len, int32_t max_seq_len, int32_t split_tokens,
                                void* workspace, size_t workspace_bytes, void* o_lat, float* lse,
                                mla_stream_t stream);

/* For callers that cannot allocate (code under graph capture, tight
 * serving loops, harnesses that forbid allocation): mla_decode_uniform with
 * its split partials in a static scratch array of the library instead of a
 * workspace.  No allocation of any kind happens in this call.  The scratch
 * holds MLA_NOALLOC_SCRATCH_BYTES (48 MiB) on each GPU the library runs on,
 * from the library's load until the process ends; a decode whose
 * mla_decode_uniform_workspace_size() exceeds it is rejected with
 * MLA_ERR_WORKSPACE_TOO_SMALL before anything is launched.
 * Every call on one GPU uses that GPU's one array: calls that overlap on a
 * GPU (e.g. on two streams without ordering) race and may return wrong
 * results.  Nothing in it needs clearing between calls (each call writes
 * every partial it reads).  Other arguments and errors as for
 * mla_decode_uniform. */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
mla_status_t mla_decode_uniform_noalloc(const mla_dims_t* dims, const void* q_lat, const float* q_scale,
                                        const void* cache, const float* cache_scale,
                                        const int32_t* block_table, int32_t max_blocks_per_seq,
                                        int32_t num_blocks, const int32_t* seq_lens, int32_t batch,
                                        int32_t q_len, int32_t max_seq_len, int32_t split_tokens,
                                        void* o_lat, float* lse, mla_stream_t stream);

/* The chunk length mla_decode_uniform uses for split_tokens = 0 (host helper). */
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

/* Chunked and multi-sequence prefill: the same attention over a table of
 * num_seqs sequences [MLA explainer, trade-offs section (prefill is
 * processed without absorption); decoupled RoPE eqs.(14)-(16)].  Sequence s
 * has keys cu_k[s] .. cu_k[s+1]-1 (rows of k_nope, v and k_rope): its cached
 * context of ctx_s tokens followed by its new tokens, and queries cu_q[s] ..
 * cu_q[s+1]-1 (rows of q_nope, q_pe, out, lse), the new tokens, with
 * Tq_s = cu_q[s+1] - cu_q[s] <= Tk_s = cu_k[s+1] - cu_k[s] and ctx_s =
 * Tk_s - Tq_s.  Query t of sequence s sits at position ctx_s + t (its RoPE
 * angle) and attends to keys 0 .. ctx_s + t of its sequence; ctx_s = 0 is a
 * whole prompt, ctx_s > 0 continues one after ctx_s cached tokens.
 * cu_q, cu_k: [num_seqs + 1] int32 device arrays, non-decreasing, cu_q[0] =
 * cu_k[0] = 0 (a sequence with Tk_s < Tq_s is computed as if ctx_s = 0 and
 * only its first Tk_s keys existed; out-of-order offsets are the caller's
 * error).  max_q (host): at least every Tq_s; it sizes the grid.
 * total_q (host): cu_q[num_seqs], rows of the query-side arrays.  Keys are
 * per head and already up-projected (k_nope = W^UK_i c, v = W^UV_i c, e.g.
 * by mla_linear over the sequences' latent rows); k_rope rows as above.
 * Same dims, dtypes and errors as mla_prefill_attention; num_seqs = 0 or
 * max_q = 0 returns MLA_OK and launches nothing. */
mla_status_t mla_prefill_attention_varlen(const mla_dims_t* dims, const void* q_nope, const void* q_pe,
                                          const void* k_nope, const void* k_rope, int32_t k_rope_stride,
                                          const void* v, const int32_t* cu_q, const int32_t* cu_k,
                                          int32_t num_seqs, int32_t max_q, int32_t total_q, void* out,
                                          float* lse, mla_stream_t stream);

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

/* Two projections of the same activations in one launch: y1 [m, n1] =
 * x w1^T and y2 [m, n2] = x w2^T, e.g. the query path's q^C = W^UQ c^Q and
 * the RoPE query input W^QR c^Q [MLA explainer, query-compression eq.(17);
 * decoupled RoPE eq.(15)], which share c^Q.  The same as two mla_linear
 * calls (up to the order of the fp32 partial sums); n1 and n2 multiples of
 * 128; workspace: at least mla_linear_workspace_size(m, n1 + n2, k) bytes.
 * Arguments and errors otherwise as for mla_linear. */
mla_status_t mla_linear_pair(const void* x, int32_t ldx, int32_t m, int32_t k, const void* w1, int32_t n1,
                             void* y1, const void* w2, int32_t n2, void* y2, void* workspace,
                             size_t workspace_bytes, mla_stream_t stream);

/* ------------------------------------------------------- absorbed weights
 * Formed once when a model is loaded, not per step.  act_dtype buffers
 * (bf16 or fp32), caller-owned device memory; fp32 accumulation.
 *
 * Output side [MLA explainer, value-side absorption eq.(11)]: B_i = W^O_i
 * W^UV_i, so that u = sum_i B_i o_lat_i.
 *   w_o [hidden_size, n_h * d_v] (W^O_i = column block i), w_uv [n_h, d_v,
 *   d_c] -> b [hidden_size, n_h * d_c] (B_i = column block i); mla_linear
 *   with x = o_lat viewed as [m, n_h * d_c] and w = b gives u.
 * Query side [MLA explainer, matrix absorption eqs.(7)-(8), query-compression
 * section]: A_i = W^UK_i^T W^UQ_i (d_c x d'_c), so that q~_i = A_i c^Q.
 *   w_uq [n_h * d_h, d_cq] (head i's rows contiguous), w_uk [n_h, d_h, d_c]
 *   -> a [n_h * d_c, d_cq]; mla_linear with x = c^Q and w = a gives the
 *   latent queries [m, n_h * d_c].
 * d_cq > 0.  Nothing is launched on an argument error. */
mla_status_t mla_absorb_output_weights(const mla_dims_t* dims, const void* w_o, const void* w_uv,
                                       void* b, mla_stream_t stream);
mla_status_t mla_absorb_query_weights(const mla_dims_t* dims, int32_t d_cq, const void* w_uq,
                                      const void* w_uk, void* a, mla_stream_t stream);

/* ------------------------------------------------------------ measurement
 * The achievable HBM read rate, measured beside the published peak: decode
 * time is set by reading the latent cache from HBM [MLA explainer, why the
 * KV cache is the bottleneck of inference: arithmetic intensity], so its
 * rate is read against both.  Reads the `bytes` at device pointer `buf` once
 * and computes nothing from them that the path uses.
 *   mode 0: 16-byte loads into registers from 2048 workgroups; bytes a
 *           multiple of 16; sink: device array of at least 2048 uint32
 *           (one XOR of the words read per workgroup, so no load is elided)
 *   mode 1: the decode kernels' copy structure (36 KB tiles by direct
 *           global->LDS copies, one workgroup per CU, three tiles in flight);
 *           bytes a multiple of 36864; sink unused (may be NULL)
 * Asynchronous on `stream`; errors as for the other calls. */
mla_status_t mla_hbm_read_probe(const void* buf, size_t bytes, int32_t mode, uint32_t* sink, size_t sink_words,
                                mla_stream_t stream);

/* ------------------------------------------------------------ diagnostics */
const char* mla_status_string(mla_status_t status);
const char* mla_last_error_message(void); /* thread-local, never NULL */
int32_t mla_version(void);                /* major * 10000 + minor * 100 + patch */

#ifdef __cplusplus
}
#endif

#endif /* LIBMLA_MLA_H */
