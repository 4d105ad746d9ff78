"""Plain float64 MLA reference (TEST INFRASTRUCTURE ONLY).

What it follows (pages on Multi-head Latent Attention):

* [MLA explainer] disassemble-channel.com, "Multi-head Latent Attention（MLA）
  とは？KVキャッシュを圧縮するDeepSeekの注意機構を完全解説":
  low-rank section eqs.(2)-(3); matrix-absorption section eq.(8);
  value-side absorption eqs.(9)-(10); "RoPE breaks absorption" section
  (its rope() helper fixes the half-split pairing); decoupled-RoPE section
  eqs.(14)-(16) and the 1/sqrt(d_h+d_R) softmax scale; query-compression
  section eq.(17); value-side absorption into W^O, eq.(11); trade-offs
  section (RMSNorm on the cached latent; absorbed form = MQA with head dim
  576).
* [V2 summary] abeam.tech, DeepSeek-V2 / MLA KV-cache article: the
  four-step inference flow.
* [attention variants] youngju.dev: the extra RMSNorm after the compressed
  latent (DeepSeek-V3).

Conventions (row-major, one token per row):

* W_dkv_kr [d_c + d_R, d_model]: rows 0..d_c-1 are W^DKV, the rest W^KR.
  kv = h @ W_dkv_kr.T gives [W^DKV h ; W^KR h].
* W_UK [n_h, d_h, d_c] stacks W^UK_i (d_h x d_c): k^C_{j,i} = W^UK_i c_j.
* W_UV [n_h, d_v, d_c] stacks W^UV_i (d_v x d_c): v^C_{j,i} = W^UV_i c_j.
* W_DQ [d'_c, d_model], W_UQ [n_h*d_h, d'_c], W_QR [n_h*d_R, d'_c] (head
  i's rows contiguous); W_O [d_model, n_h*d_v] (W^O_i = column block i).
* RoPE: half-split pairs (x_k, x_{k+d/2}), angle pos / base^(2k/d).
* Query t of a request with T cached rows (the rows appended this step
  included) sits at position T - q_len + t and sees keys 0..its position.

Nothing is blocked, fused or reordered beyond the definitions; loops are
per request and per head so a reader can check each line against the pages.

Parity unpinned: the RMSNorm eps constant (the pages name the norm but no
eps; 1e-6 is a reading).  The norm's form is pinned by closed forms, the
constant is not.
"""

import numpy as np


# ------------------------------------------------------------------ pieces
def rope_half(x, pos, base=10000.0):
    """Rotary embedding with half-split pairing.

    x: [..., d] (d even); pos: positions broadcastable to x.shape[:-1].
    Element k of the first half and element k of the second half form one
    plane, turned by the angle pos * base^(-2k/d).  Written here as complex
    multiplication: z_k = x_k + i x_{k+d/2} becomes z_k e^{i angle}.
    [MLA explainer, "RoPE breaks absorption" section (pairing and angles);
    decoupled-RoPE section eq.(15)]."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    k = np.arange(half, dtype=np.float64)
    angle = np.asarray(pos, dtype=np.float64)[..., None] * np.power(base, -2.0 * k / x.shape[-1])
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * angle)
    return np.concatenate([z.real, z.imag], axis=-1)


def rmsnorm(x, gamma, eps):
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis.
    [MLA explainer, trade-offs section (normalisation of the latent)];
    [attention variants, trade-off section (RMSNorm after the latent)]."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * gamma


def softmax_stats(s):
    """Max-subtracted softmax over the last axis, with its log-sum-exp.
    Entries equal to -inf are masked.  Rows with no visible entry get
    weights 0 and lse = -inf (the empty sum)."""
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    m = np.where(empty, 0.0, m)
    p = np.exp(s - m)
    l = np.sum(p, axis=-1, keepdims=True)
    a = np.where(empty, 0.0, p / np.where(empty, 1.0, l))
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))
    return a, lse[..., 0]


def query_positions(T, q_len):
    """Positions of the q_len queries of a request with T cached rows."""
    return np.arange(q_len) + (T - q_len)


def causal_mask(q_pos, T):
    """Boolean [q_len, T]: query at position p sees keys 0..p."""
    return np.arange(T)[None, :] <= np.asarray(q_pos)[:, None]


# ------------------------------------------------------------ append step
def latent_rows(h, w_dkv_kr, gamma, pos, d_c, eps, base=10000.0):
    """New cache rows from hidden states.

    c = RMSNorm_gamma(W^DKV h)          [MLA explainer, low-rank eq.(2); norm]
    k^R = RoPE(W^KR h, pos)             [MLA explainer, decoupled eq.(15)]
    Returns (c [N, d_c], k^R [N, d_R])."""
    kv = np.asarray(h, np.float64) @ np.asarray(w_dkv_kr, np.float64).T
    c = rmsnorm(kv[:, :d_c], np.asarray(gamma, np.float64), eps)
    kr = rope_half(kv[:, d_c:], pos, base)
    return c, kr


def append_from_projection(kv, gamma, pos, d_c, eps, base=10000.0):
    """Same as latent_rows when the down-projection output kv [N, d_c+d_R]
    is given instead of h."""
    kv = np.asarray(kv, np.float64)
    c = rmsnorm(kv[:, :d_c], np.asarray(gamma, np.float64), eps)
    kr = rope_half(kv[:, d_c:], pos, base)
    return c, kr


# ---------------------------------------------- non-absorbed attention
def attention_nonabsorbed(q_nope, q_pe, q_pos, C, KR, w_uk, w_uv, scale,
                          base=10000.0, heads=None):
    """Standard MLA attention for one request, keys and values expanded.

    q_nope [Q, n_h, d_h]; q_pe [Q, n_h, d_R] (before RoPE); q_pos [Q];
    C [T, d_c] latent rows; KR [T, d_R] RoPE'd shared keys.
    For each head i:
      k_{j,i} = [W^UK_i c_j ; k^R_j]     [MLA explainer eq.(3), eq.(14)]
      v_{j,i} = W^UV_i c_j               [MLA explainer eq.(3)]
      q_{t,i} = [q^C ; RoPE(q^R, pos_t)] [MLA explainer eq.(14)-(15)]
      s = q.k * scale, causal            [eq.(16); scale 1/sqrt(d_h+d_R)]
      o = softmax(s) @ v                 [MLA explainer eq.(9)]
    Returns o [Q, len(heads), d_v]."""
    q_nope = np.asarray(q_nope, np.float64)
    q_pe = np.asarray(q_pe, np.float64)
    C = np.asarray(C, np.float64)
    KR = np.asarray(KR, np.float64)
    n_h = q_nope.shape[1]
    heads = range(n_h) if heads is None else heads
    mask = causal_mask(q_pos, C.shape[0])
    out = []
    for i in heads:
        k_c = C @ np.asarray(w_uk[i], np.float64).T          # [T, d_h]
        v = C @ np.asarray(w_uv[i], np.float64).T            # [T, d_v]
        k = np.concatenate([k_c, KR], axis=-1)               # [T, d_h+d_R]
        q = np.concatenate([q_nope[:, i], rope_half(q_pe[:, i], q_pos, base)], axis=-1)
        s = (q @ k.T) * scale
        s = np.where(mask, s, -np.inf)
        a, _ = softmax_stats(s)
        out.append(a @ v)
    return np.stack(out, axis=1)


# --------------------------------------------------- absorbed pieces
def absorb_q(q_nope, q_pe, q_pos, w_uk, base=10000.0):
    """Latent query per head: q~ = W^UK_i^T q^C, then the RoPE'd q^R appended.
    [MLA explainer, matrix absorption eq.(8); decoupled eq.(15)-(16)].
    q_nope [N, n_h, d_h], q_pe [N, n_h, d_R], q_pos [N] -> [N, n_h, d_c+d_R]."""
    q_nope = np.asarray(q_nope, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    n_h = q_nope.shape[1]
    lat = np.stack([q_nope[:, i] @ w_uk[i] for i in range(n_h)], axis=1)
    rot = rope_half(q_pe, np.asarray(q_pos)[:, None], base)
    return np.concatenate([lat, rot], axis=-1)


def decode_absorbed(q_lat, q_pos, C, KR, scale):
    """Attention over the latent cache with the absorbed query.

    q_lat [Q, n_h, d_c+d_R]; rows [C | KR] shared by every head (MQA with
    head dim d_c+d_R whose value is the latent part).
    s = q_lat . [c ; k^R] * scale (causal); o_lat = softmax(s) @ C.
    [MLA explainer eq.(8), eq.(10), eq.(16); trade-offs section (MQA view)].
    Returns (o_lat [Q, n_h, d_c], lse [Q, n_h]) with lse natural-log."""
    q_lat = np.asarray(q_lat, np.float64)
    C = np.asarray(C, np.float64)
    rows = np.concatenate([C, np.asarray(KR, np.float64)], axis=-1)
    mask = causal_mask(q_pos, C.shape[0])                     # [Q, T]
    s = np.einsum("qhd,td->qht", q_lat, rows) * scale
    s = np.where(mask[:, None, :], s, -np.inf)
    a, lse = softmax_stats(s)
    return np.einsum("qht,tc->qhc", a, C), lse


def out_proj(o_lat, w_uv):
    """Per-head output o = W^UV_i o_lat.  [MLA explainer eq.(10)].
    o_lat [N, n_h, d_c], W_UV [n_h, d_v, d_c] -> [N, n_h, d_v]."""
    o_lat = np.asarray(o_lat, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    return np.stack([o_lat[:, i] @ w_uv[i].T for i in range(o_lat.shape[1])], axis=1)


# ------------------------------------ projections around the attention block
def query_from_hidden(h, w_dq, w_uq, w_qr, n_h):
    """The query of every head from the hidden state, through the query
    latent.  c^Q = W^DQ h; content part q^C = W^UQ c^Q; RoPE part W^QR c^Q
    before its rotation (absorb_q rotates it).  [MLA explainer,
    query-compression section eq.(17); decoupled RoPE section eq.(15)].
    h [N, d]; w_dq [d'_c, d]; w_uq [n_h*d_h, d'_c] and w_qr [n_h*d_R, d'_c]
    with head i's rows contiguous.  Returns (c_q [N, d'_c],
    q_nope [N, n_h, d_h], q_pe [N, n_h, d_R])."""
    h = np.asarray(h, np.float64)
    c_q = h @ np.asarray(w_dq, np.float64).T
    q_nope = (c_q @ np.asarray(w_uq, np.float64).T).reshape(h.shape[0], n_h, -1)
    q_pe = (c_q @ np.asarray(w_qr, np.float64).T).reshape(h.shape[0], n_h, -1)
    return c_q, q_nope, q_pe


def absorbed_query_weights(w_uq, w_uk):
    """Query-side absorption: the latent query of head i straight from the
    query latent, q~_i = A_i c^Q with A_i = W^UK_i^T W^UQ_i (d_c x d'_c).
    [MLA explainer, matrix absorption eq.(7)-(8) and query-compression
    section (A_i becomes d'_c x d_c in the page's row-vector form)].
    w_uq [n_h*d_h, d'_c] (head i's rows contiguous), w_uk [n_h, d_h, d_c]
    -> A stacked by head, [n_h*d_c, d'_c] (an [out, in] weight)."""
    w_uq = np.asarray(w_uq, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    n_h, d_h, _ = w_uk.shape
    return np.concatenate([w_uk[i].T @ w_uq[i * d_h:(i + 1) * d_h] for i in range(n_h)], axis=0)


def query_latent_absorbed(c_q, a, n_h):
    """q~ [N, n_h, d_c] = A c^Q per head with A from absorbed_query_weights.
    [MLA explainer eq.(8) with the query-compression form of q^C]."""
    c_q = np.asarray(c_q, np.float64)
    return (c_q @ np.asarray(a, np.float64).T).reshape(c_q.shape[0], n_h, -1)


def output_projection(o, w_o):
    """u = sum_i W^O_i o_i, where W^O_i (d x d_v) is column block i of W^O.
    [MLA explainer, value-side absorption eq.(11), left-hand form].
    o [N, n_h, d_v], w_o [d, n_h*d_v] -> u [N, d]."""
    o = np.asarray(o, np.float64)
    w_o = np.asarray(w_o, np.float64)
    d_v = o.shape[2]
    return sum(o[:, i] @ w_o[:, i * d_v:(i + 1) * d_v].T for i in range(o.shape[1]))


def absorbed_output_weights(w_o, w_uv):
    """B_i = W^O_i W^UV_i (d x d_c), side by side: [d, n_h*d_c].
    [MLA explainer, value-side absorption eq.(11)].  w_o [d, n_h*d_v],
    w_uv [n_h, d_v, d_c]."""
    w_o = np.asarray(w_o, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    d_v = w_uv.shape[1]
    return np.concatenate([w_o[:, i * d_v:(i + 1) * d_v] @ w_uv[i] for i in range(w_uv.shape[0])], axis=1)


def output_projection_absorbed(o_lat, b):
    """u = sum_i B_i o_lat_i [MLA explainer eq.(11), right-hand form].
    o_lat [N, n_h, d_c], b [d, n_h*d_c] -> u [N, d]."""
    o_lat = np.asarray(o_lat, np.float64)
    b = np.asarray(b, np.float64)
    d_c = o_lat.shape[2]
    return sum(o_lat[:, i] @ b[:, i * d_c:(i + 1) * d_c].T for i in range(o_lat.shape[1]))


def combine_partials(o_parts, lse_parts):
    """Merge attention results over disjoint key sets (exact identity of
    softmax): L = log sum_s exp(lse_s); o = sum_s exp(lse_s - L) o_s.
    Used only to check split-context invariance."""
    lse_parts = np.asarray(lse_parts, np.float64)
    m = np.max(lse_parts, axis=0)
    w = np.exp(lse_parts - m)
    L = m + np.log(np.sum(w, axis=0))
    o = np.sum(np.exp(lse_parts - L)[..., None] * np.asarray(o_parts, np.float64), axis=0)
    return o, L


# ------------------------------------------- paged cache (host indexing)
def gather_rows(pool, block_table_row, T, block_size):
    """Rows 0..T-1 of one request from a paged pool [blocks, block_size, D]
    through its block table (plain indexing; no arithmetic on values)."""
    idx = np.arange(T)
    blocks = np.asarray(block_table_row)[idx // block_size]
    return pool[blocks, idx % block_size]
