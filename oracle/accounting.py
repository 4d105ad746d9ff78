"""Cache-size and work accounting in closed form (TEST INFRASTRUCTURE ONLY).

Each function states the count it follows.  Sources are the pages on MLA:

* [MLA explainer] disassemble-channel.com, "Multi-head Latent Attention（MLA）
  とは？KVキャッシュを圧縮するDeepSeekの注意機構を完全解説"
* [V2 summary] abeam.tech, summary of the DeepSeek-V2 paper (MLA / KV-cache
  compression article)
* [attention variants] youngju.dev, "model internals: attention variants" (ja)
"""


def mha_elems_per_token(layers, n_h, d_h):
    """Per-token cache elements of multi-head attention: keys and values for
    every head of every layer, 2*l*n_h*d_h.
    [MLA explainer, section on why the KV cache is the bottleneck, eq.(1)];
    [V2 summary, cache-size section, Table 1 formula];
    [attention variants, bytes formula for MHA/GQA]."""
    return 2 * layers * n_h * d_h


def gqa_elems_per_token(layers, n_groups, d_h):
    """Grouped-query attention keeps one K and one V per group.
    [MLA explainer, cache comparison section, the code's GQA row]."""
    return 2 * layers * n_groups * d_h


def mqa_elems_per_token(layers, d_h):
    """Multi-query attention keeps one K and one V for all heads.
    [MLA explainer, MHA->MQA->GQA section; cache comparison code]."""
    return 2 * layers * d_h


def mla_elems_per_token(layers, d_c, d_r):
    """MLA keeps the latent c^KV (d_c) and the shared RoPE key k^R (d_R) per
    layer: l*(d_c + d_R), with no factor 2 because K and V share the latent.
    [MLA explainer, cache comparison section]; [V2 summary, Table 1];
    [attention variants, MLA section: layers x (kv_lora_rank+qk_rope_head_dim)]."""
    return layers * (d_c + d_r)


def gqa_equivalent_groups(d_c, d_r, d_h):
    """Number of GQA groups with the same cache as MLA: (d_c+d_R)/(2 d_h).
    [MLA explainer, cache comparison section, eq.(18)]; [V2 summary, Table 1]."""
    return (d_c + d_r) / (2.0 * d_h)


def cache_bytes(elems_per_token, tokens, bytes_per_elem):
    """Bytes of cache for `tokens` tokens."""
    return elems_per_token * tokens * bytes_per_elem


def latent_row_bytes(d_c, d_r, elem_bytes, per_token_scale_bytes=0):
    """Bytes of one latent-cache row of one layer: (d_c + d_R) elements, plus
    a per-token scale when the cache is quantised per token."""
    return (d_c + d_r) * elem_bytes + per_token_scale_bytes


def naive_mults_per_cached_token(n_h, d_h, d_c):
    """Multiplies per cached token when K is re-expanded from the latent
    every step: n_h*d_h*d_c.  [MLA explainer, matrix absorption section]."""
    return n_h * d_h * d_c


def absorbed_mults_per_cached_token(n_h, d_c):
    """Multiplies per cached token in the absorbed score q~ . c: n_h*d_c.
    [MLA explainer, matrix absorption section; trade-offs section]."""
    return n_h * d_c


def mha_mults_per_cached_token(n_h, d_h):
    """Multiplies per cached token for the MHA score q . k: n_h*d_h.
    [MLA explainer, trade-offs section]."""
    return n_h * d_h


def naive_step_mults(T, n_h, d_h, d_c):
    """Multiplies per decode step to rebuild every cached key: T*n_h*d_h*d_c.
    [MLA explainer, low-rank section]."""
    return T * n_h * d_h * d_c


def decode_flops_per_visible_token(n_h, d_c, d_r):
    """Algorithmic FLOPs of absorbed decode per (cached token, query):
    n_h heads x (QK over d_c+d_R plus PV over d_c) x 2 FLOP per multiply-add."""
    return 2 * n_h * ((d_c + d_r) + d_c)
