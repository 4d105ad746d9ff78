"""Pins for the CPU oracle: values the pages print, closed forms, special
cases that reduce to textbook attention or a library routine, and brute
force on tiny inputs.  CPU only."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import accounting as acc
from oracle import mla_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# The explainer page's seeded experiment, rebuilt from its stated shapes,
# seed and draw order, evaluated through the oracle's own functions.
# ---------------------------------------------------------------------------
def _draw_schedule(setup):
    """Draw the page's matrices from the schedule in the golden file: one
    generator, in the listed order, each draw shaped and scaled as listed."""
    rng = np.random.default_rng(setup["seed"])

    def dim(expr):
        return math.prod(setup[name] for name in expr.split("*"))

    out = {}
    for spec in setup["draws"]:
        shape = tuple(dim(e) for e in spec["shape"])
        if spec["dist"] == "normal":
            x = rng.normal(size=shape)
            fan_in = math.prod(setup[n] for n in spec["fan_in"])
            out[spec["name"]] = x / np.sqrt(fan_in) if spec["fan_in"] else x
        else:
            x = rng.random(shape)
            out[spec["name"]] = x / x.sum(axis=spec["normalise_axis"], keepdims=True)
    return out


@pytest.fixture(scope="module")
def page_example():
    g = _golden("page_worked_example.json")
    s = g["setup"]
    d_c, d_h, n_h, T, d_r = (s[k] for k in ("d_c", "d_h", "n_h", "T", "d_r"))
    m = _draw_schedule(s)
    # page layout (row vectors, head blocks of columns) -> oracle layout
    w_uk = np.stack([m["W_UK"][:, i * d_h:(i + 1) * d_h].T for i in range(n_h)])   # [n_h, d_h, d_c]
    w_uv = np.stack([m["W_UV"][:, i * d_h:(i + 1) * d_h].T for i in range(n_h)])   # [n_h, d_v, d_c]
    C_kv = m["H"] @ m["W_DKV"]
    C_q = m["H"] @ m["W_DQ"]
    q_c = (C_q @ m["W_UQ"]).reshape(T, n_h, d_h)                                   # query content part
    return dict(g=g, d_c=d_c, d_h=d_h, n_h=n_h, T=T, d_r=d_r, H=m["H"], C_kv=C_kv, C_q=C_q,
                q_c=q_c, w_uk=w_uk, w_uv=w_uv, W_O=m["W_O"], P=m["P"], W_QR=m["W_QR"], W_KR=m["W_KR"],
                W_UQ=m["W_UQ"], W_UK=m["W_UK"], W_DQ=m["W_DQ"])


def _expanded_keys(e):
    # k^C_{j,i} = W^UK_i c_j for every token j and head i -> [T, n_h, d_h]
    return np.stack([e["C_kv"] @ e["w_uk"][i].T for i in range(e["n_h"])], axis=1)


def test_page_key_absorption_value(page_example):
    e = page_example
    g = e["g"]["key_absorption"]
    n_h, T, d_c = e["n_h"], e["T"], e["d_c"]
    # absorbed path through the oracle: q~ = W^UK_i^T q (no RoPE part)
    q_lat = ref.absorb_q(e["q_c"], np.zeros((T, n_h, 0)), np.arange(T), e["w_uk"])
    assert q_lat.shape == (T, n_h, d_c)
    S_abs = np.einsum("tic,jc->tji", q_lat, e["C_kv"])
    assert abs(S_abs[3, 1, 0] - g["S_naive_t3_j1_h0"]) < 1e-12
    # explicit keys from the oracle's up-projection convention
    K = _expanded_keys(e)
    S_naive = np.einsum("tih,jih->tji", e["q_c"], K)
    assert abs(S_naive[3, 1, 0] - g["S_naive_t3_j1_h0"]) < 1e-12
    assert np.max(np.abs(S_naive - S_abs)) < 1e-12
    # the absorbed matrix A_i = W^UQ_i W^UK_i^T has rank d_h
    A = np.stack([e["W_UQ"][:, i * e["d_h"]:(i + 1) * e["d_h"]] @ e["w_uk"][i] for i in range(n_h)])
    assert list(A.shape) == g["A_shape"]
    assert np.linalg.matrix_rank(A[0]) == g["A0_rank"]


def test_page_value_absorption(page_example):
    e = page_example
    n_h, T = e["n_h"], e["T"]
    P = e["P"]                                                   # [T(query), T(key), n_h]
    # naive: expand V, weight, concatenate heads, output projection
    V = np.stack([e["C_kv"] @ e["w_uv"][i].T for i in range(n_h)], axis=1)
    naive = np.einsum("tji,jih->tih", P, V).reshape(T, -1) @ e["W_O"]
    # oracle: latent weighted sum, then per-head W^UV (out_proj), then W^O
    o_lat = np.einsum("tji,jc->tic", P, e["C_kv"])
    o = ref.out_proj(o_lat, e["w_uv"])
    absorbed = o.reshape(T, -1) @ e["W_O"]
    assert np.max(np.abs(naive - absorbed)) < 1e-12


def test_page_rope_breaks_absorption(page_example):
    """The printed RoPE'd score pins the half-split pairing and the angle
    formula of the oracle's rope_half at positions 0..5."""
    e = page_example
    g = e["g"]["rope_breaks_absorption"]
    T = e["T"]
    K = _expanded_keys(e)
    pos = np.arange(T)
    Qr = ref.rope_half(e["q_c"], pos[:, None])
    Kr = ref.rope_half(K, pos[:, None])
    S_true = np.einsum("tih,jih->tji", Qr, Kr)
    assert abs(S_true[3, 1, 0] - g["S_true_t3_j1_h0"]) < 1e-12
    q_lat = ref.absorb_q(e["q_c"], np.zeros((T, e["n_h"], 0)), pos, e["w_uk"])
    S_sub = np.einsum("tic,jc->tji", q_lat, e["C_kv"])
    assert abs(S_sub[3, 1, 0] - g["S_substituted_t3_j1_h0"]) < 1e-12
    assert abs(np.max(np.abs(S_true - S_sub)) - g["max_abs_err"]) < 1e-9


def test_rope_pairing_is_half_split_not_interleaved(page_example):
    """A plausible mistake (interleaved pairs) misses the printed value."""
    e = page_example
    K = _expanded_keys(e)

    def rope_interleaved(x, p):
        d = x.shape[-1]
        th = p / 10000.0 ** (2 * np.arange(d // 2) / d)
        x1, x2 = x[..., 0::2], x[..., 1::2]
        out = np.empty_like(x)
        out[..., 0::2] = x1 * np.cos(th) - x2 * np.sin(th)
        out[..., 1::2] = x1 * np.sin(th) + x2 * np.cos(th)
        return out

    wrong = rope_interleaved(e["q_c"][3, 0], 3) @ rope_interleaved(K[1, 0], 1)
    right = ref.rope_half(e["q_c"][3, 0], 3) @ ref.rope_half(K[1, 0], 1)
    pinned = e["g"]["rope_breaks_absorption"]["S_true_t3_j1_h0"]
    assert abs(right - pinned) < 1e-12
    assert abs(wrong - pinned) > 1e-3


def test_page_decoupled_rope(page_example):
    """Decoupled RoPE keeps absorption exact; checked through the oracle's
    full absorbed and non-absorbed attention with the page's matrices."""
    e = page_example
    n_h, T, d_r = e["n_h"], e["T"], e["d_r"]
    pos = np.arange(T)
    q_pe = (e["C_q"] @ e["W_QR"]).reshape(T, n_h, d_r)          # before RoPE
    KR = ref.rope_half(e["H"] @ e["W_KR"], pos)
    scale = 1.0 / math.sqrt(e["d_h"] + d_r)
    # scores both ways (page's check)
    K = _expanded_keys(e)
    QR = ref.rope_half(q_pe, pos[:, None])
    S_naive = np.einsum("tih,jih->tji", e["q_c"], K) + np.einsum("tir,jr->tji", QR, KR)
    q_lat = ref.absorb_q(e["q_c"], q_pe, pos, e["w_uk"])
    S_abs = np.einsum("tic,jc->tji", q_lat, np.concatenate([e["C_kv"], KR], axis=1))
    assert np.max(np.abs(S_naive - S_abs)) < 1e-12
    # full attention (causal, every position as a query) both ways
    o_ref = ref.attention_nonabsorbed(e["q_c"], q_pe, pos, e["C_kv"], KR, e["w_uk"], e["w_uv"], scale)
    o_lat, _ = ref.decode_absorbed(q_lat, pos, e["C_kv"], KR, scale)
    o_abs = ref.out_proj(o_lat, e["w_uv"])
    assert np.max(np.abs(o_ref - o_abs)) < 1e-12 * max(1.0, np.max(np.abs(o_ref)))


# ---------------------------------------------------------------------------
# Closed forms the pages print.
# ---------------------------------------------------------------------------
def test_cache_accounting_closed_forms():
    g = _golden("cache_accounting.json")
    v2 = g["explainer_v2_dims"]
    l, n_h, d_h, d_c, d_r, ng = (v2[k] for k in ("layers", "n_h", "d_h", "d_c", "d_r", "gqa_groups"))
    mha = acc.mha_elems_per_token(l, n_h, d_h)
    gqa = acc.gqa_elems_per_token(l, ng, d_h)
    mqa = acc.mqa_elems_per_token(l, d_h)
    mla = acc.mla_elems_per_token(l, d_c, d_r)
    printed = g["explainer_printed_elems_per_token"]
    assert (mha, gqa, mqa, mla) == (printed["MHA"], printed["GQA8"], printed["MQA"], printed["MLA"])
    mb = g["explainer_printed_MB_fp16"]
    for name, e in (("MHA", mha), ("GQA8", gqa), ("MQA", mqa), ("MLA", mla)):
        assert round(e * 2 / 1e6, 3) == mb[name]
    r = g["explainer_ratios"]
    assert round(mha / mla, 1) == r["MHA_over_MLA"]
    assert round(gqa / mla, 2) == r["GQA8_over_MLA"]
    assert round(mqa / mla, 2) == r["MQA_over_MLA"]
    assert round(100 * mla / mha, 2) == r["MLA_over_MHA_percent"]
    assert acc.gqa_equivalent_groups(d_c, d_r, d_h) == g["explainer_equivalent_groups"]
    assert 100 * d_r / d_c == g["explainer_kR_overhead_percent"]
    assert n_h * d_r == g["explainer_kR_if_per_head"]
    m = g["explainer_mults_per_cached_token"]
    assert acc.naive_mults_per_cached_token(n_h, d_h, d_c) == m["naive"]
    assert acc.absorbed_mults_per_cached_token(n_h, d_c) == m["absorbed"]
    assert acc.mha_mults_per_cached_token(n_h, d_h) == m["mha"]
    assert m["absorbed"] // m["mha"] == m["absorbed_over_mha"]
    assert m["naive"] // m["absorbed"] == d_h
    assert abs(acc.naive_step_mults(8192, n_h, d_h, d_c) / 1e9 - g["explainer_naive_step_mults_T8192_approx"] / 1e9) < 1.0
    assert 2 * n_h * d_h // d_c == g["explainer_compression_32768_to_512"]
    assert round(2 * n_h * d_h / 5120, 1) == g["explainer_redundancy_32768_over_5120"]
    # 8192-token MHA cache ~32 GB, read at ~2 TB/s -> ~16 ms -> ~62 tokens/s
    gb = acc.cache_bytes(mha, 8192, 2) / 1e9
    assert round(gb) == g["explainer_mha_ctx8192_GB"]
    ms = acc.cache_bytes(mha, 8192, 2) / (g["explainer_a100_TBps"] * 1e12) * 1e3
    assert round(ms) == g["explainer_ms_per_token"]
    assert int(1e3 / ms) == g["explainer_tokens_per_s"]
    for gbs, T in g["explainer_mha_fills_GB_at_T"].items():
        assert abs(acc.cache_bytes(mha, T, 2) / 1e9 - float(gbs)) / float(gbs) < 0.03
    assert round(acc.cache_bytes(mla, 131072, 2) / 1e9) == g["explainer_mla_T131072_GB"]
    # V2 summary Table 1: d_c = 4 d_h, d_R = d_h/2 -> 4.5 d_h l, i.e. 2.25 groups
    t1 = g["v2_summary_table1"]
    dh = 128
    assert acc.mla_elems_per_token(1, t1["d_c_over_d_h"] * dh, int(t1["d_r_over_d_h"] * dh)) == t1["mla_over_d_h_l"] * dh
    assert acc.gqa_equivalent_groups(4 * dh, dh // 2, dh) == t1["equivalent_groups"]
    # attention-variants page: DeepSeek-V3 and Kimi K2
    v3 = g["variants_v3"]
    e3 = acc.mla_elems_per_token(v3["layers"], v3["kv_lora_rank"], v3["qk_rope_head_dim"])
    assert e3 == v3["mla_elems"]
    assert acc.mha_elems_per_token(v3["layers"], v3["n_h"], v3["d_h"]) == v3["mha_elems"]
    assert round(v3["mha_elems"] / e3, 1) == v3["ratio"]
    assert round(acc.cache_bytes(e3, v3["ctx"], 2) / 2 ** 30, 2) == v3["fp16_GiB"]
    k2 = g["variants_kimi_k2"]
    assert acc.mla_elems_per_token(k2["layers"], 512, 64) == k2["mla_elems"]
    assert round(acc.mha_elems_per_token(k2["layers"], k2["n_h"], 128) / k2["mla_elems"], 1) == k2["ratio"]


def test_decode_flops_per_token_is_four_times_mha_scores():
    # absorbed QK multiplies per token (content part) = 4x MHA's at V2/V3 dims
    assert acc.absorbed_mults_per_cached_token(128, 512) == 4 * acc.mha_mults_per_cached_token(128, 128)
    # total FLOPs per visible (token, query): QK over 576 + PV over 512, x2
    assert acc.decode_flops_per_visible_token(128, 512, 64) == 2176 * 128


# ---------------------------------------------------------------------------
# Brute force on tiny inputs (pure Python loops, math.exp/cos/sin).
# ---------------------------------------------------------------------------
def _bf_rope(vec, pos, base=10000.0):
    d = len(vec)
    half = d // 2
    out = [0.0] * d
    for k in range(half):
        th = pos / base ** (2.0 * k / d)
        out[k] = vec[k] * math.cos(th) - vec[k + half] * math.sin(th)
        out[k + half] = vec[k] * math.sin(th) + vec[k + half] * math.cos(th)
    return out


def _bf_mla(q_nope, q_pe, q_pos, C, KR, w_uk, w_uv, scale):
    Q, n_h, d_h = q_nope.shape
    T, d_c = C.shape
    d_v = w_uv.shape[1]
    out = np.zeros((Q, n_h, d_v))
    for t in range(Q):
        for i in range(n_h):
            qr = _bf_rope(list(q_pe[t, i]), float(q_pos[t]))
            scores = []
            for j in range(T):
                if j > q_pos[t]:
                    continue
                s = 0.0
                for a in range(d_h):
                    kc = sum(w_uk[i, a, b] * C[j, b] for b in range(d_c))
                    s += q_nope[t, i, a] * kc
                for r in range(len(qr)):
                    s += qr[r] * KR[j, r]
                scores.append((j, s * scale))
            mx = max(s for _, s in scores)
            den = sum(math.exp(s - mx) for _, s in scores)
            for j, s in scores:
                w = math.exp(s - mx) / den
                for v in range(d_v):
                    out[t, i, v] += w * sum(w_uv[i, v, b] * C[j, b] for b in range(d_c))
    return out


def test_brute_force_tiny_mla():
    rng = np.random.default_rng(123)
    n_h, d_c, d_h, d_r, d_v, T, q_len, d = 3, 6, 4, 4, 5, 7, 2, 10
    h = rng.normal(size=(T, d))
    w = rng.normal(size=(d_c + d_r, d)) / np.sqrt(d)
    gamma = rng.uniform(0.5, 1.5, size=d_c)
    pos = np.arange(T)
    C, KR = ref.latent_rows(h, w, gamma, pos, d_c, 1e-6)
    # brute-force the append step too
    for j in range(T):
        kv = [sum(w[r, a] * h[j, a] for a in range(d)) for r in range(d_c + d_r)]
        ms = sum(x * x for x in kv[:d_c]) / d_c
        c = [kv[r] / math.sqrt(ms + 1e-6) * gamma[r] for r in range(d_c)]
        assert np.allclose(C[j], c, rtol=0, atol=1e-12)
        assert np.allclose(KR[j], _bf_rope(kv[d_c:], float(j)), rtol=0, atol=1e-12)
    w_uk = rng.normal(size=(n_h, d_h, d_c)) / np.sqrt(d_c)
    w_uv = rng.normal(size=(n_h, d_v, d_c)) / np.sqrt(d_c)
    q_nope = rng.normal(size=(q_len, n_h, d_h))
    q_pe = rng.normal(size=(q_len, n_h, d_r))
    q_pos = ref.query_positions(T, q_len)
    scale = 1.0 / math.sqrt(d_h + d_r)
    o = ref.attention_nonabsorbed(q_nope, q_pe, q_pos, C, KR, w_uk, w_uv, scale)
    o_bf = _bf_mla(q_nope, q_pe, q_pos, C, KR, w_uk, w_uv, scale)
    assert np.max(np.abs(o - o_bf)) < 1e-12
    # and the absorbed form
    q_lat = ref.absorb_q(q_nope, q_pe, q_pos, w_uk)
    o_lat, _ = ref.decode_absorbed(q_lat, q_pos, C, KR, scale)
    assert np.max(np.abs(ref.out_proj(o_lat, w_uv) - o_bf)) < 1e-12


# ---------------------------------------------------------------------------
# Special cases: MQA as a special case of MLA (wiki page, cross-cutting
# findings; explainer MHA->MQA->GQA section), MQA with head dim d_c+d_R
# (explainer trade-offs), GQA representable by MLA (TransMLA dialogue page).
# ---------------------------------------------------------------------------
def _bf_single_kv_attention(q, K, V, scale, visible):
    Q, n_h, _ = q.shape
    out = np.zeros((Q, n_h, V.shape[1]))
    for t in range(Q):
        for i in range(n_h):
            js = [j for j in range(K.shape[0]) if j <= visible[t]]
            s = [scale * sum(q[t, i, a] * K[j, a] for a in range(K.shape[1])) for j in js]
            mx = max(s)
            den = sum(math.exp(x - mx) for x in s)
            for jj, j in enumerate(js):
                out[t, i] += math.exp(s[jj] - mx) / den * V[j]
    return out


def test_mqa_is_special_case_identity_projections():
    rng = np.random.default_rng(5)
    n_h, d_h, T = 4, 6, 9
    C = rng.normal(size=(T, d_h))
    eye = np.stack([np.eye(d_h)] * n_h)
    q = rng.normal(size=(1, n_h, d_h))
    pos = np.array([T - 1])
    scale = 1 / math.sqrt(d_h)
    o = ref.attention_nonabsorbed(q, np.zeros((1, n_h, 0)), pos, C, np.zeros((T, 0)), eye, eye, scale)
    o_bf = _bf_single_kv_attention(q, C, C, scale, pos)
    assert np.max(np.abs(o - o_bf)) < 1e-12


def test_mqa_general_k_neq_v():
    rng = np.random.default_rng(6)
    n_h, d_h, T, Q = 3, 4, 8, 2
    Kmat = rng.normal(size=(T, d_h))
    Vmat = rng.normal(size=(T, d_h))
    C = np.concatenate([Kmat, Vmat], axis=1)                  # d_c = 2 d_h
    sel_k = np.stack([np.concatenate([np.eye(d_h), np.zeros((d_h, d_h))], axis=1)] * n_h)
    sel_v = np.stack([np.concatenate([np.zeros((d_h, d_h)), np.eye(d_h)], axis=1)] * n_h)
    q = rng.normal(size=(Q, n_h, d_h))
    pos = ref.query_positions(T, Q)
    scale = 1 / math.sqrt(d_h)
    o = ref.attention_nonabsorbed(q, np.zeros((Q, n_h, 0)), pos, C, np.zeros((T, 0)), sel_k, sel_v, scale)
    assert np.max(np.abs(o - _bf_single_kv_attention(q, Kmat, Vmat, scale, pos))) < 1e-12


def test_gqa_representable_by_mla():
    rng = np.random.default_rng(7)
    n_h, n_g, d_h, T = 6, 2, 3, 5
    Ks = rng.normal(size=(n_g, T, d_h))
    Vs = rng.normal(size=(n_g, T, d_h))
    C = np.concatenate(list(Ks) + list(Vs), axis=1)           # d_c = 2 n_g d_h
    d_c = C.shape[1]
    w_uk = np.zeros((n_h, d_h, d_c))
    w_uv = np.zeros((n_h, d_h, d_c))
    for i in range(n_h):
        g = i // (n_h // n_g)
        w_uk[i][:, g * d_h:(g + 1) * d_h] = np.eye(d_h)
        w_uv[i][:, (n_g + g) * d_h:(n_g + g + 1) * d_h] = np.eye(d_h)
    q = rng.normal(size=(1, n_h, d_h))
    pos = np.array([T - 1])
    o = ref.attention_nonabsorbed(q, np.zeros((1, n_h, 0)), pos, C, np.zeros((T, 0)), w_uk, w_uv, 0.7)
    for i in range(n_h):
        g = i // (n_h // n_g)
        bf = _bf_single_kv_attention(q[:, i:i + 1], Ks[g], Vs[g], 0.7, pos)
        assert np.max(np.abs(o[:, i] - bf[:, 0])) < 1e-12


def test_decode_equals_library_mqa_576():
    """The absorbed decode is MQA with one KV head of width d_c+d_R whose
    value is the latent part; torch's CPU scaled_dot_product_attention in
    float64 gives a second opinion."""
    rng = np.random.default_rng(8)
    n_h, d_c, d_r, T, q_len = 8, 32, 8, 40, 2
    C = rng.normal(size=(T, d_c))
    KR = rng.normal(size=(T, d_r))
    q_lat = rng.normal(size=(q_len, n_h, d_c + d_r))
    pos = ref.query_positions(T, q_len)
    scale = 0.3
    o_lat, lse = ref.decode_absorbed(q_lat, pos, C, KR, scale)
    q = torch.from_numpy(q_lat).permute(1, 0, 2)[None]                     # [1, n_h, q_len, D]
    k = torch.from_numpy(np.concatenate([C, KR], 1))[None, None].expand(1, n_h, T, d_c + d_r)
    v = torch.from_numpy(C)[None, None].expand(1, n_h, T, d_c)
    mask = torch.from_numpy(ref.causal_mask(pos, T))[None, None]
    o_t = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    assert np.max(np.abs(o_t[0].permute(1, 0, 2).numpy() - o_lat)) < 1e-12
    s = torch.einsum("bhqd,bhkd->bhqk", q, k) * scale
    s = s.masked_fill(~mask, float("-inf"))
    lse_t = torch.logsumexp(s, dim=-1)[0].permute(1, 0).numpy()
    assert np.max(np.abs(lse_t - lse)) < 1e-12


# ---------------------------------------------------------------------------
# Invariants.
# ---------------------------------------------------------------------------
def test_rope_relative_position_and_identity():
    rng = np.random.default_rng(9)
    q = rng.normal(size=16)
    k = rng.normal(size=16)
    assert np.allclose(ref.rope_half(q, 0), q, atol=0, rtol=0)
    base = ref.rope_half(q, 7) @ ref.rope_half(k, 3)
    for shift in (1, 100, 131071):
        assert abs(ref.rope_half(q, 7 + shift) @ ref.rope_half(k, 3 + shift) - base) < 1e-9
    assert abs(np.linalg.norm(ref.rope_half(q, 12345)) - np.linalg.norm(q)) < 1e-12


def test_rmsnorm_gain_folds_into_up_projections():
    """Caching RMSNorm_gamma(c) with W^UK, W^UV equals caching RMSNorm_1(c)
    with W^UK diag(gamma), W^UV diag(gamma)."""
    rng = np.random.default_rng(10)
    n_h, d_c, d_h, d_r, d_v, T, d = 2, 8, 4, 4, 4, 6, 12
    h = rng.normal(size=(T, d))
    w = rng.normal(size=(d_c + d_r, d)) / np.sqrt(d)
    gamma = rng.uniform(0.5, 1.5, size=d_c)
    pos = np.arange(T)
    C_g, KR = ref.latent_rows(h, w, gamma, pos, d_c, 1e-6)
    C_1, _ = ref.latent_rows(h, w, np.ones(d_c), pos, d_c, 1e-6)
    w_uk = rng.normal(size=(n_h, d_h, d_c))
    w_uv = rng.normal(size=(n_h, d_v, d_c))
    q_nope = rng.normal(size=(1, n_h, d_h))
    q_pe = rng.normal(size=(1, n_h, d_r))
    qp = np.array([T - 1])
    a = ref.attention_nonabsorbed(q_nope, q_pe, qp, C_g, KR, w_uk, w_uv, 0.4)
    b = ref.attention_nonabsorbed(q_nope, q_pe, qp, C_1, KR, w_uk * gamma, w_uv * gamma, 0.4)
    assert np.max(np.abs(a - b)) < 1e-12
    # a dropped gain is visible
    c = ref.attention_nonabsorbed(q_nope, q_pe, qp, C_1, KR, w_uk, w_uv, 0.4)
    assert np.max(np.abs(a - c)) > 1e-3


def test_rmsnorm_closed_forms():
    """RMSNorm's own definition: with gain 1 and eps 0 the output has unit
    root-mean-square, it is invariant to a positive rescaling of its input,
    a constant vector maps to its sign times the gain, and eps only matters
    against mean(x^2).  (The eps constant itself is a reading, not pinned.)"""
    rng = np.random.default_rng(12)
    x = rng.normal(size=(5, 16)) * rng.uniform(0.1, 10, size=(5, 1))
    y = ref.rmsnorm(x, np.ones(16), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-14)
    assert np.allclose(ref.rmsnorm(3.7 * x, np.ones(16), 0.0), y, atol=1e-14)
    gamma = rng.uniform(0.5, 1.5, size=16)
    assert np.allclose(ref.rmsnorm(np.full(16, -2.5), gamma, 0.0), -gamma, atol=1e-15)
    assert np.allclose(ref.rmsnorm(x, gamma, 0.0), y * gamma, atol=1e-14)
    small = np.full(16, 1e-4)      # mean(x^2) = 1e-8: eps = 1e-6 dominates
    assert abs(ref.rmsnorm(small, np.ones(16), 1e-6)[0] - 1e-4 / math.sqrt(1e-8 + 1e-6)) < 1e-15
    assert np.all(ref.rmsnorm(np.zeros(16), gamma, 1e-6) == 0)


def test_softmax_special_cases():
    rng = np.random.default_rng(11)
    T, n_h, d_c, d_r = 10, 3, 8, 4
    C = rng.normal(size=(T, d_c))
    KR = rng.normal(size=(T, d_r))
    # one visible row: output is that row exactly, lse = its score
    q = rng.normal(size=(1, n_h, d_c + d_r))
    o, lse = ref.decode_absorbed(q, np.array([0]), C[:1], KR[:1], 0.5)
    assert np.array_equal(o[0], np.broadcast_to(C[0], (n_h, d_c)))
    assert np.allclose(lse[0], 0.5 * (q[0] @ np.concatenate([C[0], KR[0]])), rtol=0, atol=1e-14)
    # zero query: uniform weights, output = mean of rows, lse = log T
    o, lse = ref.decode_absorbed(np.zeros((1, n_h, d_c + d_r)), np.array([T - 1]), C, KR, 0.5)
    assert np.max(np.abs(o[0] - C.mean(axis=0))) < 1e-14
    assert np.allclose(lse, math.log(T), rtol=0, atol=1e-14)
    # two queries, causal: query 0 equals a one-query decode over T-1 rows
    q2 = rng.normal(size=(2, n_h, d_c + d_r))
    o2, l2 = ref.decode_absorbed(q2, ref.query_positions(T, 2), C, KR, 0.5)
    o1, l1 = ref.decode_absorbed(q2[:1], np.array([T - 2]), C[:T - 1], KR[:T - 1], 0.5)
    assert np.max(np.abs(o2[0] - o1[0])) < 1e-14 and np.max(np.abs(l2[0] - l1[0])) < 1e-14
    # no visible key: zero output and lse = -inf
    o, lse = ref.decode_absorbed(q, np.array([-1]), C, KR, 0.5)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_split_context_combine_identity():
    """Splitting the keys into ranges and merging with the log-sum-exp rule
    gives the unsplit result (the basis of split-KV decode)."""
    rng = np.random.default_rng(12)
    T, n_h, d_c, d_r = 50, 4, 16, 4
    C = rng.normal(size=(T, d_c))
    KR = rng.normal(size=(T, d_r))
    q = rng.normal(size=(1, n_h, d_c + d_r)) * 3
    pos = np.array([T - 1])
    full_o, full_l = ref.decode_absorbed(q, pos, C, KR, 0.2)
    parts_o, parts_l = [], []
    for a, b in ((0, 13), (13, 30), (30, 50)):
        o, l = ref.decode_absorbed(q, np.array([b - a - 1]), C[a:b], KR[a:b], 0.2)
        parts_o.append(o)
        parts_l.append(l)
    o, l = ref.combine_partials(np.stack(parts_o), np.stack(parts_l))
    assert np.max(np.abs(o - full_o)) < 1e-13 and np.max(np.abs(l - full_l)) < 1e-13


@pytest.mark.parametrize("shape", [
    dict(n_h=4, d_c=32, d_h=16, d_r=8, d_v=16, T=64, q_len=1),      # tiny fp32 decode shape
    dict(n_h=128, d_c=512, d_h=128, d_r=64, d_v=128, T=96, q_len=1),  # V3 dims, short context
    dict(n_h=64, d_c=512, d_h=128, d_r=64, d_v=128, T=80, q_len=1),   # Kimi-K2 head count
    dict(n_h=128, d_c=512, d_h=128, d_r=64, d_v=128, T=70, q_len=2),  # V3, two causal queries
])
def test_absorbed_equals_nonabsorbed_at_workload_dims(shape):
    rng = np.random.default_rng(13)
    s = shape
    C = rng.normal(size=(s["T"], s["d_c"]))
    KR = rng.normal(size=(s["T"], s["d_r"]))
    w_uk = rng.normal(size=(s["n_h"], s["d_h"], s["d_c"])) / np.sqrt(s["d_c"])
    w_uv = rng.normal(size=(s["n_h"], s["d_v"], s["d_c"])) / np.sqrt(s["d_c"])
    q_nope = rng.normal(size=(s["q_len"], s["n_h"], s["d_h"]))
    q_pe = rng.normal(size=(s["q_len"], s["n_h"], s["d_r"]))
    pos = ref.query_positions(s["T"], s["q_len"])
    scale = 1 / math.sqrt(s["d_h"] + s["d_r"])
    heads = [0, s["n_h"] // 2, s["n_h"] - 1]
    o = ref.attention_nonabsorbed(q_nope, q_pe, pos, C, KR, w_uk, w_uv, scale, heads=heads)
    q_lat = ref.absorb_q(q_nope, q_pe, pos, w_uk)
    o_lat, _ = ref.decode_absorbed(q_lat, pos, C, KR, scale)
    o_abs = ref.out_proj(o_lat, w_uv)[:, heads]
    assert np.max(np.abs(o - o_abs)) <= 1e-12 * np.max(np.abs(o))


def test_paged_gather_follows_block_table():
    rng = np.random.default_rng(14)
    bs, nblk, D, T = 4, 6, 3, 10
    pool = rng.normal(size=(nblk, bs, D))
    table = np.array([5, 2, 0])
    rows = ref.gather_rows(pool, table, T, bs)
    for t in range(T):
        assert np.array_equal(rows[t], pool[table[t // bs], t % bs])


# ---------------------------------------------------------------------------
# The projections around the attention block: query path and W^O.
# ---------------------------------------------------------------------------
def test_page_query_path_value(page_example):
    """The page's printed score pins the oracle's query path: c^Q = W^DQ h,
    q^C = W^UQ c^Q with head i's rows contiguous (a transposed or mis-sliced
    W^UQ changes the value)."""
    e = page_example
    g = e["g"]["key_absorption"]
    n_h, d_h, d_r = e["n_h"], e["d_h"], e["d_r"]
    W_DQ, W_UQ = e["W_DQ"], e["W_UQ"]
    # page layout (row vectors) -> [out, in]
    c_q, q_nope, q_pe = ref.query_from_hidden(e["H"], W_DQ.T, W_UQ.T, e["W_QR"].T, n_h)
    assert q_nope.shape == (e["T"], n_h, d_h) and q_pe.shape == (e["T"], n_h, d_r)
    S = np.einsum("tih,jih->tji", q_nope, _expanded_keys(e))
    assert abs(S[3, 1, 0] - g["S_naive_t3_j1_h0"]) < 1e-12


def test_output_projection_picks_head_column_blocks():
    """A one-hot per-head output selects exactly one column of W^O: o_i with a
    single 1 at position k gives u = W^O[:, i*d_v + k] (eq.(11), W^O_i is
    column block i)."""
    rng = np.random.default_rng(31)
    n_h, d_v, d = 3, 4, 5
    w_o = rng.normal(size=(d, n_h * d_v))
    for i in range(n_h):
        for k in range(d_v):
            o = np.zeros((1, n_h, d_v))
            o[0, i, k] = 1.0
            assert np.array_equal(ref.output_projection(o, w_o)[0], w_o[:, i * d_v + k])


def test_output_projection_brute_force():
    rng = np.random.default_rng(32)
    n_h, d_v, d, N = 3, 4, 5, 2
    w_o = rng.normal(size=(d, n_h * d_v))
    o = rng.normal(size=(N, n_h, d_v))
    u = ref.output_projection(o, w_o)
    for t in range(N):
        for m in range(d):
            acc = 0.0
            for i in range(n_h):
                for k in range(d_v):
                    acc += w_o[m, i * d_v + k] * o[t, i, k]
            assert abs(u[t, m] - acc) < 1e-12


def test_absorbed_output_weights_equal_the_two_step_path():
    """eq.(11): sum_i B_i o_lat_i with B_i = W^O_i W^UV_i equals W^O applied
    after the per-head W^UV, in float64 at the V3 head shape (few heads)."""
    rng = np.random.default_rng(33)
    n_h, d_c, d_v, d, N = 4, 512, 128, 256, 3
    w_uv = rng.normal(size=(n_h, d_v, d_c)) / np.sqrt(d_c)
    w_o = rng.normal(size=(d, n_h * d_v)) / np.sqrt(n_h * d_v)
    o_lat = rng.normal(size=(N, n_h, d_c))
    two_step = ref.output_projection(ref.out_proj(o_lat, w_uv), w_o)
    b = ref.absorbed_output_weights(w_o, w_uv)
    assert b.shape == (d, n_h * d_c)
    absorbed = ref.output_projection_absorbed(o_lat, b)
    assert np.max(np.abs(two_step - absorbed)) <= 1e-12 * np.max(np.abs(two_step))


def test_query_rope_part_brute_force():
    """The RoPE half of the query path, W^QR c^Q with head i's d_R rows
    contiguous, against plain loops over the page's draws (a transposed or
    mis-sliced W^QR fails here); and the page's decoupled-RoPE equality
    with q^R taken from the oracle's query path."""
    rng = np.random.default_rng(41)
    n_h, d_r, d_h, d_cq, d, N = 3, 4, 2, 5, 6, 2
    h = rng.normal(size=(N, d))
    w_dq = rng.normal(size=(d_cq, d))
    w_uq = rng.normal(size=(n_h * d_h, d_cq))
    w_qr = rng.normal(size=(n_h * d_r, d_cq))
    _, q_nope, q_pe = ref.query_from_hidden(h, w_dq, w_uq, w_qr, n_h)
    for t in range(N):
        c_q = [sum(w_dq[a, m] * h[t, m] for m in range(d)) for a in range(d_cq)]
        for i in range(n_h):
            for r in range(d_r):
                want = sum(w_qr[i * d_r + r, a] * c_q[a] for a in range(d_cq))
                assert abs(q_pe[t, i, r] - want) < 1e-12
            for k in range(d_h):
                want = sum(w_uq[i * d_h + k, a] * c_q[a] for a in range(d_cq))
                assert abs(q_nope[t, i, k] - want) < 1e-12


def test_page_decoupled_rope_through_query_path(page_example):
    """The page's decoupled-RoPE check with q^R from query_from_hidden: the
    scores of the expanded keys equal the absorbed scores over [c ; k^R]."""
    e = page_example
    n_h, T = e["n_h"], e["T"]
    pos = np.arange(T)
    _, q_nope, q_pe = ref.query_from_hidden(e["H"], e["W_DQ"].T, e["W_UQ"].T, e["W_QR"].T, n_h)
    # the page's own layout: q^R = (C_q W_QR) split into head blocks of d_R columns
    q_pe_page = (e["C_q"] @ e["W_QR"]).reshape(T, n_h, e["d_r"])
    assert np.max(np.abs(q_pe - q_pe_page)) < 1e-12
    KR = ref.rope_half(e["H"] @ e["W_KR"], pos)
    QR = ref.rope_half(q_pe, pos[:, None])
    S_naive = np.einsum("tih,jih->tji", q_nope, _expanded_keys(e)) + np.einsum("tir,jr->tji", QR, KR)
    q_lat = ref.absorb_q(q_nope, q_pe, pos, e["w_uk"])
    S_abs = np.einsum("tic,jc->tji", q_lat, np.concatenate([e["C_kv"], KR], axis=1))
    assert np.max(np.abs(S_naive - S_abs)) < 1e-12


def test_append_from_projection_matches_hidden_path_and_loops():
    """The append step fed the down-projection output: equal to latent_rows
    fed h, and to plain loops (norm over the latent only, RoPE on the rest)."""
    rng = np.random.default_rng(42)
    d_c, d_r, d, N = 6, 4, 9, 5
    h = rng.normal(size=(N, d))
    w = rng.normal(size=(d_c + d_r, d)) / np.sqrt(d)
    gamma = rng.uniform(0.5, 1.5, size=d_c)
    pos = np.array([0, 3, 17, 4095, 131071])
    kv = h @ w.T
    c, kr = ref.append_from_projection(kv, gamma, pos, d_c, 1e-6)
    c2, kr2 = ref.latent_rows(h, w, gamma, pos, d_c, 1e-6)
    assert np.max(np.abs(c - c2)) < 1e-12 and np.max(np.abs(kr - kr2)) < 1e-12
    for j in range(N):
        ms = sum(kv[j, r] ** 2 for r in range(d_c)) / d_c
        for r in range(d_c):
            assert abs(c[j, r] - kv[j, r] / math.sqrt(ms + 1e-6) * gamma[r]) < 1e-12
        assert np.allclose(kr[j], _bf_rope(list(kv[j, d_c:]), float(pos[j])), rtol=0, atol=1e-9)
    # the RoPE part is not normalised: scaling it scales k^R alone
    c3, kr3 = ref.append_from_projection(np.concatenate([kv[:, :d_c], 3 * kv[:, d_c:]], 1), gamma, pos, d_c, 1e-6)
    assert np.max(np.abs(c3 - c)) < 1e-12 and np.max(np.abs(kr3 - 3 * kr)) < 1e-12


def test_page_query_absorbed_weights(page_example):
    """A_i = W^UK_i^T W^UQ_i: the page's shape and rank (printed), and the
    same latent query as the two-step path (c^Q -> q^C -> W^UK_i^T q^C)."""
    e = page_example
    g = e["g"]["key_absorption"]
    n_h, d_c, d_h = e["n_h"], e["d_c"], e["d_h"]
    a = ref.absorbed_query_weights(e["W_UQ"].T, e["w_uk"])
    d_cq = e["g"]["setup"]["d_cq"]
    assert a.shape == (n_h * d_c, d_cq)
    # the page prints A as [n_h, d'_c, d_c] (row-vector form): the transpose of each block
    blocks = np.stack([a[i * d_c:(i + 1) * d_c].T for i in range(n_h)])
    assert list(blocks.shape) == g["A_shape"]
    assert np.linalg.matrix_rank(blocks[0]) == g["A0_rank"] == d_h
    q_lat = ref.query_latent_absorbed(e["C_q"], a, n_h)
    two_step = ref.absorb_q(e["q_c"], np.zeros((e["T"], n_h, 0)), np.arange(e["T"]), e["w_uk"])
    assert np.max(np.abs(q_lat - two_step)) < 1e-12
    # and the page's printed score through it
    S = np.einsum("tic,jc->tji", q_lat, e["C_kv"])
    assert abs(S[3, 1, 0] - g["S_naive_t3_j1_h0"]) < 1e-12


def test_absorbed_query_weights_brute_force():
    rng = np.random.default_rng(43)
    n_h, d_h, d_c, d_cq = 2, 3, 4, 5
    w_uq = rng.normal(size=(n_h * d_h, d_cq))
    w_uk = rng.normal(size=(n_h, d_h, d_c))
    a = ref.absorbed_query_weights(w_uq, w_uk)
    for i in range(n_h):
        for c in range(d_c):
            for m in range(d_cq):
                want = sum(w_uk[i, k, c] * w_uq[i * d_h + k, m] for k in range(d_h))
                assert abs(a[i * d_c + c, m] - want) < 1e-12


def test_absorbed_output_weights_brute_force():
    rng = np.random.default_rng(44)
    n_h, d_v, d_c, d = 2, 3, 4, 5
    w_o = rng.normal(size=(d, n_h * d_v))
    w_uv = rng.normal(size=(n_h, d_v, d_c))
    b = ref.absorbed_output_weights(w_o, w_uv)
    for m in range(d):
        for i in range(n_h):
            for c in range(d_c):
                want = sum(w_o[m, i * d_v + k] * w_uv[i, k, c] for k in range(d_v))
                assert abs(b[m, i * d_c + c] - want) < 1e-12
