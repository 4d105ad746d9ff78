"""Test helpers that turn generated inputs (storage form) into the oracle's
float64 views and evaluate the oracle on them.  Uses only oracle/ and the
shared input generator; nothing from the HIP path."""

import numpy as np

from oracle import codecs
from oracle import mla_ref as ref


def f64(a, fmt):
    if fmt == "f32":
        return np.asarray(a, dtype=np.float64)
    if fmt == "bf16":
        return codecs.bf16_decode(a)
    raise ValueError(fmt)


def decode_rows(raw, scales, fmt, d_c=512, D=576):
    """Stored rows [n, row bytes or elements] (+ per-row scales) -> float64
    [n, D], exactly as a reader of the stored bits reconstructs them."""
    if fmt == "fp8":
        return codecs.e4m3_dequantize_rows(raw, scales)
    if fmt == "fp4":       # [D/2 bytes of E2M1 codes | D/32 E8M0 scales | padding]
        codes = codecs.unpack_nibbles(raw[:, :D // 2], D)
        return codecs.mx_fp4_dequantize_rows(codes, raw[:, D // 2:D // 2 + D // 32])
    if fmt == "fp8kr":     # [d_c e4m3 codes | d_R bf16 values]
        lat = codecs.e4m3_dequantize_rows(raw[:, :d_c], scales)
        kr = codecs.bf16_decode(np.ascontiguousarray(raw[:, d_c:]).view(np.uint16))
        return np.concatenate([lat, kr], axis=1)
    return f64(raw, fmt)


def stored_rows(pool, pool_scale, table_row, T, bs, fmt, d_c=512, D=576):
    """Rows 0..T-1 of one request as float64, exactly as stored."""
    raw = ref.gather_rows(pool, table_row, T, bs)
    sc = ref.gather_rows(pool_scale[..., None], table_row, T, bs)[:, 0] if pool_scale is not None else None
    return decode_rows(raw, sc, fmt, d_c, D)


def weights(gen):
    w = gen["workload"]
    act = w.act_dtype
    return (f64(gen["w_dkv_kr"], act), f64(gen["w_uk"], act), f64(gen["w_uv"], act),
            np.asarray(gen["gamma"], np.float64))


def new_rows(gen, b):
    """Oracle rows appended this step for request b (fp64, from hidden states):
    returns (first position, c [n, d_c], k^R [n, d_R])."""
    w = gen["workload"]
    wd, _, _, gamma = weights(gen)
    h = f64(gen["h"], w.act_dtype)
    T = int(gen["seq_lens"][b])
    if w.all_rows_appended:
        hb = h[:T]
        pos = np.arange(T)
    else:
        n = min(T, w.q_len)
        hb = h[b * w.q_len + (w.q_len - n): (b + 1) * w.q_len]
        pos = np.arange(T - n, T)
    c, kr = ref.latent_rows(hb, wd, gamma, pos, w.d_c, 1e-6, 10000.0)
    return (T - len(pos)), c, kr


def reference_cache(gen, b):
    """All T rows of request b as the method defines them: pre-filled rows as
    stored, this step's rows computed in fp64 by the oracle."""
    w = gen["workload"]
    T = int(gen["seq_lens"][b])
    rows = stored_rows(gen["pool"], gen["pool_scale"], gen["block_table"][b], T, w.block_size, w.dtype, w.d_c,
                       w.row_dim)
    start, c, kr = new_rows(gen, b)
    rows[start:, :w.d_c] = c
    rows[start:, w.d_c:] = kr
    return rows


def reference_output(gen, b, heads=None):
    """Non-absorbed fp64 MLA output of request b: [q_len, len(heads), d_v]."""
    w = gen["workload"]
    _, wuk, wuv, _ = weights(gen)
    rows = reference_cache(gen, b)
    sl = slice(b * w.q_len, (b + 1) * w.q_len)
    q_nope = f64(gen["q_nope"], w.act_dtype)[sl]
    q_pe = f64(gen["q_pe"], w.act_dtype)[sl]
    q_pos = gen["q_positions"][sl]
    return ref.attention_nonabsorbed(q_nope, q_pe, q_pos, rows[:, :w.d_c], rows[:, w.d_c:], wuk, wuv,
                                     w.softmax_scale, heads=heads)


def rel_err(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    denom = np.max(np.abs(want))
    return float(np.max(np.abs(got - want)) / (denom if denom > 0 else 1.0))


# fp4 and fp8kr caches are read exactly as stored (the oracle uses the stored
# values) and attended in bf16 arithmetic: the bf16 bar.
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "fp4": 2e-2, "fp8kr": 2e-2}
