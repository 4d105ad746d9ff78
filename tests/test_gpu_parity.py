"""GPU parity: every libmla call against the CPU oracle, through the C ABI.

Per call (diagnostic, each fed the GPU's own inputs to that call):
  append -> cache rows at this step's slots vs oracle RMSNorm/RoPE rows
  absorb -> q_lat vs oracle latent query
  decode -> o_lat, lse vs oracle absorbed attention over the GPU cache rows
  out    -> out vs oracle per-head W^UV
End to end (graded): out vs the non-absorbed fp64 oracle fed the raw inputs.
Bar: max|err| <= tol * max|ref| with tol = 1e-5 (fp32), 2e-2 (bf16),
6e-2 (fp8).  Small shapes are checked on every (request, head); the full
workload sizes are checked on sampled requests and heads.
"""

import math

import numpy as np
import pytest
import torch

from oracle import codecs
from oracle import mla_ref as ref
from tests import oracle_views as ov

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mla_latent_kv_18_amd.inputs import WORKLOADS, generate
    from mla_latent_kv_18_amd.step import DeviceStep


def _host(t, fmt):
    t = t.detach().cpu()
    if fmt == "bf16":
        return codecs.bf16_decode(t.view(torch.int16).numpy().view(np.uint16))
    if fmt == "fp8":
        return codecs.e4m3_decode(t.numpy())
    return t.numpy().astype(np.float64)


def _gpu_raw_rows(step, b, T):
    """Stored rows 0..T-1 of request b as the GPU holds them, and their scales."""
    w = step.w
    nb = (T + w.block_size - 1) // w.block_size
    blocks = step.block_table[b, :nb].long()
    width = w.row_dim if w.dtype in ("f32", "bf16") else w.row_bytes
    raw = step.cache[blocks].reshape(-1, width)[:T]
    sc = None
    if step.cache_scale is not None:
        sc = step.cache_scale[blocks].reshape(-1)[:T].cpu().numpy().astype(np.float64)
    return raw, sc


def _gpu_rows(step, b, T):
    w = step.w
    raw, sc = _gpu_raw_rows(step, b, T)
    if w.dtype in ("f32", "bf16"):
        return _host(raw, w.dtype)
    return ov.decode_rows(raw.cpu().numpy(), sc, w.dtype, w.d_c, w.row_dim)


def _q_fmt(w):
    return "fp8" if w.dtype == "fp8" else ("f32" if w.dtype == "f32" else "bf16")


E2M1_BOUNDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def check_fp4_rows(raw, exact):
    """Stored MX FP4 rows against the oracle's quantisation of the exact rows.
    The kernel rounds from fp32 values and the oracle from fp64 ones, so a
    scale may differ where a block maximum sits at a power of two and a code
    where x / scale sits at a rounding boundary; everything else is equal,
    and the padding is zero."""
    D = exact.shape[1]
    codes = codecs.unpack_nibbles(raw[:, :D // 2], D).astype(np.int64)
    sb = raw[:, D // 2:D // 2 + D // 32].astype(np.int64)
    assert not np.any(raw[:, D // 2 + D // 32:]), "padding"
    oc, osb = codecs.mx_fp4_quantize_rows(exact)
    blocks = np.abs(exact).reshape(exact.shape[0], -1, 32)
    amax = blocks.max(axis=-1)
    with np.errstate(divide="ignore"):
        l2 = np.log2(np.where(amax > 0, amax, 1.0))
    near_pow2 = np.abs(l2 - np.round(l2)) < 1e-4
    same_scale = sb == osb
    assert np.all(same_scale | near_pow2), "block scales"
    y = np.abs(exact) / np.repeat(codecs.e8m0_decode(osb), 32, axis=1)
    near_tie = np.min(np.abs(y[..., None] - E2M1_BOUNDS) / E2M1_BOUNDS, axis=-1) < 1e-3
    both_zero = ((codes & 7) == 0) & ((oc.astype(np.int64) & 7) == 0)
    ok = (codes == oc) | near_tie | both_zero | ~np.repeat(same_scale, 32, axis=1)
    assert ok.all(), "E2M1 codes"


def check_request(step, gen, b, heads, tol, lse_tol):
    w = step.w
    T = int(gen["seq_lens"][b])
    sl = slice(b * w.q_len, (b + 1) * w.q_len)
    act = w.act_dtype
    _, wuk, wuv, _ = ov.weights(gen)
    # append
    start, c, kr = ov.new_rows(gen, b)
    rows = _gpu_rows(step, b, T)
    if T > start:
        if w.dtype == "fp4":
            raw, _ = _gpu_raw_rows(step, b, T)
            check_fp4_rows(raw[start:].cpu().numpy(), np.concatenate([c, kr], axis=1))
        else:
            lat_tol = ov.TOL["fp8"] if w.dtype == "fp8kr" else tol   # e4m3 latent
            assert ov.rel_err(rows[start:, :w.d_c], c) <= lat_tol, "append latent"
            if w.d_r > 0:
                assert ov.rel_err(rows[start:, w.d_c:], kr) <= tol, "append rope key"
    # absorb
    q_nope = ov.f64(gen["q_nope"], act)[sl]
    q_pe = ov.f64(gen["q_pe"], act)[sl]
    q_pos = gen["q_positions"][sl]
    q_lat_ref = ref.absorb_q(q_nope, q_pe, q_pos, wuk)
    if w.dtype == "fp8":   # two planes: row = scale * (hi + lo / 16)
        planes = _host(step.q_lat[sl], "fp8")
        D = w.row_dim
        q_lat = (planes[..., :D] + planes[..., D:] / 16.0) * \
            step.q_scale[sl].cpu().numpy().astype(np.float64)[..., None]
    else:
        q_lat = _host(step.q_lat[sl], _q_fmt(w))
    assert ov.rel_err(q_lat[:, heads], q_lat_ref[:, heads]) <= tol, "absorb q"
    # decode, fed the GPU's q_lat and cache rows
    o_ref, lse_ref = ref.decode_absorbed(q_lat[:, heads], q_pos, rows[:, :w.d_c], rows[:, w.d_c:],
                                         w.softmax_scale)
    o_lat = _host(step.o_lat[sl], act)
    lse = step.lse[sl].cpu().numpy().astype(np.float64)
    assert ov.rel_err(o_lat[:, heads], o_ref) <= tol, "decode o_lat"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse[:, heads]), fin), "decode lse finiteness"
    if fin.any():
        assert np.max(np.abs(lse[:, heads][fin] - lse_ref[fin])) <= lse_tol, "decode lse"
    # out proj, fed the GPU's o_lat
    out = _host(step.out[sl], act)
    assert ov.rel_err(out[:, heads], ref.out_proj(o_lat, wuv)[:, heads]) <= tol, "out proj"
    # end to end against the non-absorbed oracle (for the FP4 and fp8-latent
    # caches over every row as stored, this step's too: the oracle reads the
    # cache it is given)
    if w.dtype in ("fp4", "fp8kr"):
        want = ref.attention_nonabsorbed(q_nope, q_pe, q_pos, rows[:, :w.d_c], rows[:, w.d_c:], wuk, wuv,
                                         w.softmax_scale, heads=heads)
    else:
        want = ov.reference_output(gen, b, heads=heads)
    assert ov.rel_err(out[:, heads], want) <= tol, "end to end"


def _run(w, split_tokens=0, mode="planned", gen=None):
    gen = generate(w) if gen is None else gen
    step = DeviceStep(gen, split_tokens=split_tokens, mode=mode)
    step.run()
    torch.cuda.synchronize()
    return gen, step


def test_tiny_f32_end_to_end():
    w = WORKLOADS["tiny_f32"]
    gen, step = _run(w)
    check_request(step, gen, 0, list(range(w.n_h)), ov.TOL["f32"], 1e-5)


SMALL_BF16 = {
    "v3_ragged_tails": dict(batch=3, lens=(1, 100, 257), shuffle=True),
    "v3_two_queries": dict(batch=2, lens=(70, 129), q_len=2),
    "kimi_heads64": dict(n_h=64, batch=3, lens=(33, 64, 300), shuffle=True),
    "kimi_heads64_q2": dict(n_h=64, batch=2, lens=(2, 200), q_len=2),
    # a batch of 8: each request's chunks share an XCD and so do its merge rows
    "v3_batch8_grouped": dict(batch=8, lens=(1, 2, 63, 64, 65, 500, 1000, 2048), shuffle=True),
}


@pytest.mark.parametrize("mode", ["planned", "uniform"])
@pytest.mark.parametrize("name", sorted(SMALL_BF16))
@pytest.mark.parametrize("split_tokens", [0, 64, 128])
def test_small_bf16_all_heads(name, split_tokens, mode):
    w = WORKLOADS["v3_bs64_ctx4k"].scaled(name=name, seed=7, **SMALL_BF16[name])
    gen, step = _run(w, split_tokens, mode)
    for b in range(w.batch):
        check_request(step, gen, b, list(range(w.n_h)), ov.TOL["bf16"], 2e-2)


# Split invariance bar: two results that differ only in where the context
# is cut each carry one bf16 rounding of o_lat (2^-9 relative), of the bf16
# partials (2^-9) and of the bf16 softmax numerators P taken against a
# different reference point (2^-9): 4 x 2^-9 = 2^-7 of max|o_lat|.
INVARIANCE = 2.0 ** -7


def test_split_and_paging_invariance_and_determinism():
    w = WORKLOADS["v3_bs64_ctx4k"].scaled(name="inv", batch=2, lens=(1000, 777), seed=8)
    gen, step = _run(w)
    base = step.o_lat.clone()
    step.decode()
    torch.cuda.synchronize()
    assert torch.equal(step.o_lat, base), "decode is not bitwise deterministic"
    bound = INVARIANCE * base.float().abs().max().item()
    for mode in ("planned", "uniform"):
        for st in (0, 64, 256, 512):
            step.decode(split_tokens=st, mode=mode)
            torch.cuda.synchronize()
            d = (step.o_lat.float() - base.float()).abs().max().item()
            assert d <= bound, f"{mode} split {st} changes o_lat by {d}"
    # same rows under a permuted block table
    ws = w.scaled(shuffle=True)
    gen2 = generate(ws)
    step2 = DeviceStep(gen2)
    step2.run()
    torch.cuda.synchronize()
    d = (step2.o_lat.float() - base.float()).abs().max().item()
    assert d <= 1e-6, f"block-table permutation changes o_lat by {d}"


@pytest.mark.parametrize("mode", ["planned", "uniform"])
@pytest.mark.parametrize("lens", [(0, 50), (0, 50, 0, 1, 100, 0, 64, 65)])
def test_empty_request_gives_zero_and_neg_inf(lens, mode):
    # the batch of 8 runs with each request's chunks and merge rows on one XCD
    w = WORKLOADS["v3_bs64_ctx4k"].scaled(name="empty", batch=len(lens), lens=lens, seed=9)
    for st in (0, 64):
        gen, step = _run(w, st, mode)
        for b, T in enumerate(lens):
            if T == 0:
                assert torch.all(step.o_lat[b].float() == 0).item()
                assert torch.all(torch.isneginf(step.lse[b])).item()
            else:
                check_request(step, gen, b, list(range(w.n_h)), ov.TOL["bf16"], 2e-2)


SMALL_FP8 = {
    "fp8_q2_ragged": dict(batch=3, lens=(1, 100, 257), shuffle=True),
    "fp8_q2_tiles": dict(batch=2, lens=(64, 130)),
    "fp8_q1": dict(batch=2, lens=(65, 300), q_len=1),
    "fp8_heads64_q2": dict(n_h=64, batch=2, lens=(2, 200), shuffle=True),
    "fp8_heads64_q1": dict(n_h=64, batch=2, lens=(129, 33), q_len=1),
}


@pytest.mark.parametrize("mode", ["planned", "uniform"])
@pytest.mark.parametrize("name", sorted(SMALL_FP8))
@pytest.mark.parametrize("split_tokens", [0, 64, 128])
def test_small_fp8_all_heads(name, split_tokens, mode):
    w = WORKLOADS["v3_fp8_bs4_ctx128k_q2"].scaled(name=name, seed=11, **SMALL_FP8[name])
    gen, step = _run(w, split_tokens, mode)
    for b in range(w.batch):
        check_request(step, gen, b, list(range(w.n_h)), ov.TOL["fp8"], 2e-2)


# Cache variants: MX FP4 rows, an e4m3 latent beside a bf16 RoPE key, and
# no RoPE part (d_R = 0), on both decode workgroup shapes (128 and 64 rows).
SMALL_VARIANTS = {
    "fp4_ragged": ("v3_fp4_bs64_ctx4k", dict(batch=3, lens=(1, 100, 257), shuffle=True)),
    "fp4_heads64_q2": ("v3_fp4_bs64_ctx4k", dict(n_h=64, batch=2, lens=(2, 200), q_len=2)),
    "fp8kr_ragged": ("v3_fp8kr_bs64_ctx4k", dict(batch=3, lens=(1, 100, 257), shuffle=True)),
    "fp8kr_heads64": ("v3_fp8kr_bs64_ctx4k", dict(n_h=64, batch=3, lens=(33, 64, 300))),
    "nope_ragged": ("nope_bs64_ctx4k", dict(batch=3, lens=(1, 100, 257), shuffle=True)),
    "nope_heads64_q2": ("nope_bs64_ctx4k", dict(n_h=64, batch=2, lens=(2, 200), q_len=2)),
    "nope_batch8": ("nope_bs64_ctx4k", dict(batch=8, lens=(0, 2, 63, 64, 65, 500, 1000, 2048))),
    "nope_q2": ("nope_bs64_ctx4k", dict(batch=2, lens=(3, 300), q_len=2)),
    "fp4_batch8": ("v3_fp4_bs64_ctx4k", dict(batch=8, lens=(0, 2, 63, 64, 65, 97, 161, 2048))),
    "fp4_q2": ("v3_fp4_bs64_ctx4k", dict(batch=2, lens=(3, 300), q_len=2)),
    "fp8kr_batch8": ("v3_fp8kr_bs64_ctx4k", dict(batch=8, lens=(0, 2, 63, 64, 65, 97, 161, 2048))),
    "fp8kr_q2": ("v3_fp8kr_bs64_ctx4k", dict(batch=2, lens=(3, 300), q_len=2)),
}


@pytest.mark.parametrize("mode", ["planned", "uniform"])
@pytest.mark.parametrize("name", sorted(SMALL_VARIANTS))
@pytest.mark.parametrize("split_tokens", [0, 64, 128])
def test_small_cache_variants_all_heads(name, split_tokens, mode):
    base, over = SMALL_VARIANTS[name]
    w = WORKLOADS[base].scaled(name=name, seed=17, **over)
    gen, step = _run(w, split_tokens, mode)
    for b in range(w.batch):
        if int(gen["seq_lens"][b]) == 0:
            assert torch.all(step.o_lat[b * w.q_len:(b + 1) * w.q_len].float() == 0).item()
            continue
        check_request(step, gen, b, list(range(w.n_h)), ov.TOL[w.dtype], 2e-2)


FULL = ["v3_bs64_ctx4k", "v3_paged_bs16_ctx32k", "kimi_k2_ragged_bs32", "v3_fp8_bs4_ctx128k_q2",
        "v3_fp4_bs64_ctx4k", "v3_fp8kr_bs64_ctx4k", "nope_bs64_ctx4k"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    """In the launch configuration bench.py times (planned decode)."""
    w = WORKLOADS[name]
    gen, step = _run(w)
    rng = np.random.default_rng(100)
    reqs = sorted(set([0, w.batch - 1, int(rng.integers(w.batch))]))
    if name.startswith("kimi"):
        reqs = sorted(set(reqs + [int(np.argmax(gen["seq_lens"])), int(np.argmin(gen["seq_lens"]))]))
    for b in reqs:
        heads = sorted(set([0, w.n_h - 1] + [int(x) for x in rng.integers(w.n_h, size=2)]))
        check_request(step, gen, b, heads, ov.TOL[w.dtype], 2e-2)


def test_graph_replay_matches_eager():
    """A captured step replays the same kernels: every replay, with eager
    work and synchronisations between replays, equals the eager step
    bitwise (the path is deterministic)."""
    w = WORKLOADS["v3_bs64_ctx4k"].scaled(name="graph", batch=3, lens=(300, 77, 1000), shuffle=True, seed=12)
    gen, step = _run(w, 256)
    ref = [step.out.clone(), step.o_lat.clone(), step.lse.clone()]
    g = step.capture()
    for _ in range(3):
        step.out.zero_()
        step.o_lat.zero_()
        step.lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((step.out, step.o_lat, step.lse), ref):
            assert torch.equal(got, want)
        step.decode(split_tokens=64)   # eager work between replays
        torch.cuda.synchronize()
    gd = step.capture(decode_only=True)
    step.o_lat.zero_()
    gd.replay()
    torch.cuda.synchronize()
    assert torch.equal(step.o_lat, ref[1])


def test_planned_equals_uniform_on_full_ragged_workload():
    """The balanced plan and the uniform split cut the Kimi-like ragged
    context differently; both agree to the invariance bar on every row."""
    w = WORKLOADS["kimi_k2_ragged_bs32"]
    gen, step = _run(w)
    planned = step.o_lat.float().clone()
    step.decode(mode="uniform")
    torch.cuda.synchronize()
    d = (step.o_lat.float() - planned).abs().max().item()
    assert d <= INVARIANCE * planned.abs().max().item()


# ---------------------------------------------------------------------------
# Peaked attention: keys planted after the first tile of a chunk whose score
# exceeds that tile's maximum by more than 2^64 (and 2^128) in the exponent.
# Every decode kernel then redoes the chunk with the exact chunk maximum as
# its softmax reference.  Checked per call: o_lat and lse against the
# absorbed oracle fed the GPU's latent queries and cache rows (with logits
# this large, the rounding of q_lat itself moves the softmax weights, so the
# end-to-end comparison is not the meaningful one here).
# ---------------------------------------------------------------------------
def plant_peaks(gen, plants, seed):
    """plants: (request, position, query t, head, score) -> overwrite the
    pre-filled row at `position` so that (query t, head) scores about
    `score` (natural log units) against it: row = score/scale * q / |q|^2
    plus N(0, 1) noise, with q the oracle's latent query."""
    w = gen["workload"]
    rng = np.random.default_rng(seed)
    _, wuk, _, _ = ov.weights(gen)
    q_nope = ov.f64(gen["q_nope"], w.act_dtype)
    q_pe = ov.f64(gen["q_pe"], w.act_dtype)
    q_lat = ref.absorb_q(q_nope, q_pe, gen["q_positions"], wuk)
    from mla_latent_kv_18_amd.inputs import to_bf16_bits, to_fp4_rows, to_fp8_rows, to_fp8kr_rows
    for b, pos, t, h, score in plants:
        assert pos < int(gen["seq_lens"][b]) - w.q_len, "plant a pre-filled row"
        q = q_lat[b * w.q_len + t, h]
        row = score / w.softmax_scale * q / (q @ q) + rng.standard_normal(q.shape)
        blk = gen["block_table"][b, pos // w.block_size]
        if w.dtype == "bf16":
            gen["pool"][blk, pos % w.block_size] = to_bf16_bits(row[None])[0]
        elif w.dtype == "fp4":
            gen["pool"][blk, pos % w.block_size] = to_fp4_rows(row[None].astype(np.float32))[0]
        elif w.dtype == "fp8kr":
            codes, sc = to_fp8kr_rows(row[None].astype(np.float32), w.d_c)
            gen["pool"][blk, pos % w.block_size] = codes[0]
            gen["pool_scale"][blk, pos % w.block_size] = sc[0]
        else:
            codes, sc = to_fp8_rows(row[None].astype(np.float32))
            gen["pool"][blk, pos % w.block_size] = codes[0]
            gen["pool_scale"][blk, pos % w.block_size] = sc[0]
    return gen


def check_decode_call(step, gen, b, tol, lse_tol=2e-2):
    w = step.w
    T = int(gen["seq_lens"][b])
    sl = slice(b * w.q_len, (b + 1) * w.q_len)
    rows = _gpu_rows(step, b, T)
    if w.dtype == "fp8":
        planes = _host(step.q_lat[sl], "fp8")
        D = w.row_dim
        q_lat = (planes[..., :D] + planes[..., D:] / 16.0) * \
            step.q_scale[sl].cpu().numpy().astype(np.float64)[..., None]
    else:
        q_lat = _host(step.q_lat[sl], _q_fmt(w))
    o_ref, lse_ref = ref.decode_absorbed(q_lat, gen["q_positions"][sl], rows[:, :w.d_c], rows[:, w.d_c:],
                                         w.softmax_scale)
    o_lat = _host(step.o_lat[sl], w.act_dtype)
    lse = step.lse[sl].cpu().numpy().astype(np.float64)
    assert ov.rel_err(o_lat, o_ref) <= tol, "decode o_lat"
    assert np.max(np.abs(lse - lse_ref)) <= lse_tol, "decode lse"
    return float(np.max(lse_ref))


PEAK_CASES = {   # base workload, overrides: the four decode kernels and the cache-variant kernels
    "fp4_h128": ("v3_fp4_bs64_ctx4k", dict(batch=2, lens=(400, 700))),
    "fp8kr_h64_q2": ("v3_fp8kr_bs64_ctx4k", dict(n_h=64, batch=2, lens=(400, 700), q_len=2)),
    "fp8kr_h128": ("v3_fp8kr_bs64_ctx4k", dict(batch=2, lens=(400, 700))),
    "nope_h64": ("nope_bs64_ctx4k", dict(n_h=64, batch=2, lens=(400, 700))),
    "bf16_pipelined_h128": ("v3_bs64_ctx4k", dict(batch=2, lens=(400, 700))),
    "bf16_pipelined_h128_q2": ("v3_bs64_ctx4k", dict(batch=2, lens=(400, 700), q_len=2)),
    "bf16_plain_h64": ("v3_bs64_ctx4k", dict(n_h=64, batch=2, lens=(400, 700))),
    "fp8_pipelined_h128_q2": ("v3_fp8_bs4_ctx128k_q2", dict(batch=2, lens=(400, 700))),
    "fp8_plain_h64_q1": ("v3_fp8_bs4_ctx128k_q2", dict(n_h=64, batch=2, lens=(400, 700), q_len=1)),
}


@pytest.mark.parametrize("mode", ["planned", "uniform"])
@pytest.mark.parametrize("split_tokens", [0, 64, 128])
@pytest.mark.parametrize("score", [60.0, 120.0])
@pytest.mark.parametrize("case", sorted(PEAK_CASES))
def test_peaked_logits_take_the_second_pass(case, score, split_tokens, mode):
    base, over = PEAK_CASES[case]
    w = WORKLOADS[base].scaled(name="peak", seed=13, **over)
    gen = generate(w)
    last = w.q_len - 1
    # position % 64 = 36 and % 128 = 100: a later tile of its chunk for 32- and
    # 64-token tiles and chunks of 64, 128, 256 or more rows.  A few keys at
    # nearly the same height keep the softmax from being one-hot; heads in
    # different waves and both queries get their own peaks.
    plants = []
    for b in range(w.batch):
        for k, (t, h) in enumerate([(0, 5), (last, w.n_h - 3), (0, w.n_h // 2 + 1)]):
            p0 = 100 + 256 * k
            if p0 + 2 < int(gen["seq_lens"][b]) - w.q_len:
                plants += [(b, p0, t, h, score), (b, p0 + 1, t, h, score - 1.0), (b, p0 + 2, t, h, score + 0.5)]
    plant_peaks(gen, plants, seed=14)
    gen, step = _run(w, split_tokens, mode, gen=gen)
    top = max(check_decode_call(step, gen, b, ov.TOL[w.dtype]) for b in range(w.batch))
    # the planted keys dominate: far above the unit-variance logits of the rest
    assert top > 0.9 * score


@pytest.mark.parametrize("base,over", [
    ("v3_bs64_ctx4k", dict(batch=3, lens=(1, 100, 257), shuffle=True)),
    ("v3_fp8_bs4_ctx128k_q2", dict(batch=2, lens=(64, 130))),
    ("v3_fp4_bs64_ctx4k", dict(n_h=64, batch=40, lens=tuple(range(10, 410, 10)))),
    ("nope_bs64_ctx4k", dict(batch=2, lens=(70, 129), q_len=2)),
    ("tiny_f32", dict()),
])
def test_fused_append_absorb_equals_the_two_calls(base, over):
    """mla_append_absorb (one launch for the down-projection and the latent
    query) writes the same cache rows and latent queries as the two calls."""
    w = WORKLOADS[base].scaled(name="fused", seed=19, **over)
    gen = generate(w)
    a = DeviceStep(gen, fused=True)
    b = DeviceStep(gen, fused=False)
    a.run()
    b.run()
    torch.cuda.synchronize()
    assert torch.equal(a.cache, b.cache)
    assert torch.equal(a.q_lat, b.q_lat)
    if a.q_scale is not None:
        assert torch.equal(a.q_scale, b.q_scale)
    if a.cache_scale is not None:
        assert torch.equal(a.cache_scale, b.cache_scale)
    assert torch.equal(a.out, b.out)
    check_request(a, gen, 0, list(range(w.n_h)), ov.TOL[w.dtype], 2e-2)


@pytest.mark.parametrize("nbytes", [36864 * 3, 36864 * 8192 + 16 * 5])
def test_hbm_read_probe_reads_every_word_once(nbytes):
    """The register form of the read probe XOR-folds every 32-bit word it
    loads: folded over the workgroups, it equals the XOR of the buffer
    (a word read twice or skipped would change it); the copy form runs on
    whole tiles."""
    import mla_latent_kv_18_amd as mla
    rng = np.random.default_rng(nbytes % 1000)
    words = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(mla.PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    mla.hbm_read_probe(buf, 0, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
    tiles = buf[: (nbytes // 36864) * 36864 // 4]
    mla.hbm_read_probe(tiles, 1)
    torch.cuda.synchronize()


BLOCK_CASES = {   # 128- and 256-token cache blocks, shuffled tables: tiles sit at offsets 0..224 of a block
    "bf16_h128": ("v3_bs64_ctx4k", dict(batch=3, lens=(1, 300, 1000))),
    "bf16_h64": ("v3_bs64_ctx4k", dict(n_h=64, batch=2, lens=(130, 700))),
    "fp8_h128_q2": ("v3_fp8_bs4_ctx128k_q2", dict(batch=2, lens=(130, 700))),
    "fp4_h128": ("v3_fp4_bs64_ctx4k", dict(batch=2, lens=(97, 700))),
    "fp8kr_h128": ("v3_fp8kr_bs64_ctx4k", dict(batch=3, lens=(2, 333, 1000))),
    "fp8kr_h64": ("v3_fp8kr_bs64_ctx4k", dict(n_h=64, batch=2, lens=(65, 500))),
    "nope_h128": ("nope_bs64_ctx4k", dict(batch=2, lens=(64, 545))),
}


@pytest.mark.parametrize("block_size", [128, 256])
@pytest.mark.parametrize("split_tokens", [0, 128])
@pytest.mark.parametrize("case", sorted(BLOCK_CASES))
def test_larger_cache_blocks(case, split_tokens, block_size):
    base, over = BLOCK_CASES[case]
    w = WORKLOADS[base].scaled(name="blocks", seed=23, block_size=block_size, shuffle=True, **over)
    gen, step = _run(w, split_tokens, "planned")
    for b in range(w.batch):
        check_request(step, gen, b, list(range(w.n_h)), ov.TOL[w.dtype], 2e-2)
