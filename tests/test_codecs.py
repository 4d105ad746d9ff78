"""Pins for the oracle's number-format codecs: exhaustive agreement with
torch's CPU dtypes (a library implementation of the same public formats) and
the defining properties of each format.  CPU only."""

import numpy as np
import torch

from oracle import codecs


def test_bf16_decode_all_codes_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ours = codecs.bf16_decode(bits)
    theirs = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == theirs) | (np.isnan(ours) & np.isnan(theirs))
    assert same.all()


def test_bf16_encode_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.normal(size=200000).astype(np.float32),
        (rng.normal(size=50000) * 1e-38).astype(np.float32),       # subnormal range
        (rng.normal(size=50000) * 1e37).astype(np.float32),
        # exact ties between neighbouring bf16 values
        (np.arange(1, 20000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 3.0e38, -3.39e38], dtype=np.float32),
    ])
    ours = codecs.bf16_encode(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_bf16_round_properties():
    assert codecs.bf16_round(1.0 + 2 ** -8) == 1.0                     # tie -> even (1.0)
    assert codecs.bf16_round(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6       # tie -> even (odd below)
    assert codecs.bf16_round(1.0 + 2 ** -8 + 2 ** -20) == 1.0 + 2 ** -7
    assert np.isinf(codecs.bf16_round(3.4e38))


def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == theirs) | (np.isnan(ours) & np.isnan(theirs))
    assert same.all()
    assert np.nanmax(ours) == 448.0 and np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert ours[1] == 2.0 ** -9                                          # smallest subnormal


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.normal(size=100000) * 50, rng.normal(size=20000) * 0.01,
                        rng.uniform(-448, 448, size=20000)]).astype(np.float32)
    # every midpoint between adjacent finite codes (ties)
    vals = np.sort(codecs.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ours = codecs.e4m3_encode(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e4m3_saturates_and_roundtrips():
    assert codecs.e4m3_round(1000.0) == 448.0 and codecs.e4m3_round(-1e9) == -448.0
    assert codecs.e4m3_encode(np.array([np.nan]))[0] == 0x7F
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    back = codecs.e4m3_encode(codecs.e4m3_decode(codes))
    # +0 and -0 both decode to zero; every other finite code round-trips
    nz = codecs.e4m3_decode(codes) != 0
    assert np.array_equal(back[nz], codes[nz])


def test_per_row_fp8_quantisation():
    rng = np.random.default_rng(2)
    x = rng.normal(size=(64, 576))
    x[3] = 0.0
    codes, scales = codecs.e4m3_quantize_rows(x)
    assert scales.dtype == np.float32 and scales[3] == 1.0
    back = codecs.e4m3_dequantize_rows(codes, scales)
    # the largest element of each row maps to +-448 exactly
    amax_code = np.max(np.abs(codecs.e4m3_decode(codes)), axis=1)
    assert np.all(amax_code[np.arange(64) != 3] == 448.0)
    # relative error of e4m3 rounding is at most 2^-4 for normals
    big = np.abs(x) > 2.0 ** -6 * scales[:, None] * 2
    rel = np.abs(back - x)[big] / np.abs(x)[big]
    assert rel.max() <= 2.0 ** -4 + 1e-6


# OCP MX v1.0, FP4 E2M1 element encodings (positive half; bit 3 is the sign)
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_all_codes_matches_the_format_table():
    ours = codecs.e2m1_decode(np.arange(16))
    assert list(ours[:8]) == E2M1_TABLE
    assert list(-ours[8:]) == E2M1_TABLE and np.signbit(ours[8])   # code 8 is -0


def test_e2m1_encode_round_trips_and_rounds_to_even():
    codes = np.arange(16)
    assert np.array_equal(codecs.e2m1_encode(codecs.e2m1_decode(codes)), codes)
    # midpoints between neighbours go to the code with an even mantissa bit
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for x, want in ties.items():
        assert codecs.e2m1_round(x) == want and codecs.e2m1_round(-x) == -want
    assert codecs.e2m1_round(0.26) == 0.5 and codecs.e2m1_round(5.01) == 6.0
    assert codecs.e2m1_round(7.0) == 6.0 and codecs.e2m1_round(1e30) == 6.0      # saturation
    # brute force: every value goes to a nearest representable value
    x = np.linspace(-8, 8, 20001)
    r = codecs.e2m1_round(x)
    grid = np.array(sorted(set(E2M1_TABLE + [-v for v in E2M1_TABLE])))
    best = np.min(np.abs(np.clip(x, -6, 6)[:, None] - grid[None, :]), axis=1)
    assert np.allclose(np.abs(np.clip(x, -6, 6) - r), best, atol=1e-12)


def test_e8m0_decode_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    ours = codecs.e8m0_decode(b)
    theirs = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    same = (ours == theirs) | (np.isnan(ours) & np.isnan(theirs))
    assert same.all()


def test_mx_fp4_block_scale_rule_and_error_bound():
    rng = np.random.default_rng(7)
    x = rng.normal(size=(64, 576)) * rng.uniform(0.01, 100, size=(64, 1))
    x[3] = 0.0                                                   # an all-zero row
    x[5, :32] = 0.0                                              # an all-zero block
    codes, sb = codecs.mx_fp4_quantize_rows(x)
    assert codes.shape == x.shape and sb.shape == (64, 18)
    blocks = np.abs(x).reshape(64, 18, 32)
    amax = blocks.max(axis=-1)
    scale = codecs.e8m0_decode(sb)
    nz = amax > 0
    # the largest element of a block lands in [4, 8) before saturating at 6
    assert np.all((amax[nz] / scale[nz] >= 4) & (amax[nz] / scale[nz] < 8))
    assert np.all(sb[~nz] == 127)
    y = codecs.mx_fp4_dequantize_rows(codes, sb)
    # error: half a grid step (at most 2 x 2^-2 of the block scale, i.e. 1 scale unit)
    # below the saturation point, and at most 2 scale units above it (8 -> 6)
    err = np.abs(y - x).reshape(64, 18, 32)
    assert np.all(err <= 2.0 * scale[..., None] + 1e-300)
    assert np.all(y[3] == 0) and np.all(y[5, :32] == 0)
    # values exactly on the grid survive
    grid_vals = codecs.mx_fp4_dequantize_rows(codes, sb)
    c2, s2 = codecs.mx_fp4_quantize_rows(grid_vals)
    assert np.array_equal(codecs.mx_fp4_dequantize_rows(c2, s2), grid_vals)


def test_unpack_nibbles_order():
    packed = np.array([[0x21, 0x43, 0xF5]], dtype=np.uint8)
    assert codecs.unpack_nibbles(packed, 6).tolist() == [[1, 2, 3, 4, 5, 15]]
    assert codecs.unpack_nibbles(packed, 5).tolist() == [[1, 2, 3, 4, 5]]


def test_fp8kr_generator_rows_use_power_of_two_scales():
    """The input generator's rows for the e4m3-latent cache: the scale is the
    smallest power of two s with max|latent| / s <= 448, the codes are the
    e4m3 rounding of latent / s, and the RoPE key is the bf16 rounding."""
    import numpy as np
    from mla_latent_kv_18_amd.inputs import to_fp8kr_rows
    from oracle import codecs
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((50, 576)) * np.exp(rng.uniform(-8, 8, size=(50, 1)))).astype(np.float32)
    x[3] = 0.0
    rows, scale = to_fp8kr_rows(x, 512)
    s = scale.astype(np.float64)
    assert np.all(np.frexp(s)[0] == 0.5)
    amax = np.abs(x[:, :512].astype(np.float64)).max(axis=1)
    nz = amax > 0
    assert np.all(amax[nz] / s[nz] <= 448.0) and np.all(amax[nz] / s[nz] > 224.0)
    assert s[3] == 1.0
    lat = codecs.e4m3_decode(rows[:, :512]) * s[:, None]
    want = codecs.e4m3_round(x[:, :512].astype(np.float64) / s[:, None]) * s[:, None]
    assert np.array_equal(lat, want)
    kr = codecs.bf16_decode(rows[:, 512:].copy().view(np.uint16))
    assert np.array_equal(kr, codecs.bf16_round(x[:, 512:].astype(np.float64)))
