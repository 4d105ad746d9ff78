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
