"""Pins of the oracle's number-format codecs (CPU only).

Each decode table is checked against something other than itself: the
landmarks the pages print (tests/golden/format_landmarks.txt), an independent
library decoder (torch.float8_e4m3fn), and the pages' exactness argument.
The output roundings are checked exhaustively and against torch's own CPU
conversions.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _landmarks():
    out = {}
    with open(os.path.join(GOLDEN, "format_landmarks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def _sig_bits(x: float) -> int:
    """Number of significand bits of a finite non-zero float."""
    m, _ = math.frexp(abs(x))
    bits = 0
    while m != 0:
        m = m * 2
        bits += 1
        m -= math.floor(m)
    return bits


def test_e4m3fn_all_codes_match_torch_decoder():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = codecs.E4M3FN_TABLE
    assert np.array_equal(np.isnan(lib), np.isnan(ours))
    fin = ~np.isnan(ours)
    assert np.array_equal(lib[fin], ours[fin])
    assert np.array_equal(np.signbit(lib[fin]), np.signbit(ours[fin]))


def test_e4m3fn_landmarks_from_pages():
    lm = _landmarks()
    t = codecs.E4M3FN_TABLE
    finite = t[~np.isnan(t)]
    assert finite.max() == float(lm["e4m3_max"][0])
    assert t[int(lm["e4m3_max_code"][0], 16)] == float(lm["e4m3_max"][0])
    assert finite[finite > 0].min() == float(lm["e4m3_min_positive"][0])
    assert t[int(lm["e4m3_min_positive_code"][0], 16)] == float(lm["e4m3_min_positive"][0])
    nan_codes = sorted(int(v, 16) for v in lm["e4m3_nan_codes"])
    assert sorted(np.nonzero(np.isnan(t))[0].tolist()) == nan_codes
    nbits = int(lm["e4m3_significand_bits"][0])
    assert all(_sig_bits(v) <= nbits for v in finite if v != 0)
    # sign-magnitude: code | 0x80 is the negation
    for b in range(128):
        if not math.isnan(t[b]):
            assert t[b | 0x80] == -t[b]
    # strictly increasing over the positive codes 0..0x7E
    assert np.all(np.diff(t[:0x7F]) > 0)


def test_e2m1_landmarks_from_pages():
    lm = _landmarks()
    t = codecs.E2M1_TABLE
    assert np.abs(t).max() == float(lm["e2m1_max_magnitude"][0])
    assert t[t > 0].min() == float(lm["e2m1_min_positive"][0])
    nz = int(lm["e2m1_negative_zero_code"][0])
    assert t[nz] == 0.0 and np.signbit(t[nz])
    assert not np.signbit(t[0])
    nbits = int(lm["e2m1_significand_bits"][0])
    assert all(_sig_bits(v) <= nbits for v in t if v != 0)
    # 8 magnitudes, strictly increasing with the code, sign bit = bit 3
    assert np.all(np.diff(t[:8]) > 0)
    for c in range(8):
        assert t[c | 8] == -t[c] and np.signbit(t[c | 8])
    # only 8 distinct magnitudes, each a multiple of the smallest one
    mags = t[:8]
    assert np.all(np.mod(mags, 0.5) == 0)


def test_products_exact_in_fp16_and_bf16_and_in_printed_range():
    """[FP4 doc] §4: every E2M1 x E4M3 product is exact in FP16 and BF16 and
    lies in [2^-10, 2688] in magnitude (non-zero, non-NaN products)."""
    lm = _landmarks()
    q = codecs.E2M1_TABLE[:, None]
    s = codecs.E4M3FN_TABLE[None, :]
    p = (q * s).ravel()
    p = p[~np.isnan(p)]
    nz = np.abs(p[p != 0])
    assert nz.max() == float(lm["product_max"][0])
    assert nz.min() == float(lm["product_min_positive"][0])
    as16 = torch.from_numpy(p).to(torch.float16).to(torch.float64).numpy()
    asbf = torch.from_numpy(p).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(as16, p)
    assert np.array_equal(asbf, p)


def test_f16_rounding_round_trip_and_ties():
    # every finite f16 survives f16 -> f32 -> oracle rounding unchanged
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16)
    fin = np.isfinite(v)
    back = codecs.f32_to_f16_bits(v[fin].astype(np.float32))
    assert np.array_equal(back, h[fin])
    # midpoints between consecutive positive finite f16 values: ties to even
    pos = np.arange(0, 0x7C00, dtype=np.uint32)
    lo = pos.astype(np.uint16).view(np.float16).astype(np.float64)
    hi = (pos + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)  # midpoints exact in f32
    got = codecs.f32_to_f16_bits(mid).astype(np.uint32)
    want = np.where(pos % 2 == 0, pos, pos + 1)
    assert np.array_equal(got, want)


def test_f16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # bias toward the f16 range (exponents 100..145) including subnormals
    e = rng.integers(100, 146, size=u.size, dtype=np.uint32)
    u2 = (u & np.uint32(0x807FFFFF)) | (e << np.uint32(23))
    x = np.concatenate([u, u2]).view(np.float32)
    x = x[~np.isnan(x)]
    ours = codecs.f32_to_f16_bits(x)
    lib = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(6)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # exact ties and near-ties in the low half
    ties = (u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    near = ties + np.uint32(1)
    special = np.array([0x7F7FFFFF, 0x7F7F8000, 0x00000001, 0x00008000, 0x00018000, 0x80008000,
                        0x7F800000, 0xFF800000, 0x00000000, 0x80000000], dtype=np.uint32)
    x = np.concatenate([u, ties, near, special]).view(np.float32)
    ours = codecs.f32_to_bf16_bits(x)
    lib = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    fin = ~np.isnan(x)
    assert np.array_equal(ours[fin], lib[fin])
    # NaNs stay NaNs
    nan_out = ours[~fin]
    assert np.all((nan_out & 0x7F80) == 0x7F80) and np.all((nan_out & 0x007F) != 0)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_bits_to_f64_matches_torch(dtype):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = codecs.bits_to_f64(h, dtype)
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    lib = torch.from_numpy(h.view(np.int16)).view(tdt).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])


# ---------------------------------------------------------------------------
# E4M3 encoder (optional W8A8 activation path, [FP8 doc] §6)
# ---------------------------------------------------------------------------

def _finite_codes():
    c = np.arange(256)
    return c[~np.isnan(codecs.E4M3FN_TABLE)]


def test_e4m3fn_encode_round_trips_every_finite_code():
    c = _finite_codes()
    got = codecs.e4m3fn_encode(codecs.E4M3FN_TABLE[c])
    assert np.array_equal(got.astype(np.int64), c)


def test_e4m3fn_encode_midpoints_go_to_even_code_and_neighbours_to_nearest():
    pos = np.arange(0, 0x7E)                       # pairs (c, c+1) of finite positive codes
    lo = codecs.E4M3FN_TABLE[pos]
    hi = codecs.E4M3FN_TABLE[pos + 1]
    mid = (lo + hi) / 2
    want_mid = np.where(pos % 2 == 0, pos, pos + 1)
    assert np.array_equal(codecs.e4m3fn_encode(mid).astype(np.int64), want_mid)
    assert np.array_equal(codecs.e4m3fn_encode(-mid).astype(np.int64), want_mid | 0x80)
    gap = hi - lo
    assert np.array_equal(codecs.e4m3fn_encode(mid - gap / 8).astype(np.int64), pos)
    assert np.array_equal(codecs.e4m3fn_encode(mid + gap / 8).astype(np.int64), pos + 1)


def test_e4m3fn_encode_saturation_nan_zero_and_underflow():
    lm = _landmarks()
    top = float(lm["e4m3_max"][0])
    tiny = float(lm["e4m3_min_positive"][0])
    enc = lambda v: int(codecs.e4m3fn_encode(np.array([v]))[0])
    for v in (top, top * (1 + 2 ** -20), 464.0, 480.0, 1e30, math.inf):
        assert enc(v) == 0x7E and enc(-v) == 0xFE
    assert enc(math.nan) == 0x7F
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert enc(tiny / 2) == 0x00                  # midpoint of 0 and 2^-9: even code 0
    assert enc(tiny / 2 * (1 + 2 ** -20)) == 0x01
    assert enc(-tiny / 4) == 0x80
    assert enc(tiny * 1.5) == 0x02                # midpoint of codes 1 and 2: even code 2


def test_e4m3fn_encode_matches_torch_conversion_in_range():
    rng = np.random.default_rng(11)
    u = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    e = rng.integers(110, 136, size=u.size, dtype=np.uint32)     # 2^-17 .. 2^8
    x = ((u & np.uint32(0x807FFFFF)) | (e << np.uint32(23))).view(np.float32)
    # exact E4M3 midpoints and their float32 neighbours
    mids = ((codecs.E4M3FN_TABLE[0:0x7E] + codecs.E4M3FN_TABLE[1:0x7F]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                        -mids]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ours = codecs.e4m3fn_encode(x)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, lib)
