"""Pins of the oracle's NVFP4 formats and quantiser against things other than itself:
library float8 conversions, brute-force nearest-value searches, and the worked
values printed on the pages (tests/golden)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import nvfp4_ref as ref

RNG = np.random.default_rng(12345)


# ------------------------------------------------------- minifloat fields ----

def minifloat_value(code, ebits, mbits, bias):
    """Value of a sign / exponent / mantissa code read from its bit fields (OCP FP8 and
    MX v1.0 layouts): exponent field 0 is subnormal, 2^(1-bias) * m / 2^mbits; any other
    e is 2^(e-bias) * (1 + m / 2^mbits).  Written from the field definitions, not from
    the oracle, and pinned on the FP8 formats by torch's own conversions below."""
    sign = (code >> (ebits + mbits)) & 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        mag = 2.0 ** (1 - bias) * (m / 2.0 ** mbits)
    else:
        mag = 2.0 ** (e - bias) * (1.0 + m / 2.0 ** mbits)
    return -mag if sign else mag


def test_minifloat_fields_match_torch_fp8_formats():
    # e4m3fn: bias 7, only 0x7F / 0xFF are NaN; e5m2: bias 15, exponent 31 is inf/NaN
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    t43 = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t52 = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    for c in range(256):
        if (c & 0x7F) != 0x7F:
            assert minifloat_value(c, 4, 3, 7) == t43[c], c
        if (c >> 2) & 0x1F != 0x1F:
            assert minifloat_value(c, 5, 2, 15) == t52[c], c


# e2m1 = 1 sign bit (bit 3), 2 exponent bits with bias 1, 1 mantissa bit (OCP MX v1.0)
E2M1_FROM_FIELDS = np.array([minifloat_value(c, 2, 1, 1) for c in range(8)])


def test_e2m1_values_follow_the_bit_fields():
    for code in range(16):
        want = minifloat_value(code, 2, 1, 1)
        got = float(ref.e2m1_value(code))
        assert got == want and np.signbit(got) == np.signbit(want), (code, got, want)


# ----------------------------------------------------------------- e2m1 ----

def brute_e2m1(r):
    """Nearest of the 8 magnitudes (from the bit fields) by exhaustive search; ties to
    the even code."""
    out = []
    for x in np.ravel(r):
        best, best_d = None, None
        for code in range(8):
            d = abs(x - E2M1_FROM_FIELDS[code])
            if best is None or d < best_d or (d == best_d and code % 2 == 0):
                best, best_d = code, d
        if x > 6.0:
            best = 7
        out.append(best)
    return np.array(out).reshape(np.shape(r))


def test_e2m1_table_roundtrip():
    for code in range(16):
        v = ref.e2m1_value(code)
        assert ref.e2m1_round(abs(v)) == (code & 7)
        assert np.signbit(v) == bool(code & 8) or v == 0
    assert list(ref.e2m1_value(np.arange(8))) == list(E2M1_FROM_FIELDS)
    assert list(ref.e2m1_value(np.arange(8, 16))) == list(-E2M1_FROM_FIELDS)


def test_e2m1_ties_to_even_and_saturation():
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for r, code in ties.items():
        assert ref.e2m1_round(r) == code, r
    assert ref.e2m1_round(6.0) == 7 and ref.e2m1_round(7.0) == 7 and ref.e2m1_round(1e30) == 7
    assert ref.e2m1_round(0.0) == 0


def test_e2m1_matches_brute_force():
    r = np.concatenate([RNG.uniform(0, 7, 20000), RNG.uniform(0, 0.3, 2000),
                        np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 6.5])])
    assert np.array_equal(ref.e2m1_round(r), brute_e2m1(r))


# ----------------------------------------------------------------- e4m3 ----

def test_e4m3_decode_matches_torch_for_all_256_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ov = ref.e4m3_value(np.arange(256))
    assert np.array_equal(np.isnan(tv), np.isnan(ov))
    ok = ~np.isnan(tv)
    assert np.array_equal(tv[ok], ov[ok])
    assert np.array_equal(np.signbit(tv[ok]), np.signbit(ov[ok]))
    assert ref.e4m3_value(0x7E) == 448.0 and np.isnan(ref.e4m3_value(0x7F))
    assert ref.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_round_matches_torch_cast():
    # torch's float32 -> float8_e4m3fn cast is round-to-nearest-even; compare on
    # in-range values (torch does not saturate, so stay at or below 448).
    x = np.concatenate([
        RNG.uniform(0, 448, 400000),
        np.exp2(RNG.uniform(-12, 8.8, 400000)),
        RNG.uniform(0, 2.0 ** -6, 200000),            # subnormal range
    ])
    x = x[x <= 448].astype(np.float32)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    o = ref.e4m3_round(x.astype(np.float64))
    bad = np.nonzero(t != o)[0]
    assert bad.size == 0, (x[bad[:5]], t[bad[:5]], o[bad[:5]])


def brute_e4m3(x):
    vals = ref.e4m3_value(np.arange(127))
    out = []
    for xi in np.ravel(x):
        d = np.abs(vals - xi)
        best = np.flatnonzero(d == d.min())
        code = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
        out.append(126 if xi > 448 else code)
    return np.array(out)


def test_e4m3_matches_brute_force_and_saturates():
    x = np.concatenate([np.exp2(RNG.uniform(-11, 10, 5000)),
                        np.array([0, 2.0 ** -10, 2.0 ** -10 * 1.0001, 3 * 2.0 ** -10, 448, 449,
                                  463.9, 464, 1e9])])
    assert np.array_equal(ref.e4m3_round(x), brute_e4m3(x))
    assert ref.e4m3_round(2.0 ** -10) == 0          # tie between 0 and 2^-9 -> even code 0
    assert ref.e4m3_round(3 * 2.0 ** -10) == 2      # tie between codes 1 and 2 -> 2
    assert ref.e4m3_round(1e9) == 0x7E


# ------------------------------------------------------------ quantiser ----

def test_vones_probe_matches_page(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "vones_probe.json")))
    ones = np.full((3, 128), g["v_value"])
    packed, sf = ref.quantize(ones)
    deq = ref.dequantize(packed, sf)
    assert np.all(deq == deq.flat[0])
    val = float(deq.flat[0])
    assert round(val, g["printed_fixed_decimals"]) == g["printed_fixed"]
    assert round(val / 2, g["printed_halved_decimals"]) == g["printed_halved"]
    assert val == 1.03125                   # 6 * RNE_e4m3(1/6) = 6 * 0.171875
    assert np.all(sf == 0x23)
    assert np.all(packed == 0x77)


def bf16_rows(shape, scale=1.0):
    x = torch.from_numpy(RNG.standard_normal(shape) * scale).to(torch.bfloat16)
    return x.to(torch.float64).numpy()


def test_quantiser_is_nearest_value_brute_force():
    x = bf16_rows((64, 64))
    x[3, :16] = 0.0
    x[5, 16:32] = np.array([6.0, -3.0, 1.5, 0.75, -0.25, 5.0, 2.5, 1.75] * 2)  # tie-laden block
    packed, sf = ref.quantize(x)
    nib = ref.unpack_nibbles(packed)
    blocks = x.reshape(64, 4, 16)
    svals = ref.e4m3_value(sf)
    for r in range(64):
        for b in range(4):
            amax = np.abs(blocks[r, b]).max()
            # scale: nearest e4m3 to amax/6 (compare |amax - 6 v| exactly)
            cand = ref.e4m3_value(np.arange(127))
            d = np.abs(amax - 6 * cand)
            best = np.flatnonzero(d == d.min())
            want = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
            assert sf[r, b] == want
            s = svals[r, b]
            for e in range(16):
                xe = blocks[r, b, e]
                code = nib[r, 16 * b + e]
                assert bool(code & 8) == bool(np.signbit(xe))
                if s == 0:
                    assert code & 7 == 0
                    continue
                dist = [abs(abs(xe) - m * s) for m in E2M1_FROM_FIELDS]
                mn = min(dist)
                ok = [c for c in range(8) if dist[c] == mn]
                exp = ok[0] if len(ok) == 1 else [c for c in ok if c % 2 == 0][0]
                if abs(xe) > 6 * s:
                    exp = 7
                assert code & 7 == exp


def test_quantiser_block_axis_and_nibble_order():
    x = np.zeros((1, 64))
    x[0, 0] = 1.0          # element 0 -> low nibble of byte 0
    x[0, 17] = -2.0        # element 17 -> high nibble of byte 8, block 1
    packed, sf = ref.quantize(x)
    assert sf[0, 0] != 0 and sf[0, 1] != 0 and sf[0, 2] == 0 and sf[0, 3] == 0
    assert packed[0, 0] & 0xF == 7 and packed[0, 0] >> 4 == 0
    assert packed[0, 8] >> 4 == 0x8 | 7 and packed[0, 8] & 0xF == 0
    # changing block 1 leaves block 0's bytes alone
    y = x.copy()
    y[0, 16:32] *= 100
    p2, s2 = ref.quantize(y)
    assert np.array_equal(p2[0, :8], packed[0, :8]) and s2[0, 0] == sf[0, 0]


def test_quantiser_zero_block_and_signed_zero():
    x = np.zeros((2, 16))
    x[1] = -0.0
    x[1, 3] = -1e-30       # far below the smallest scale: code 0, sign kept
    packed, sf = ref.quantize(x)
    assert np.all(sf == 0)
    assert np.all(packed[0] == 0)
    assert np.all(packed[1] == 0x88)
    assert np.all(ref.dequantize(packed, sf) == 0)


def test_quantiser_saturation():
    x = np.full((1, 16), 1e6)
    packed, sf = ref.quantize(x)
    assert sf[0, 0] == 0x7E and np.all(packed == 0x77)
    assert np.all(ref.dequantize(packed, sf) == 6 * 448)


def test_global_scale_power_of_two_is_exact_rescale():
    x = bf16_rows((32, 128))
    p1, s1 = ref.quantize(x)
    for g in (0.25, 2.0, 8.0):
        p2, s2 = ref.quantize(x * g, global_scale=g)
        assert np.array_equal(p1, p2) and np.array_equal(s1, s2)
        assert np.array_equal(ref.dequantize(p2, s2, g), ref.dequantize(p1, s1) * g)


def test_dequant_error_bound():
    x = bf16_rows((256, 128), scale=3.0)
    packed, sf = ref.quantize(x)
    xh = ref.dequantize(packed, sf)
    s = np.repeat(ref.e4m3_value(sf), 16, axis=-1)
    # within the grid the error is at most half the local gap (gap <= 2 s);
    # above 6 s (only when s rounded down) it is at most the excess.
    err = np.abs(x - xh)
    bound = np.maximum(s * 1.0, np.abs(x) - 6 * s)
    assert np.all(err <= bound + 1e-300)
    # the dequantised products are exact in float32, float16 and bfloat16
    for dt in (np.float32, np.float16):
        assert np.array_equal(xh.astype(dt).astype(np.float64), xh)
    tb = torch.from_numpy(xh).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(tb, xh)
