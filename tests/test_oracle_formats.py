"""Pins of the oracle's number formats against things other than itself:
torch's float8_e4m3fn (a library decoder / RNE encoder), brute-force nearest
search, exponent re-biasing into E4M3, and the byte counts the source pages
print (tests/golden/page_facts.json)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import traffic

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def torch_e4m3_decode(bytes_):
    return torch.tensor(np.asarray(bytes_, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_e4m3_encode(x):
    return torch.tensor(np.asarray(x, dtype=np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_256_codes_match_torch():
    ours = F.e4m3_value(np.arange(256))
    ref = torch_e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.nanmax(ours) == 448.0 and F.e4m3_value(1) == 2.0 ** -9


def test_e2m1_decode_by_exponent_rebias_into_e4m3():
    # An E2M1 code (s, e, m) is the E4M3 byte with the same sign, exponent
    # re-biased from 1 to 7 and the mantissa bit moved to the top of E4M3's
    # three; the subnormal code 1 (0.5) is the normal E4M3 2**-1.
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e == 0 and m == 0:
            byte = s << 7
        elif e == 0:
            byte = (s << 7) | (6 << 3)
        else:
            byte = (s << 7) | ((e - 1 + 7) << 3) | (m << 2)
        assert F.e2m1_value(c) == torch_e4m3_decode([byte])[0], c
    mags = F.e2m1_value(np.arange(8))
    assert len(set(mags)) == 8 and np.all(np.diff(mags) > 0)
    assert mags.max() == 6.0 and mags[1] == 0.5
    assert GOLD["lut_magnitudes"]["value"] == 8


def test_e4m3_encode_matches_torch_rne_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.normal(0, 1, 20000), rng.normal(0, 50, 20000),
        rng.uniform(-463.9, 463.9, 5000), rng.normal(0, 2e-3, 5000),
    ])
    # exact midpoints between neighbouring finite codes (ties to even)
    pos = F.e4m3_value(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.concatenate([x, mids, -mids, pos, -pos])
    assert np.array_equal(F.e4m3_encode(x), torch_e4m3_encode(x))


def test_e4m3_encode_saturates():
    big = np.array([448.0, 463.99, 464.0, 1e6, -500.0, -448.0])
    assert list(F.e4m3_encode(big)) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_e2m1_encode_brute_force_nearest_even():
    grid = np.concatenate([np.arange(-7.0, 7.01, 0.125), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]])
    vals = F.e2m1_value(np.arange(16))
    for v in grid:
        c = int(F.e2m1_encode(v))
        d = np.abs(vals - v)
        target = min(abs(v), 6.0)
        # nearest magnitude (clamped), ties to the even code
        mags = vals[:8]
        dm = np.abs(mags - target)
        cand = np.flatnonzero(dm == dm.min())
        expect_mag = cand[0] if len(cand) == 1 else [k for k in cand if k % 2 == 0][0]
        assert (c & 7) == expect_mag, (v, c)
        assert (c >> 3) == int(np.signbit(v)), v
        assert d[c] == np.abs(vals[c] - v)


def test_fp8_rounded_table_2048_entries_match_torch():
    tab = F.fp8_rounded_table()
    assert tab.size == GOLD["lut_scales"]["value"] * GOLD["lut_magnitudes"]["value"]
    assert tab.nbytes == GOLD["lut_bytes"]["value"]
    for s in range(256):
        if s & 0x80 or s == 0x7F:
            continue
        prod = F.e4m3_value(s) * F.e2m1_value(np.arange(8))
        ref = torch_e4m3_encode(np.minimum(prod, 448.0))     # torch does not saturate
        assert np.array_equal(tab[s], ref), s


def test_nvfp4_dequant_modes_on_all_codes_and_scales():
    scales = np.array([s for s in range(256) if not (s & 0x80) and s != 0x7F], dtype=np.uint8)
    codes = np.arange(16, dtype=np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)          # 16 codes -> 8 bytes
    packed = np.tile(packed, (len(scales), 1))
    sb = scales[:, None]
    ex = F.nvfp4_dequantize(packed, sb, 1.0, F.EXACT)
    f8 = F.nvfp4_dequantize(packed, sb, 1.0, F.FP8_ROUNDED)
    tab = F.fp8_rounded_table()
    for r, s in enumerate(scales):
        for c in range(16):
            p = F.e4m3_value(s) * F.e2m1_value(c)
            assert ex[r, c] == p
            ref = torch_e4m3_decode([tab[s, c & 7]])[0]
            assert f8[r, c] == (-ref if c & 8 else ref)
    # the per-tensor scale multiplies afterwards, exactly
    assert np.array_equal(F.nvfp4_dequantize(packed, sb, 0.375, F.EXACT), 0.375 * ex)


def test_nvfp4_quantize_properties():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 1, (64, 128)).astype(np.float32)
    x[::7, 3] *= 9.0                                     # some outliers
    S = 32.0 / 448.0
    codes, sb = F.nvfp4_quantize(x, S)
    assert codes.shape == (64, 64) and sb.shape == (64, 8)
    # row bytes: 64 code bytes + 8 scale bytes = 72 per 128-dim row
    assert codes.shape[1] + sb.shape[1] == traffic.ROW_BYTES["nvfp4"] == 72
    # scale byte = torch's E4M3 rounding of amax / (6 S), computed in fp32
    amax = np.abs(x.reshape(64, 8, 16)).max(-1)
    t = (amax / (np.float32(6.0) * np.float32(S))).astype(np.float32)
    assert np.array_equal(sb, torch_e4m3_encode(t.astype(np.float64)))
    # every code is the nearest E2M1 value of x / (s S) (brute force in fp64,
    # ignoring values within 1e-6 of a rounding midpoint)
    deq = F.nvfp4_dequantize(codes, sb, S, F.EXACT).reshape(64, 8, 16)
    cv = F.e2m1_value(F.nvfp4_unpack_codes(codes)).reshape(64, 8, 16)
    sv = (F.e4m3_value(sb) * S)[..., None]
    y = x.reshape(64, 8, 16).astype(np.float64) / sv
    vals = F.e2m1_value(np.arange(16))
    checked = 0
    for idx in np.ndindex(y.shape):
        d = np.abs(vals - y[idx])
        order = np.sort(d)
        if order[1] - order[0] < 1e-6:
            continue
        assert cv[idx] == vals[np.argmin(d)]
        checked += 1
    assert checked > 7000
    # the group's amax element lands on +-6 or within one grid step of it
    err = np.abs(deq - x.reshape(64, 8, 16))
    assert np.all(err <= sv * 1.0 + 1e-12)


def test_nvfp4_quantize_zero_group_and_packing_order():
    x = np.zeros((1, 32), np.float32)
    x[0, 16] = 1.0
    x[0, 17] = -2.0
    codes, sb = F.nvfp4_quantize(x, 1.0)
    assert sb[0, 0] == 0 and np.all(codes[0, :8] == 0)
    # even element in the low nibble
    lo, hi = codes[0, 8] & 0xF, codes[0, 8] >> 4
    s = F.e4m3_value(sb[0, 1])
    assert F.e2m1_value(lo) * s == pytest.approx(1.0, rel=0.2)
    assert F.e2m1_value(hi) * s == pytest.approx(-2.0, rel=0.05) and hi & 7 == 7


def test_fp8_quantize_matches_torch_cast():
    rng = np.random.default_rng(2)
    x = rng.normal(0, 1, 5000).astype(np.float32)
    assert np.array_equal(F.fp8_quantize(x, 1.0), torch_e4m3_encode(x.astype(np.float64)))
    S = np.float32(0.37)
    y = (x / S).astype(np.float64)
    assert np.array_equal(F.fp8_quantize(x, S), torch_e4m3_encode(y))


def _e4m3_half_step(v):
    """Half the spacing of the E4M3 grid at magnitude v (subnormal spacing 2^-9 below
    2^-6; 2^(floor(log2 v) - 3) in the normal range)."""
    v = np.asarray(v, np.float64)
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    return 0.5 * np.exp2(e - 3)


@pytest.mark.parametrize("S", [float(np.float32(0.37)), float(np.float32(32.0 / 448.0)), 5.0,
                               float(np.float32(0.0123)), 3.0])
def test_fp8_tensor_scale_round_trip_bound(S):
    """The quantiser stores RNE(x / S), so a decoded byte is S * e4m3(byte): the round
    trip lands within half an E4M3 step of x / S, times S, for every S.  A decoder
    that divided by S (mirroring the quantiser) would be off by a factor S^2."""
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.normal(0, 1, 4000), rng.normal(0, 20, 2000) * S, rng.normal(0, 1e-3, 500)])
    x = x[np.abs(x) / S < 440.0].astype(np.float32)
    back = F.fp8_dequantize(F.fp8_quantize(x, S), S)
    y = np.abs(x.astype(np.float64)) / S
    assert np.all(np.abs(back - x) <= _e4m3_half_step(y) * S * (1 + 1e-6) + 1e-300)
    # worked values from the definition: byte 0x40 is 2.0 and 0x38 is 1.0 (exponent 8
    # and 7, bias 7), 0xC4 is -3.0; the decoded value is the tensor scale times that
    assert F.fp8_dequantize(np.uint8(0x40), 3.0) == 6.0
    assert F.fp8_dequantize(np.uint8(0x38), 0.25) == 0.25
    assert F.fp8_dequantize(np.uint8(0xC4), 0.5) == -1.5


@pytest.mark.parametrize("s", [float(np.float32(0.37)), 4.0, float(np.float32(1.0 / 48.0))])
def test_decode_query_applies_its_scale(s):
    """FP8 query bytes quantised with scale s decode to s * e4m3(byte), within half an
    E4M3 step of the source; fp32 queries are multiplied by s."""
    from oracle import msa as OM
    rng = np.random.default_rng(12)
    x = (rng.normal(0, 1, (3, 4, 128)) * s * 8).astype(np.float32)
    x = np.clip(x, -440 * s, 440 * s).astype(np.float32)
    dq = OM.decode_query(F.fp8_quantize(x, s), "fp8", s)
    y = np.abs(x.astype(np.float64)) / s
    assert np.all(np.abs(dq - x) <= _e4m3_half_step(y) * s * (1 + 1e-6))
    assert np.array_equal(OM.decode_query(x, "f32", s), s * x.astype(np.float64))
    assert OM.decode_query(np.uint8(0x40), "fp8", s) == 2.0 * s
