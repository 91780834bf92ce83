"""Number formats of the MSA caches, written out from their bit definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援" (English post),
* "What is new in the MiniMax-M3.1 architecture": K/V and index keys are held
  in an NVFP4 KV cache (34,560 B/token against 61,440 B/token in FP8, i.e.
  4.5 bits per element: a 4-bit E2M1 code plus one 8-bit E4M3 scale per 16).
* "NVIDIA Blackwell optimized MSA kernels": the query is FP8; the kernels turn
  NVFP4 into FP8 (each scaled value re-rounded to E4M3) and run an FP8 MMA.
* "NVIDIA Rubin optimized MSA": NVFP4 turned into FP16 gives exact scores,
  without the E4M3 re-rounding.
* "NVFP4 MSA kernel" (AMD): 256 possible E4M3 scales times 8 E2M1
  magnitudes, every scaled value pre-rounded to FP8, fit a 2 KB table.

The pages name the formats but do not spell out their bits.  E2M1 and E4M3
are taken as the OCP microscaling / OCP FP8 definitions:
* E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; no inf or NaN;
  magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* E4M3 ("fn"): sign, 4 exponent bits (bias 7), 3 mantissa bits; no inf;
  0x7F / 0xFF are NaN; largest finite 448; smallest subnormal 2**-9.

The NVFP4 quantiser is not described on the pages; the reading used here
(per-16 amax scale, round-to-nearest-even, fp32 arithmetic in a fixed order)
is the one the pack kernels implement, so that both sides take every integer
decision in the same precision.
"""
import numpy as np

# ---------------------------------------------------------------- decoding


def e2m1_value(code):
    """Value of a 4-bit E2M1 code (array or int).  Bit 3 is the sign."""
    code = np.asarray(code, dtype=np.int64)
    sign = (code >> 3) & 1
    exp = (code >> 1) & 3
    man = code & 1
    # exponent 0 is subnormal: man * 2**-1 ; otherwise (1 + man/2) * 2**(exp-1)
    mag = np.where(exp == 0, man * 0.5, (1.0 + man * 0.5) * np.exp2(exp - 1.0))
    return np.where(sign == 1, -mag, mag)


def e4m3_value(byte):
    """Value of an 8-bit OCP E4M3 byte (array or int); NaN for 0x7F / 0xFF."""
    byte = np.asarray(byte, dtype=np.int64)
    sign = (byte >> 7) & 1
    exp = (byte >> 3) & 15
    man = byte & 7
    mag = np.where(exp == 0, (man / 8.0) * 2.0 ** -6,
                   (1.0 + man / 8.0) * np.exp2(exp - 7.0))
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


E4M3_MAX = 448.0
E2M1_MAX = 6.0

# The positive finite grids, in code order (both encodings are monotone in
# the code for non-negative values).
_E4M3_POS = e4m3_value(np.arange(0x7F))          # codes 0x00 .. 0x7E
_E2M1_POS = e2m1_value(np.arange(8))             # codes 0 .. 7


def _rne_on_grid(a, grid):
    """Index of the grid point nearest to a >= 0; ties go to the even index.

    ``grid`` is ascending and its index is the code, so "even index" is
    "even mantissa LSB".  Values above the top of the grid saturate to it.
    """
    a = np.asarray(a, dtype=np.float64)
    hi = np.searchsorted(grid, a, side="left")          # grid[hi-1] < a <= grid[hi]
    hi = np.clip(hi, 1, len(grid) - 1)
    lo = hi - 1
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(a >= grid[-1], len(grid) - 1, idx)    # saturate
    idx = np.where(a <= 0.0, 0, idx)
    return idx.astype(np.int64)


def e4m3_encode(x):
    """Round finite x to E4M3, nearest-even, saturating at +-448.

    The sign bit follows IEEE signbit (so -0.0 encodes as 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(x)), "E4M3 encoder takes finite inputs only"
    code = _rne_on_grid(np.abs(x), _E4M3_POS)
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def e2m1_encode(x):
    """Round finite x to E2M1, nearest-even, clamped to +-6; sign = signbit."""
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(x)), "E2M1 encoder takes finite inputs only"
    code = _rne_on_grid(np.abs(x), _E2M1_POS)
    return (code | (np.signbit(x).astype(np.int64) << 3)).astype(np.uint8)


# ---------------------------------------------------------------- FP8


def fp8_quantize(x, tensor_scale):
    """FP8 E4M3 bytes of x / S, the division done in fp32 (as the pack kernel)."""
    x32 = np.asarray(x, dtype=np.float32)
    y = x32 / np.float32(tensor_scale)
    return e4m3_encode(y.astype(np.float64))


def fp8_dequantize(b, tensor_scale):
    """S * e4m3(b) in fp64 (exact)."""
    return float(tensor_scale) * e4m3_value(b)


# ---------------------------------------------------------------- NVFP4

GROUP = 16          # elements per E4M3 scale


def nvfp4_quantize(x, tensor_scale):
    """Quantise rows of x (last axis a multiple of 16) to NVFP4.

    Reading (the pages give none): per group of 16 consecutive elements,
      scale byte s  = E4M3_RNE( amax / (6 * S) )
      code          = E2M1_RNE( x / (e4m3(s) * S) ), clamped to +-6
    with every arithmetic step in fp32 in exactly that order; a zero scale
    gives all-zero codes.  Codes are packed two per byte, the even element in
    the low nibble.  Returns (codes [..., n/2] uint8, scales [..., n/16] uint8).
    """
    x32 = np.asarray(x, dtype=np.float32)
    n = x32.shape[-1]
    assert n % GROUP == 0
    g = x32.reshape(x32.shape[:-1] + (n // GROUP, GROUP))
    amax = np.max(np.abs(g), axis=-1)                                  # fp32, exact
    six_s = np.float32(6.0) * np.float32(tensor_scale)                 # fp32
    t = (amax / six_s).astype(np.float32)                              # fp32
    sbyte = e4m3_encode(t.astype(np.float64))
    sval = e4m3_value(sbyte).astype(np.float32)                        # exact
    denom = (sval * np.float32(tensor_scale)).astype(np.float32)       # fp32
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (g / denom[..., None]).astype(np.float32)                  # fp32
    y = np.where(denom[..., None] > 0, y, np.float32(0.0))
    codes = e2m1_encode(y.astype(np.float64)).reshape(x32.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, sbyte


def nvfp4_unpack_codes(packed):
    """[..., n/2] bytes -> [..., n] 4-bit codes (even element = low nibble)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def _check_scale_bytes(sbytes):
    sbytes = np.asarray(sbytes)
    # Negative or NaN scale bytes never come out of the quantiser; they are
    # undefined input for every consumer.
    assert not np.any(sbytes & 0x80), "NVFP4 scale byte with sign bit set"
    assert not np.any(sbytes == 0x7F), "NVFP4 scale byte is NaN"


EXACT = "exact"        # value = S * e4m3(scale) * e2m1(code)           (Rubin FP16 path)
FP8_ROUNDED = "fp8"    # value = S * E4M3_RNE(e4m3(scale) * e2m1(code)) (Blackwell / CDNA4 LUT)


def nvfp4_dequantize(packed, sbytes, tensor_scale, mode=EXACT):
    """Dequantise NVFP4 to fp64 under one of the two readings.

    EXACT       -- the product e4m3(scale) * e2m1(code), exactly; the scores
                   "become exact" in the Rubin section's words.
    FP8_ROUNDED -- that product re-rounded (nearest-even, saturating) to E4M3
                   before use, which is what an FP8 MMA on dequantised keys
                   computes (Blackwell and AMD sections).
    The per-tensor scale S multiplies afterwards, exactly (fp64).
    """
    _check_scale_bytes(sbytes)
    codes = nvfp4_unpack_codes(packed)
    n = codes.shape[-1]
    sval = e4m3_value(sbytes)                                   # [..., n/16]
    sval = np.repeat(sval, GROUP, axis=-1).reshape(codes.shape[:-1] + (n,))
    prod = e2m1_value(codes) * sval                             # exact in fp64
    if mode == FP8_ROUNDED:
        prod = e4m3_value(e4m3_encode(prod))
    elif mode != EXACT:
        raise ValueError(mode)
    return float(tensor_scale) * prod


def fp8_rounded_table():
    """The 256 x 8 table of E4M3-rounded scaled magnitudes (AMD "NVFP4 MSA
    kernel": 2 KB, one byte per entry).  Row = scale byte, column = E2M1
    magnitude code 0..7.  Rows for NaN or negative scale bytes are 0xFF."""
    tab = np.full((256, 8), 0xFF, dtype=np.uint8)
    for s in range(256):
        if s & 0x80 or s == 0x7F:
            continue
        tab[s] = e4m3_encode(e4m3_value(s) * e2m1_value(np.arange(8)))
    return tab
