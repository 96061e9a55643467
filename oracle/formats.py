"""NVFP4 / FP8 formats of the KV-cache row.  TEST INFRASTRUCTURE ONLY (see package doc).

Source: "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily",
section "Four-bit caches make room": the multi-head-latent-attention cache is
compressed with NVFP4, a four-bit format holding one FP8 scale per group of 16
values, and a cache row shrinks from 576 to 352 bytes.

Readings taken here where the page leaves the step open:
  * NVFP4 elements are E2M1 (1 sign, 2 exponent, 1 mantissa bit; values
    0, 0.5, 1, 1.5, 2, 3, 4, 6 with sign) and the group scale is FP8 E4M3 in
    the OCP "FN" flavour (bias 7, no infinities, 0x7F/0xFF are NaN, max 448).
  * 576 -> 352 bytes: a row is 512 latent values + 64 rope values.  The latent
    part is NVFP4 (256 bytes of codes + 32 bytes of E4M3 scales); the rope part
    stays FP8 E4M3 (64 bytes).  Byte layout of a row:
        [0, 256)    E2M1 codes, element 2i in bits 3:0 and 2i+1 in bits 7:4 of byte i
        [256, 288)  E4M3 scale of group j (latent elements 16j .. 16j+15) in byte 256+j
        [288, 352)  E4M3 code of rope element k in byte 288+k
  * The group scale is the exact real amax/6 rounded to nearest E4M3 (ties to
    the even code), saturating at 448; there is no per-tensor second-level
    scale.  An element's code is the exact real x/scale rounded to the nearest
    E2M1 value (ties to the even code), saturating at 6, sign kept (so small
    negatives give the -0 code 0x8).  A zero scale gives code +-0 for all 16.
  * Rope values are rounded to nearest E4M3 (ties to even), saturating at 448.
  * The FP8 cache row the page starts from (576 bytes) holds the 576 values of a
    row as E4M3 codes, one byte each, value k in byte k (latent 0..511, rope
    512..575), with no scale: each is the value rounded to nearest E4M3, ties to
    even, saturating at 448.

All arithmetic below is exact: decoded values are small dyadic rationals held
exactly in float64, and every rounding decision compares an input against a
grid point (or grid point times 6) that is itself exact in float64.
"""

import numpy as np

LATENT_DIM = 512
ROPE_DIM = 64
HEAD_DIM = LATENT_DIM + ROPE_DIM  # 576: q.k runs over latent + rope
GROUP = 16                        # values per FP8 scale
CODE_BYTES = LATENT_DIM // 2      # 256
SCALE_BYTES = LATENT_DIM // GROUP  # 32
ROPE_BYTES = ROPE_DIM             # 64
ROW_BYTES = CODE_BYTES + SCALE_BYTES + ROPE_BYTES  # 352
FP8_ROW_BYTES = HEAD_DIM          # 576: one E4M3 byte per value
E4M3_MAX = 448.0
E2M1_MAX = 6.0


# ---------------------------------------------------------------- decoding ---

def e2m1_value(code):
    """Value of a 4-bit E2M1 code: sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0."""
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = m * 0.5                               # subnormal: m * 2^(1-1) * 2^-1
    else:
        mag = 2.0 ** (e - 1) * (1.0 + m / 2.0)      # normal: 2^(e-1) * 1.m
    return sign * mag


def e4m3_value(code):
    """Value of an 8-bit OCP E4M3 ("FN") code: sign bit 7, exponent 6:3 (bias 7), mantissa 2:0."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = m * 2.0 ** -9                         # subnormal: (m/8) * 2^(1-7)
    else:
        mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return sign * mag


def e2m1_table():
    """float64[16]: value of every E2M1 code."""
    return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e4m3_table():
    """float64[256]: value of every E4M3 code (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


_E2M1 = e2m1_table()
_E4M3 = e4m3_table()
# Non-negative finite grids, ascending, with their codes.
_E2M1_POS_CODES = np.arange(8, dtype=np.uint8)            # 0, .5, 1, 1.5, 2, 3, 4, 6
_E2M1_POS = _E2M1[:8].copy()
_E4M3_POS_CODES = np.arange(0x7F, dtype=np.uint8)          # 0 .. 448 (0x7F is NaN)
_E4M3_POS = _E4M3[:0x7F].copy()


# ---------------------------------------------------------------- encoding ---

def _nearest_code(mag, grid, codes):
    """Round non-negative magnitudes to the nearest grid point, ties to the even code.

    `grid` is ascending and `codes` gives the code of each grid point.  Values
    above the last grid point saturate to it.  `mag` and `grid` must be such
    that |mag - grid| is exact in float64 (true for every caller here).
    """
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.searchsorted(grid, mag, side="left")          # first grid point >= mag
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    d_lo = np.abs(mag - grid[lo])
    d_hi = np.abs(grid[hi] - mag)
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    even_hi = (codes[hi] & 1) == 0
    pick_hi = pick_hi | (tie & even_hi)
    out = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    # saturation: anything at or beyond the top grid point maps to the top code
    out = np.where(mag >= grid[-1], codes[-1], out).astype(np.uint8)
    return out


def e4m3_encode(x):
    """Round exact values to E4M3 codes: nearest, ties to even, saturate at +-448, keep sign."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode: inputs must be finite")
    mag_code = _nearest_code(np.abs(x), _E4M3_POS, _E4M3_POS_CODES)
    sign = np.signbit(x).astype(np.uint8) << 7
    return (mag_code | sign).astype(np.uint8)


def e4m3_encode_scaled_by(amax, divisor=6.0):
    """E4M3 code of the exact real amax/divisor (nearest, ties to even, saturating).

    Rounding r = amax/divisor to the grid g is the same decision as rounding
    amax to the grid divisor*g; with divisor = 6 every divisor*g is exact in
    float64, so the comparison is exact without ever forming amax/6.
    """
    amax = np.asarray(amax, dtype=np.float64)
    if np.any(amax < 0) or not np.all(np.isfinite(amax)):
        raise ValueError("e4m3_encode_scaled_by: amax must be finite and >= 0")
    return _nearest_code(amax, _E4M3_POS * divisor, _E4M3_POS_CODES)


def e2m1_encode(x, scale):
    """E2M1 code of the exact real x/scale: nearest, ties to even code, saturate at 6, keep sign.

    Decided by comparing |x| with scale*g for the E2M1 grid g (exact products).
    A zero scale yields the signed zero code.
    """
    x = np.asarray(x, dtype=np.float64)
    scale = np.broadcast_to(np.asarray(scale, dtype=np.float64), x.shape)
    mag = np.zeros(x.shape, dtype=np.uint8)
    nz = scale > 0
    if np.any(nz):
        ax = np.abs(x[nz])
        s = scale[nz]
        # nearest of s*g over the 8 grid points, ties to even code, decided per element
        cand = s[:, None] * _E2M1_POS[None, :]                 # exact products
        d = np.abs(ax[:, None] - cand)
        best = np.zeros(ax.shape, dtype=np.int64)
        bestd = d[:, 0].copy()
        for k in range(1, 8):
            better = d[:, k] < bestd
            tie = (d[:, k] == bestd) & ((k & 1) == 0) & ((best & 1) == 1)
            take = better | tie
            best = np.where(take, k, best)
            bestd = np.where(take, d[:, k], bestd)
        mag[nz] = best.astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 3
    return (mag | sign).astype(np.uint8)


# ------------------------------------------------------------ row codecs -----

def nvfp4_pack_rows_ref(src):
    """Quantize fp16 rows [n, 576] into 352-byte NVFP4 cache rows [n, 352] (uint8).

    Latent part: per group of 16, scale = E4M3(amax/6); codes = E2M1(x/scale).
    Rope part: E4M3(x).  Layout as in the module docstring.
    """
    src = np.asarray(src)
    if src.dtype != np.float16 or src.ndim != 2 or src.shape[1] != HEAD_DIM:
        raise ValueError("nvfp4_pack_rows_ref expects float16 [n, 576]")
    x = src.astype(np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("nvfp4_pack_rows_ref: inputs must be finite")
    n = x.shape[0]
    lat = x[:, :LATENT_DIM].reshape(n, SCALE_BYTES, GROUP)
    amax = np.max(np.abs(lat), axis=2)                           # [n, 32]
    scale_code = e4m3_encode_scaled_by(amax, 6.0)                # [n, 32]
    scale_val = _E4M3[scale_code]                                 # exact, finite
    codes = e2m1_encode(lat, scale_val[:, :, None]).reshape(n, LATENT_DIM)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)   # [n, 256]
    rope_code = e4m3_encode(x[:, LATENT_DIM:])                   # [n, 64]
    return np.concatenate([packed, scale_code, rope_code], axis=1).astype(np.uint8)


def nvfp4_unpack_rows_ref(rows):
    """Decode 352-byte rows [n, 352] to exact values float64 [n, 576].

    latent[k] = E2M1(code k) * E4M3(scale k//16); rope[k] = E4M3(rope code k).
    Every value is exactly representable in fp16 (at most 6 significant bits,
    magnitude within [2^-10, 2688]), so .astype(float16) is exact.
    """
    rows = np.asarray(rows, dtype=np.uint8)
    if rows.ndim != 2 or rows.shape[1] != ROW_BYTES:
        raise ValueError("nvfp4_unpack_rows_ref expects uint8 [n, 352]")
    n = rows.shape[0]
    packed = rows[:, :CODE_BYTES]
    codes = np.empty((n, LATENT_DIM), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    scale = _E4M3[rows[:, CODE_BYTES:CODE_BYTES + SCALE_BYTES]]            # [n, 32]
    lat = _E2M1[codes] * np.repeat(scale, GROUP, axis=1)
    rope = _E4M3[rows[:, CODE_BYTES + SCALE_BYTES:]]
    return np.concatenate([lat, rope], axis=1)


def fp8_stage_rows_ref(rows):
    """Staged variant, first pass: decode rows and re-encode every value as E4M3.

    Returns uint8 [n, 576] E4M3 codes (nearest, ties to even, saturating at 448).
    This step is lossy: an E2M1 x E4M3 product can carry 6 significant bits.
    """
    vals = nvfp4_unpack_rows_ref(rows)
    return e4m3_encode(vals)


def fp8_pack_rows_ref(src):
    """Quantize fp16 rows [n, 576] into 576-byte FP8 cache rows [n, 576] (uint8):
    byte k is the E4M3 code of value k (nearest, ties to even, saturating at 448)."""
    src = np.asarray(src)
    if src.dtype != np.float16 or src.ndim != 2 or src.shape[1] != HEAD_DIM:
        raise ValueError("fp8_pack_rows_ref expects float16 [n, 576]")
    return e4m3_encode(src.astype(np.float64))


def fp8_unpack_rows_ref(rows):
    """Decode 576-byte FP8 rows [n, 576] to exact values float64 [n, 576]."""
    rows = np.asarray(rows)
    if rows.dtype != np.uint8 or rows.ndim != 2 or rows.shape[1] != FP8_ROW_BYTES:
        raise ValueError("fp8_unpack_rows_ref expects uint8 [n, 576]")
    return _E4M3[rows]
