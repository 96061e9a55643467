"""Pins of the oracle's NVFP4 / FP8 format code against sources other than itself:
hand-typed tables, a hand-worked row, torch's float8_e4m3fn casts, and exact
rational brute force (fractions.Fraction)."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        out[int(code, 16)] = float(val)
    return out


def _same(a, b):
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def test_e2m1_table_matches_hand_typed_golden():
    gold = _read_table("e2m1_values.txt")
    assert len(gold) == 16
    tab = oracle.e2m1_table()
    for c, v in gold.items():
        assert _same(tab[c], v), (c, tab[c], v)


def test_e4m3_table_matches_hand_typed_golden():
    gold = _read_table("e4m3_values.txt")
    tab = oracle.e4m3_table()
    for c, v in gold.items():
        assert _same(tab[c], v), (hex(c), tab[c], v)


def test_e4m3_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = oracle.e4m3_table()
    for c in range(256):
        assert _same(tab[c], ref[c]), (hex(c), tab[c], ref[c])


def _all_finite_fp16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    return v[np.isfinite(v)]


def test_e4m3_encode_matches_torch_cast_on_all_fp16():
    # torch casts fp16 -> fp8 e4m3fn with round-to-nearest-even; fp16 -> fp32 is exact,
    # so this is a single rounding.  torch does not saturate (|x| > 464 -> NaN), so the
    # saturation range is checked separately.
    x = _all_finite_fp16()
    small = x[np.abs(x.astype(np.float64)) < 464]
    ref = torch.from_numpy(small.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(small.astype(np.float64))
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, [(float(small[i]), hex(ref[i]), hex(got[i])) for i in bad[:5]]
    big = x[np.abs(x.astype(np.float64)) >= 464]
    got = F.e4m3_encode(big.astype(np.float64))
    assert np.all((got & 0x7F) == 0x7E)
    assert np.all((got >> 7) == np.signbit(big))


def _e4m3_pos_fractions():
    vals = []
    for c in range(0x7F):
        e, m = (c >> 3) & 15, c & 7
        v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else Fraction(2) ** (e - 7) * (1 + Fraction(m, 8))
        vals.append((v, c))
    return vals


def _nearest_fraction(r, grid):
    """Brute force nearest (value, code) to the rational r, ties to even code, saturating."""
    best = None
    for v, c in grid:
        d = abs(r - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_block_scale_is_nearest_e4m3_of_exact_amax_over_6_bruteforce():
    grid = _e4m3_pos_fractions()
    x = _all_finite_fp16()
    amax = np.unique(np.abs(x.astype(np.float64)))
    # every distinct non-negative fp16 magnitude: exhaustive over amax
    got = F.e4m3_encode_scaled_by(amax, 6.0)
    import bisect
    gv = [v for v, _ in grid]
    for a, g in zip(amax, got):
        r = Fraction(float(a)) / 6
        i = bisect.bisect_left(gv, r)
        cand = [grid[j] for j in (i - 1, i) if 0 <= j < len(grid)]
        if i >= len(grid):
            exp = grid[-1][1]
        else:
            exp = _nearest_fraction(r, cand)
        assert g == exp, (a, hex(g), hex(exp))


def test_e2m1_encode_bruteforce_over_scales_ties_and_neighbours():
    # every positive finite scale; for each, magnitudes at every grid point and tie
    # midpoint times the scale, their fp16 neighbours, beyond-saturation values and
    # random magnitudes; both signs.  Expected codes by exact rational search.
    e2 = [(Fraction(v).limit_denominator(4), c) for c, v in enumerate([0, .5, 1, 1.5, 2, 3, 4, 6])]
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rng = np.random.default_rng(3)
    xs, scs, exps = [], [], []
    for sc_code in range(1, 0x7F):
        s = F.e4m3_value(sc_code)
        mags = set()
        for g in [0, .5, 1, 1.5, 2, 3, 4, 6, 7, 100] + mids:
            h = np.float16(g * s)
            if np.isfinite(h):
                mags.update([h, np.nextafter(h, np.float16(np.inf)), np.nextafter(h, np.float16(0))])
        mags.update(np.abs(rng.standard_normal(24) * min(s * 4, 60000)).astype(np.float16))
        for h in mags:
            mag = float(h)
            if not math.isfinite(mag):
                continue
            code = _nearest_fraction(Fraction(mag) / Fraction(s), e2)
            for sign in (1.0, -1.0):
                xs.append(math.copysign(mag, sign))
                scs.append(s)
                exps.append(code | (8 if sign < 0 else 0))
    got = F.e2m1_encode(np.array(xs), np.array(scs))
    exp = np.array(exps, dtype=np.uint8)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, [(xs[i], scs[i], got[i], exp[i]) for i in bad[:5]]


def test_e2m1_encode_zero_scale_gives_signed_zero():
    got = F.e2m1_encode(np.array([0.0, -0.0, 1.0, -3.0]), 0.0)
    assert list(got) == [0, 8, 0, 8]


def test_row_layout_matches_hand_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "row_layout_example.json")))
    src = np.zeros((1, 576), dtype=np.float16)
    for k, v in ex["latent_nonzero"].items():
        src[0, int(k)] = v
    for k, v in ex["rope_values"].items():
        src[0, 512 + int(k)] = float(v)
    row = oracle.nvfp4_pack_rows_ref(src)[0]
    exp = np.zeros(352, dtype=np.uint8)
    for k, v in ex["expected_nonzero_bytes"].items():
        exp[int(k)] = v
    bad = np.nonzero(row != exp)[0]
    assert bad.size == 0, [(int(i), int(row[i]), int(exp[i])) for i in bad]


def _listed(d):
    return {int(k): float(v) for k, v in d.items()}


def test_unpack_decodes_hand_worked_row():
    # The golden row's expected bytes, decoded back to the values worked out by hand in the
    # golden file: every latent element not listed is +0.
    ex = json.load(open(os.path.join(GOLDEN, "row_layout_example.json")))
    row = np.zeros((1, 352), dtype=np.uint8)
    for k, v in ex["expected_nonzero_bytes"].items():
        row[0, int(k)] = v
    vals = oracle.nvfp4_unpack_rows_ref(row)[0]
    lat = _listed(ex["decoded_latent_listed"])
    rope = _listed(ex["decoded_rope"])
    for e in range(512):
        assert _same(vals[e], lat.get(e, 0.0)), (e, vals[e], lat.get(e, 0.0))
    for k in range(64):
        assert _same(vals[512 + k], rope.get(k, 0.0)), (k, vals[512 + k])


def test_unpack_decodes_second_hand_worked_row():
    # 32 distinct group scales and different codes in the two nibbles of every byte: pins the
    # nibble order, the element -> group-scale map and the rope offset at the listed elements.
    ex = json.load(open(os.path.join(GOLDEN, "row_decode_example.json")))
    row = np.frombuffer(bytes.fromhex(ex["row_hex"]), dtype=np.uint8).reshape(1, 352)
    vals = oracle.nvfp4_unpack_rows_ref(row)[0]
    for e, v in _listed(ex["decoded_latent"]).items():
        assert _same(vals[e], v), (e, vals[e], v)
    for k, v in _listed(ex["decoded_rope"]).items():
        assert _same(vals[512 + k], v), (k, vals[512 + k], v)


def test_unpack_of_pack_is_a_nearest_grid_point():
    # Round trip on random rows: each decoded latent value is a point of its group's scaled
    # E2M1 grid nearest to the input (scale byte decoded by torch's float8_e4m3fn), and each
    # rope value is torch's E4M3 cast of the input.  A swapped nibble or a wrong group scale
    # in the decoder moves values off their nearest grid point.
    rng = np.random.default_rng(23)
    src = (rng.standard_normal((16, 576)) * rng.choice([0.01, 1, 40], size=(16, 1))).astype(np.float16)
    rows = oracle.nvfp4_pack_rows_ref(src)
    vals = oracle.nvfp4_unpack_rows_ref(rows)
    x = src.astype(np.float64)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    for i in range(src.shape[0]):
        scales = torch.from_numpy(rows[i, 256:288].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        for g in range(32):
            s = scales[g]
            xs = x[i, 16 * g:16 * g + 16]
            got = vals[i, 16 * g:16 * g + 16]
            pts = s * grid
            for k in range(16):
                dist = np.abs(np.abs(xs[k]) - pts)
                assert abs(got[k]) in set(pts[dist == dist.min()]), (i, g, k, xs[k], got[k], s)
                if got[k] != 0:
                    assert np.sign(got[k]) == np.sign(xs[k])
        ref = torch.from_numpy(src[i, 512:].astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        assert np.array_equal(vals[i, 512:], ref)


def test_pack_decisions_bruteforce_on_random_rows():
    rng = np.random.default_rng(11)
    src = (rng.standard_normal((24, 576)) * rng.choice([1e-3, 0.1, 1, 30, 3000], size=(24, 1))).astype(np.float16)
    rows = oracle.nvfp4_pack_rows_ref(src)
    grid4 = _e4m3_pos_fractions()
    e2 = [(Fraction(v).limit_denominator(4), c) for c, v in enumerate([0, .5, 1, 1.5, 2, 3, 4, 6])]
    for i in range(src.shape[0]):
        for g in range(32):
            grp = src[i, 16 * g:16 * g + 16].astype(np.float64)
            amax = max(abs(float(v)) for v in grp)
            sc = _nearest_fraction(Fraction(amax) / 6, grid4)
            assert rows[i, 256 + g] == sc
            s = Fraction(F.e4m3_value(sc))
            for k in range(16):
                xv = float(grp[k])
                code = 0 if s == 0 else _nearest_fraction(Fraction(abs(xv)) / s, e2)
                if math.copysign(1.0, xv) < 0:
                    code |= 8
                e = 16 * g + k
                byte = rows[i, e // 2]
                got = (byte >> 4) if (e & 1) else (byte & 0xF)
                assert got == code, (i, g, k, xv, got, code)
        ref = torch.from_numpy(src[i, 512:].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        sat = np.abs(src[i, 512:].astype(np.float64)) >= 464
        ref = np.where(sat, np.where(np.signbit(src[i, 512:]), 0xFE, 0x7E), ref)
        assert np.array_equal(rows[i, 288:], ref)


def test_dequant_products_exact_in_fp16():
    e2 = oracle.e2m1_table()
    e4 = oracle.e4m3_table()
    for c in range(16):
        for s in range(256):
            if np.isnan(e4[s]):
                continue
            v = e2[c] * e4[s]
            assert float(np.float16(v)) == v, (c, s, v)


def test_unpack_inverts_pack_layout():
    # codes and scales decoded by the oracle equal E2M1(code)*E4M3(scale) at the byte positions
    rng = np.random.default_rng(5)
    rows = rng.integers(0, 256, size=(8, 352), dtype=np.uint8)
    rows[:, 256:] &= 0x77  # keep scales and rope finite (clear 0x7F patterns' top bits)
    vals = oracle.nvfp4_unpack_rows_ref(rows)
    e2 = oracle.e2m1_table()
    e4 = oracle.e4m3_table()
    for i in range(8):
        for e in range(512):
            code = (rows[i, e // 2] >> 4) if e & 1 else (rows[i, e // 2] & 0xF)
            assert _same(vals[i, e], e2[code] * e4[rows[i, 256 + e // 16]])
        for k in range(64):
            assert _same(vals[i, 512 + k], e4[rows[i, 288 + k]])


def test_fp8_stage_matches_torch_cast_of_dequantized_values():
    rng = np.random.default_rng(9)
    src = rng.standard_normal((16, 576)).astype(np.float16)
    rows = oracle.nvfp4_pack_rows_ref(src)
    staged = oracle.fp8_stage_rows_ref(rows)
    vals = oracle.nvfp4_unpack_rows_ref(rows).astype(np.float16)       # exact
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(staged, ref)


def test_pack_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.nvfp4_pack_rows_ref(np.zeros((2, 575), dtype=np.float16))
    with pytest.raises(ValueError):
        oracle.nvfp4_pack_rows_ref(np.zeros((2, 576), dtype=np.float32))
