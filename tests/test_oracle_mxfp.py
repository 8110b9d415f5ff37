"""Pins for oracle.mxfp: FP8 tables, MX quantization, bf16 rounding.

Independent references: torch's float8_e4m3fn / float8_e5m2 / bfloat16 dtypes
(a separate implementation of the same IEEE/OCP encodings), hand-derived worked
examples (tests/golden/mx_worked_examples.json), the definition of "nearest"
checked by brute force over the whole code table, and the round-trip error bound.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import mxfp

FMT_TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def all_bf16_finite():
    bits = np.arange(65536, dtype=np.uint32) << 16
    with np.errstate(invalid="ignore"):
        v = bits.view(np.float32).astype(np.float64)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_decode_table_matches_torch(fmt):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(FMT_TORCH[fmt]).to(torch.float64).numpy()
    ours = mxfp.decode_table(fmt)
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], ours[ok])


def test_known_codes():
    t4, t5 = mxfp.decode_table("e4m3"), mxfp.decode_table("e5m2")
    assert t4[0x7E] == 448.0 and t4[0x01] == 2.0 ** -9 and t4[0x08] == 2.0 ** -6 and t4[0x38] == 1.0
    assert np.isnan(t4[0x7F]) and np.isnan(t4[0xFF]) and t4[0x80] == 0.0
    assert t5[0x7B] == 57344.0 and t5[0x01] == 2.0 ** -16 and t5[0x3C] == 1.0 and np.isinf(t5[0x7C])
    assert mxfp.max_finite("e4m3") == 448.0 and mxfp.max_finite("e5m2") == 57344.0


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_rounding_matches_torch_in_range(fmt):
    """Every finite bf16 value, shifted by a range of powers of two so the whole format
    range is swept, rounded by the oracle and by torch's fp32 -> fp8 cast (RNE)."""
    top = mxfp.max_finite(fmt)
    base = all_bf16_finite()
    vals = np.concatenate([base * 2.0 ** s for s in range(-12, 13, 3)])
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= top)]
    ref = torch.from_numpy(vals.astype(np.float32)).to(FMT_TORCH[fmt]).view(torch.uint8).numpy()
    ours = mxfp.round_to_format(vals, fmt)
    assert np.array_equal(ref, ours)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_rounding_is_nearest_by_brute_force(fmt):
    """Definition check: no finite code is strictly closer, ties go to the even code,
    above max the result is max; sign kept."""
    rng = np.random.default_rng(7)
    top = mxfp.max_finite(fmt)
    table = mxfp.decode_table(fmt)
    fin = np.isfinite(table)
    y = np.concatenate([rng.standard_normal(4000) * top / 3, rng.standard_normal(2000) * 2.0 ** -8,
                        (np.arange(-600, 600) / 7.0), np.array([top * 1.02, -top * 1.5, 1e30, -0.0, 0.0])])
    # exact midpoints between neighbours (ties)
    pos = np.sort(table[fin & (table >= 0)])
    mids = (pos[1:] + pos[:-1]) / 2
    y = np.concatenate([y, mids, -mids])
    codes = mxfp.round_to_format(y, fmt)
    got = table[codes]
    tgt = np.clip(y, -top, top)
    d = np.abs(table[None, fin] - tgt[:, None])
    best = d.min(axis=1)
    assert np.all(np.abs(got - tgt) == best)
    tie = (d == best[:, None]).sum(axis=1) > 1
    tie_codes = codes[tie] & 0x7F
    assert np.all((tie_codes[tie_codes != 0] % 2) == 0)
    assert np.array_equal(codes >> 7, np.signbit(y).astype(np.uint8))


def test_worked_examples(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "mx_worked_examples.json")))
    for ex in spec["examples"]:
        g = np.zeros(32)
        if "fill" in ex:
            g[:] = ex["fill"]
        else:
            g[:len(ex["values"])] = ex["values"]
        codes, scales = mxfp.quantize(g[None, :], ex["fmt"])
        assert scales.shape == (1, 2), ex["name"]
        assert scales[0, 0] == ex["scale"], ex["name"]
        assert scales[0, 1] == 0, ex["name"]   # padding scale of an odd group count
        for j, c in ex["codes"].items():
            assert codes[0, int(j)] == c, (ex["name"], j, codes[0, int(j)], c)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_scale_rule_invariants(fmt):
    """amax / X lies in [2^emax, 2^(emax+1)) unless the E8M0 byte is clamped."""
    rng = np.random.default_rng(3)
    v = rng.standard_normal((500, 96)) * np.exp(rng.uniform(-30, 30, size=(500, 1)))
    codes, scales = mxfp.quantize(v, fmt)
    assert scales.shape == (500, 4) and np.all(scales[:, 3] == 0)
    amax = np.abs(v.reshape(500, 3, 32)).max(axis=2)
    ratio = amax / mxfp.e8m0_value(scales[:, :3])
    em = mxfp.EMAX[fmt]
    assert np.all((ratio >= 2.0 ** em) & (ratio < 2.0 ** (em + 1)))


@pytest.mark.parametrize("fmt,mbits,esub", [("e4m3", 3, -9), ("e5m2", 2, -16)])
def test_round_trip_bound_exhaustive(fmt, mbits, esub):
    """Every finite bf16 value against a sweep of shared scales: the dequantized value is
    within half an ulp of the format (relative 2^-(m+1) for normals, 2^(esub-1) absolute
    for subnormals), or clamped to max when it is above max."""
    top = mxfp.max_finite(fmt)
    v = all_bf16_finite()
    for b in (100, 112, 119, 127, 134, 150):
        x = 2.0 ** (b - 127)
        y = v / x
        codes = mxfp.round_to_format(y, fmt)
        back = mxfp.decode_table(fmt)[codes]
        err = np.abs(back - y)
        inside = np.abs(y) <= top
        bound = np.maximum(2.0 ** -(mbits + 1) * np.abs(y), 2.0 ** (esub - 1))
        assert np.all(err[inside] <= bound[inside])
        assert np.all(back[~inside] == np.sign(y[~inside]) * top)


def test_dequantize_inverts_exact_values():
    rng = np.random.default_rng(5)
    for fmt in ("e4m3", "e5m2"):
        codes = rng.integers(0, 256, size=(7, 64)).astype(np.uint8)
        t = mxfp.decode_table(fmt)
        codes[~np.isfinite(t[codes])] = 0
        scales = np.zeros((7, 2), np.uint8)
        scales[:] = rng.integers(120, 135, size=(7, 2))
        d = mxfp.dequantize(codes, scales, fmt)
        assert np.array_equal(d[:, 5], t[codes[:, 5]] * 2.0 ** (scales[:, 0].astype(int) - 127))
        assert np.array_equal(d[:, 40], t[codes[:, 40]] * 2.0 ** (scales[:, 1].astype(int) - 127))


def test_scale_cols():
    assert mxfp.scale_cols(128) == 4      # the article's MXFP8 example: H=128 -> 4 scale columns
    assert mxfp.scale_cols(7168) == 224 and mxfp.scale_cols(96) == 4 and mxfp.scale_cols(32) == 2
    assert mxfp.scale_cols(2048) == 64 and mxfp.scale_cols(1) == 2


def test_bf16_round():
    rng = np.random.default_rng(11)
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-80, 80, 20000))).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(f.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mxfp.bf16_round(f), ref)
    # one rounding from float64: just above a tie rounds up (a float32 detour would round to even)
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert mxfp.bf16_round(np.array([v]))[0] == 1.0 + 2.0 ** -7
    assert mxfp.bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert mxfp.bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    bits = mxfp.bf16_bits(np.array([1.0, -2.0, 0.0]))
    assert list(bits) == [0x3F80, 0xC000, 0x0000]


# ---- MXFP4 (FLOAT4_E2M1), quantMode 9 -------------------------------------------

def test_e2m1_table_and_closed_forms():
    """E2M1: sign bit 0x8, 2 exponent bits (bias 1), 1 mantissa bit, every code finite;
    the eight magnitudes 0, 0.5 (subnormal), 1, 1.5, 2, 3, 4, 6."""
    t = mxfp.decode_table("e2m1")
    assert t.tolist()[:8] == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.array_equal(t[8:], -t[:8])
    assert mxfp.max_finite("e2m1") == 6.0 and mxfp.EMAX["e2m1"] == 2
    # hand-derived groups: all 1.0 -> X = 2^(0 - 2) -> scale 125, 1.0 / X = 4 -> code 6
    c, s = mxfp.quantize(np.ones((1, 32)), "e2m1")
    assert np.all(c == 6) and s.tolist() == [[125, 0]]
    # amax 7.9 -> X = 2^(2 - 2) = 1: 6 -> 7, 3 -> 5, 1.5 -> 3, 0.75 (tie 0.5 / 1.0) -> 2,
    # -2.5 (tie 2 / 3) -> 0x8 | 4, 7.9 -> saturated 6 (7), 0.25 (tie 0 / 0.5) -> 0, -0.1 -> -0 (8)
    v = np.zeros((1, 32))
    v[0, :8] = [6, 3, 1.5, 0.75, -2.5, 7.9, 0.25, -0.1]
    c, s = mxfp.quantize(v, "e2m1")
    assert c[0, :8].tolist() == [7, 5, 3, 2, 12, 7, 0, 8] and s[0, 0] == 127
    # powers of two: 2^p -> scale p - 2 + 127, element 4 (code 6)
    for p in (-20, -3, 0, 5, 40):
        c, s = mxfp.quantize(np.full((1, 32), 2.0 ** p), "e2m1")
        assert s[0, 0] == p + 125 and np.all(c == 6)


def test_e2m1_rounding_is_nearest_by_brute_force():
    rng = np.random.default_rng(8)
    t = mxfp.decode_table("e2m1")
    pos = t[:8]
    mids = (pos[1:] + pos[:-1]) / 2
    y = np.concatenate([rng.uniform(-7, 7, 5000), mids, -mids, [6.5, -9.0, 1e9, 0.0, -0.0]])
    codes = mxfp.round_to_format(y, "e2m1")
    assert codes.max() < 16
    got = t[codes]
    tgt = np.clip(y, -6, 6)
    d = np.abs(t[None, :] - tgt[:, None])
    best = d.min(axis=1)
    assert np.all(np.abs(got - tgt) == best)
    tie = (d == best[:, None]).sum(axis=1) > 2      # +-0 always tie with each other
    mag = codes[tie] & 0x7
    assert np.all(mag % 2 == 0)
    assert np.array_equal(codes >> 3, np.signbit(y).astype(np.uint8))


def test_e2m1_round_trip_bound_and_scale_rule():
    """Half an E2M1 ulp (relative 2^-2 for normals, 2^-2 absolute below 1) or clamped to
    6; amax / X in [4, 8) unless the E8M0 byte is clamped."""
    v = all_bf16_finite()
    for b in (110, 125, 127, 140):
        x = 2.0 ** (b - 127)
        y = v / x
        back = mxfp.decode_table("e2m1")[mxfp.round_to_format(y, "e2m1")]
        inside = np.abs(y) <= 6
        bound = np.maximum(0.25 * np.abs(y), 0.25)
        assert np.all(np.abs(back - y)[inside] <= bound[inside])
        assert np.all(back[~inside] == np.sign(y[~inside]) * 6)
    rng = np.random.default_rng(9)
    v = rng.standard_normal((300, 64)) * np.exp(rng.uniform(-20, 20, size=(300, 1)))
    _, s = mxfp.quantize(v, "e2m1")
    ratio = np.abs(v.reshape(300, 2, 32)).max(axis=2) / mxfp.e8m0_value(s[:, :2])
    assert np.all((ratio >= 4) & (ratio < 8))


def test_fp4_packing():
    c = np.array([[1, 2, 3, 15, 0, 8]], np.uint8)
    p = mxfp.pack_fp4(c)
    assert p.tolist() == [[0x21, 0xF3, 0x80]]
    assert np.array_equal(mxfp.unpack_fp4(p), c)
