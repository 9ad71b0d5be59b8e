"""Pins for the oracle's number formats and the pinned SiLU exponential.

E4M3 is checked against a brute-force nearest-value search over the 256 code
values (ties to the even code), against hand-derived points from the OCP
definition, and against torch's float8_e4m3fn; bf16 against torch's cast; the
exponential against libm within 2 ulp.
"""
import json

import numpy as np
import pytest
import torch

from conftest import GOLDEN


def _brute_e4m3(x, table):
    """Nearest finite E4M3 value by search; ties -> even code; |x| >= 448 -> +-448."""
    fin = np.array([c for c in range(128) if not np.isnan(table[c])])
    vals = table[fin].astype(np.float64)          # non-negative codes 0x00..0x7E, increasing
    a = np.abs(x.astype(np.float64))
    pos = np.searchsorted(vals, a)                # vals[pos-1] < a <= vals[pos]
    hi = np.clip(pos, 0, len(vals) - 1)
    lo = np.clip(pos - 1, 0, len(vals) - 1)
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(fin[lo] % 2 == 0, lo, hi)))
    pick = np.where(a >= 448.0, len(vals) - 1, pick)
    code = fin[pick].astype(np.uint8)
    return code | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)


def test_e4m3_golden_points(oracle_mod):
    g = json.loads((GOLDEN / "e4m3_points.json").read_text())
    table = oracle_mod.e4m3_decode_table()
    for code, val in g["decode"]:
        assert table[int(code, 16)] == np.float32(val), code
    assert np.isnan(table[0x7F]) and np.isnan(table[0xFF])
    for val, code in g["encode"]:
        assert int(oracle_mod.e4m3_encode(np.float32(val))[0]) == int(code, 16), val


def test_e4m3_decode_matches_torch(oracle_mod):
    table = oracle_mod.e4m3_decode_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(table), ~fin)
    np.testing.assert_array_equal(table[fin], ref[fin])


def _interesting_floats(table):
    fin = np.sort(np.unique(np.abs(table[~np.isnan(table)]).astype(np.float64)))
    mids = (fin[:-1] + fin[1:]) / 2
    pts = np.concatenate([fin, mids, [464.0, 480.0, 500.0, 1e6, 3e38, 2.0 ** -10, 2.0 ** -12, 1e-30]])
    pts = pts.astype(np.float32)
    near = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)), np.nextafter(pts, np.float32(0))])
    return np.concatenate([near, -near, np.array([0.0, -0.0], np.float32)])


def test_e4m3_encode_brute_force(oracle_mod):
    table = oracle_mod.e4m3_decode_table()
    rng = np.random.default_rng(7)
    # every bf16-representable fp32 (all exponents, top 7 mantissa bits), the
    # code values, midpoints and their neighbours, and 4M random finite bit patterns
    bf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    bf = bf[np.isfinite(bf)]
    rnd = rng.integers(0, 2 ** 32, 1 << 22, dtype=np.uint64).astype(np.uint32).view(np.float32)
    rnd = rnd[np.isfinite(rnd)]
    # dense values inside the E4M3 range
    dense = rng.uniform(-460, 460, 1 << 20).astype(np.float32)
    small = (rng.uniform(-1, 1, 1 << 20) * 2.0 ** rng.integers(-14, 0, 1 << 20)).astype(np.float32)
    x = np.concatenate([bf, _interesting_floats(table), rnd, dense, small])
    np.testing.assert_array_equal(oracle_mod.e4m3_encode(x), _brute_e4m3(x, table))


def test_e4m3_encode_matches_torch_in_range(oracle_mod):
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.uniform(-448, 448, 1 << 20), rng.normal(0, 1, 1 << 20),
                        rng.normal(0, 1e-3, 1 << 18)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle_mod.e4m3_encode(x), ref)


def test_bf16_matches_torch(oracle_mod):
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 2 ** 32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # ties: low 16 bits exactly 0x8000, with both parities of bit 16
    ties = ((rng.integers(0, 2 ** 16, 4096, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    x = np.concatenate([x, ties, rng.normal(0, 1, 1 << 20).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle_mod.f32_to_bf16(x), ref)
    back = oracle_mod.bf16_to_f32(ref)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def _ulp_diff(a32, b64):
    """|a - b| in units of the fp32 ulp at b."""
    b32 = b64.astype(np.float32)
    ulp = np.abs(np.nextafter(b32, np.float32(np.inf)) - b32).astype(np.float64)
    return np.abs(a32.astype(np.float64) - b64) / ulp


def test_exp_within_2ulp(oracle_mod):
    y = np.linspace(-20, 20, 2_000_001, dtype=np.float32)
    got = oracle_mod.exp_k(y)
    assert np.max(_ulp_diff(got, np.exp(y.astype(np.float64)))) <= 2.0
    # the wider normal range it covers
    y2 = np.linspace(-87, 88, 400_001, dtype=np.float32)
    assert np.max(_ulp_diff(oracle_mod.exp_k(y2), np.exp(y2.astype(np.float64)))) <= 2.0


def test_exp_special_values(oracle_mod):
    e = oracle_mod.exp_k(np.array([0.0, -0.0, 88.5, 1000.0, -87.5, -1000.0], np.float32))
    assert e[0] == 1.0 and e[1] == 1.0
    assert np.isinf(e[2]) and np.isinf(e[3])
    assert e[4] == 0.0 and e[5] == 0.0


def test_silu_against_float64(oracle_mod):
    v = np.concatenate([np.linspace(-30, 30, 600_001), [0.0, 100.0, -100.0, 1e4, -1e4]]).astype(np.float32)
    got = oracle_mod.silu(v).astype(np.float64)
    v64 = v.astype(np.float64)
    with np.errstate(over="ignore"):
        ref = v64 / (1.0 + np.exp(-v64))
    assert got[np.where(v == 0)[0][0]] == 0.0
    # a few fp32 roundings of a well-conditioned expression
    assert np.all(np.abs(got - ref) <= 4 * 2.0 ** -24 * np.abs(ref) + 1e-37)


# ------------------------------------------------ 16-bit KV value formats ----

def test_fp16_widen_narrow_exhaustive_and_vs_torch(oracle_mod):
    """Every finite fp16 pattern widens to the fp32 torch gives and narrows
    back to itself; random fp32 values narrow as torch's fp16 cast does."""
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    fin = np.isfinite(bits.view(np.float16))
    w = oracle_mod.widen16(bits[fin], 1)
    t = torch.from_numpy(bits[fin].view(np.int16)).view(torch.float16).float().numpy()
    np.testing.assert_array_equal(w.view(np.uint32), t.view(np.uint32))
    np.testing.assert_array_equal(oracle_mod.narrow16(w, 1), bits[fin])
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(1 << 20) * np.exp2(rng.uniform(-30, 17, 1 << 20))).astype(np.float32)
    x = x[np.abs(x) < 65504]
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle_mod.narrow16(x, 1), ref)


def test_bf16_widen_narrow_round_trip(oracle_mod):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    fin = np.isfinite(oracle_mod.bf16_to_f32(bits))
    w = oracle_mod.widen16(bits[fin], 2)
    np.testing.assert_array_equal(oracle_mod.narrow16(w, 2), bits[fin])
