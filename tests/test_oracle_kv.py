"""Pins for the oracle's KV-cache codecs (boostr kv_cache_quant.wgsl).

Each test checks the oracle against something other than its own formula:
hand-derived worked examples, error bounds that follow from the definition,
invariants (clamps, extreme elements), and the page's degenerate cases.
"""
import json
import struct

import numpy as np
import pytest

from conftest import GOLDEN
from kv_quantization_amd import synth


def _hexf(h):
    return struct.unpack("<f", struct.pack("<I", int(h, 16)))[0]


def _bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


# ---------------------------------------------------------------- INT8 ----

def test_int8_worked_example(oracle_mod):
    g = json.loads((GOLDEN / "kv_int8_worked.json").read_text())
    x = np.array(g["x"], np.float32)
    codes, scales = oracle_mod.kv_int8_quant(x)
    np.testing.assert_array_equal(codes, np.array(g["codes"], np.int8))
    np.testing.assert_array_equal(_bits(scales), _bits(np.array([_hexf(h) for h in g["scales_hex"]], np.float32)))
    y = oracle_mod.kv_int8_dequant(codes, scales)
    np.testing.assert_array_equal(y, np.array(g["dequant"], np.float32))


def test_int8_fp8_section_is_same_code(oracle_mod):
    x = synth.kv_cache(512, 128, seed=11)
    c1, s1 = oracle_mod.kv_int8_quant(x)
    c2, s2 = oracle_mod.kv_fp8_quant(x)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(_bits(s1), _bits(s2))
    np.testing.assert_array_equal(oracle_mod.kv_int8_dequant(c1, s1), oracle_mod.kv_fp8_dequant(c2, s2))


@pytest.mark.parametrize("t,d", [(1000, 128), (33, 7), (5, 256), (1, 1)])
def test_int8_roundtrip_bound_and_extremes(oracle_mod, t, d):
    x = synth.kv_cache(t, d, seed=12 + d)
    codes, s = oracle_mod.kv_int8_quant(x)
    y = oracle_mod.kv_int8_dequant(codes, s)
    # scale: absmax/127 (never below the floor)
    amax = np.abs(x).astype(np.float64).max(axis=1)
    assert np.all(np.abs(s.astype(np.float64) - np.maximum(amax / 127.0, 1e-8)) <= 2.0 ** -23 * s)
    # |x - y| <= s/2 up to the fp32 rounding of the quotient and product
    err = np.abs(x.astype(np.float64) - y.astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 2.0 ** -16))
    # the absmax element reaches |code| = 127; -128 is unreachable for finite input
    idx = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(codes[np.arange(t), idx].astype(int)) == 127)
    assert codes.min() >= -127 and codes.max() <= 127


def test_int8_zero_and_tiny_tokens(oracle_mod):
    x = np.zeros((3, 16), np.float32)
    x[1, 3] = 5e-7         # absmax/127 < 1e-8: the floor wins
    x[2, :] = -1e-30
    codes, s = oracle_mod.kv_int8_quant(x)
    assert np.all(s == np.float32(1e-8))
    assert np.all(codes[0] == 0) and np.all(codes[2] == 0)
    assert codes[1, 3] == 50   # 5e-7 / 1e-8 = 50
    y = oracle_mod.kv_int8_dequant(codes, s)
    assert np.all(y[0] == 0)


# ---------------------------------------------------------------- INT4 ----

def test_int4_worked_example(oracle_mod):
    g = json.loads((GOLDEN / "kv_int4_worked.json").read_text())
    x = np.array(g["x"], np.float32)
    packed, scales, zeros = oracle_mod.kv_int4_quant(x, g["group_size"])
    np.testing.assert_array_equal(packed, np.array(g["packed"], np.uint8))
    np.testing.assert_array_equal(scales, np.array(g["scales"], np.float32))
    np.testing.assert_array_equal(_bits(zeros), _bits(np.array([_hexf(h) for h in g["zeros_hex"]], np.float32)))
    # nibble order: low nibble = even element
    codes = np.stack([packed & 0xF, packed >> 4], axis=1).ravel()
    np.testing.assert_array_equal(codes, np.array(g["codes"], np.uint8))
    y = oracle_mod.kv_int4_dequant(packed, scales, zeros, g["num_tokens"], g["head_dim"], g["group_size"])
    np.testing.assert_array_equal(y, np.array(g["dequant"], np.float32))
    assert not np.signbit(y[1, 0])  # constant group dequantizes to +0


@pytest.mark.parametrize("t,d,gs", [(512, 128, 32), (17, 96, 6), (4, 64, 128), (6, 96, 64), (8, 10, 2)])
def test_int4_roundtrip_bound_and_extremes(oracle_mod, t, d, gs):
    x = synth.kv_cache(t, d, seed=40 + gs)
    packed, s, z = oracle_mod.kv_int4_quant(x, gs)
    y = oracle_mod.kv_int4_dequant(packed, s, z, t, d, gs)
    xg = x.reshape(-1, gs).astype(np.float64)
    yg = y.reshape(-1, gs).astype(np.float64)
    mn, mx = xg.min(axis=1), xg.max(axis=1)
    s64 = s.astype(np.float64)
    assert np.all(np.abs(s64 - (mx - mn) / 15.0) <= 2.0 ** -22 * np.abs(s64) + 1e-45)
    # |x - y| <= s/2 plus the fp32 roundings of x-min, the quotient, c*s, z*s, the difference
    # (only where the scale is above the 1e-8 floor; below it the stored
    # unfloored scale no longer reconstructs, which is the page's behaviour)
    bound = s64[:, None] / 2 * (1 + 2.0 ** -20) + 8 * 2.0 ** -24 * (np.abs(xg) + np.abs(mn)[:, None])
    ok = s64 >= 1e-8
    assert ok.mean() > 0.99
    assert np.all((np.abs(xg - yg) <= bound)[ok])
    codes = np.stack([packed & 0xF, packed >> 4], axis=1).reshape(-1, gs)
    assert codes.max() <= 15
    rows = np.arange(codes.shape[0])
    assert np.all(codes[rows, xg.argmin(axis=1)] == 0)
    assert np.all(codes[rows, xg.argmax(axis=1)] == 15)


def test_int4_constant_group_literal(oracle_mod):
    x = np.full((1, 32), 3.25, np.float32)
    packed, s, z = oracle_mod.kv_int4_quant(x, 32)
    assert s[0] == 0.0 and np.all(packed == 0)
    assert z[0] == np.float32(-3.25) / np.float32(1e-8)
    y = oracle_mod.kv_int4_dequant(packed, s, z, 1, 32, 32)
    assert np.all(y == 0.0) and not np.any(np.signbit(y))


def test_int4_pack_positions(oracle_mod):
    # one group whose codes are 0..15 in order: byte i must be (2i) | (2i+1) << 4
    x = np.arange(16, dtype=np.float32)[None, :]
    packed, s, z = oracle_mod.kv_int4_quant(x, 16)
    assert s[0] == 1.0
    np.testing.assert_array_equal(packed, np.array([(2 * i) | ((2 * i + 1) << 4) for i in range(8)], np.uint8))


# ------------------------------------------------- INT8 per-tensor mode ----

def test_int8_tensor_worked_examples(oracle_mod):
    g = json.loads((GOLDEN / "kv_int8_tensor_worked.json").read_text())
    for case in g["cases"]:
        x = np.array(case["x"], np.float32)
        codes, scale = oracle_mod.kv_int8_quant_tensor(x)
        np.testing.assert_array_equal(codes, np.array(case["codes"], np.int8))
        np.testing.assert_array_equal(_bits(scale), _bits(np.array([_hexf(case["scale_hex"])], np.float32)))
        np.testing.assert_array_equal(oracle_mod.kv_int8_dequant_tensor(codes, scale),
                                      np.array(case["dequant"], np.float32))


@pytest.mark.parametrize("d", [1, 7, 128])
def test_int8_tensor_single_token_is_per_token(oracle_mod, d):
    x = synth.kv_cache(1, d, seed=40 + d)
    c1, s1 = oracle_mod.kv_int8_quant_tensor(x)
    c2, s2 = oracle_mod.kv_int8_quant(x)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(_bits(s1), _bits(s2))


@pytest.mark.parametrize("t,d", [(300, 128), (17, 5)])
def test_int8_tensor_equals_per_token_with_shared_absmax(oracle_mod, t, d):
    """Appending the tensor's absmax to every token gives each token that
    absmax, so the (separately pinned) per-token codec then uses the tensor's
    scale everywhere and must reproduce the per-tensor codes."""
    x = synth.kv_cache(t, d, seed=50 + t)
    codes, scale = oracle_mod.kv_int8_quant_tensor(x)
    a = np.float32(np.abs(x).max())
    xa = np.concatenate([x, np.full((t, 1), a, np.float32)], axis=1)
    c2, s2 = oracle_mod.kv_int8_quant(xa)
    np.testing.assert_array_equal(_bits(s2), np.full(t, _bits(scale)[0], np.uint32))
    np.testing.assert_array_equal(codes, c2[:, :d])


def test_int8_tensor_bound_and_extremes(oracle_mod):
    x = synth.kv_cache(2000, 64, seed=60)
    codes, scale = oracle_mod.kv_int8_quant_tensor(x)
    s = float(scale[0])
    assert abs(s - max(float(np.abs(x).astype(np.float64).max()) / 127.0, 1e-8)) <= 2.0 ** -23 * s
    y = oracle_mod.kv_int8_dequant_tensor(codes, scale)
    assert np.all(np.abs(x.astype(np.float64) - y) <= s * (0.5 + 2.0 ** -16))
    i = np.unravel_index(np.abs(x).argmax(), x.shape)
    assert abs(int(codes[i])) == 127
    assert codes.min() >= -127 and codes.max() <= 127
