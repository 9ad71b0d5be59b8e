"""Pins for the oracle's INT4 AWQ pieces (boostr fused_int4_qkv.rs).

Nibble order from a hand-derived example, pack/unpack round trips, the
product in exact rationals on tiny shapes, unit scales with zero offsets as
an integer matmul, z == q giving zero, and the single projection being the Q
part of the fused call.
"""
import json
from fractions import Fraction

import numpy as np

from conftest import GOLDEN
from kv_quantization_amd import synth


def test_awq_order_golden(oracle_mod):
    g = json.loads((GOLDEN / "awq_order.json").read_text())
    assert tuple(g["shifts"]) == oracle_mod.AWQ_SHIFTS
    for word, cols in g["unpack"]:
        got = oracle_mod.awq_unpack(np.array([[int(word, 16)]], np.uint32), 8)[0]
        np.testing.assert_array_equal(got, np.array(cols, np.uint8))
    for cols, word in g["pack"]:
        got = oracle_mod.awq_pack(np.array([cols], np.uint8))[0, 0]
        assert int(got) == int(word, 16)


def test_awq_round_trips(oracle_mod):
    rng = np.random.default_rng(41)
    words = rng.integers(0, 2 ** 32, (64, 32), dtype=np.uint64).astype(np.uint32)
    np.testing.assert_array_equal(oracle_mod.awq_pack(oracle_mod.awq_unpack(words, 256)), words)
    codes = rng.integers(0, 16, (64, 256), dtype=np.uint8)
    np.testing.assert_array_equal(oracle_mod.awq_unpack(oracle_mod.awq_pack(codes), 256), codes)
    # unpacked uniform words give (near-)uniform codes 0..15
    c = oracle_mod.awq_unpack(rng.integers(0, 2 ** 32, (512, 64), dtype=np.uint64).astype(np.uint32), 512)
    counts = np.bincount(c.ravel(), minlength=16)
    assert counts.min() > 0.9 * c.size / 16 and counts.max() < 1.1 * c.size / 16


def test_awq_brute_force_rationals(oracle_mod):
    rng = np.random.default_rng(42)
    m, k, n, gs = 3, 16, 16, 8
    x, (p,) = synth.int4_awq(m, k, (n,), gs, seed=43)
    codes = oracle_mod.awq_unpack(p.qweight, n)
    ref, bound = oracle_mod.int4_awq_gemm(x, p.qweight, p.scales, p.zeros, gs)
    for r in range(m):
        for j in range(n):
            tot, ab = Fraction(0), Fraction(0)
            for c in range(k):
                w = (Fraction(int(codes[c, j])) - Fraction(float(p.zeros[c // gs, j]))) * Fraction(float(p.scales[c // gs, j]))
                t = Fraction(float(x[r, c])) * w
                tot += t
                ab += abs(t)
            assert abs(ref[r, j] - float(tot)) <= 1e-12 * float(ab)
            assert abs(bound[r, j] - float(ab)) <= 1e-12 * float(ab)


def test_awq_unit_scale_zero_offset_is_int_matmul(oracle_mod):
    rng = np.random.default_rng(44)
    m, k, n, gs = 5, 256, 64, 128
    codes = rng.integers(0, 16, (k, n), dtype=np.uint8)
    xi = rng.integers(-50, 50, (m, k))
    qw = oracle_mod.awq_pack(codes)
    ones = np.ones((k // gs, n), np.float32)
    zeros = np.zeros((k // gs, n), np.float32)
    ref, _ = oracle_mod.int4_awq_gemm(xi.astype(np.float32), qw, ones, zeros, gs)
    np.testing.assert_array_equal(ref, (xi.astype(np.int64) @ codes.astype(np.int64)).astype(np.float64))


def test_awq_zero_equals_code_gives_zero(oracle_mod):
    rng = np.random.default_rng(45)
    k, n, gs = 128, 32, 32
    const = rng.integers(0, 16, (k // gs, n), dtype=np.uint8)
    codes = np.repeat(const, gs, axis=0)
    qw = oracle_mod.awq_pack(codes)
    x = rng.normal(0, 1, (3, k)).astype(np.float32)
    ref, _ = oracle_mod.int4_awq_gemm(x, qw, rng.uniform(0.001, 0.02, (k // gs, n)).astype(np.float32),
                                      const.astype(np.float32), gs)
    assert np.all(ref == 0.0)


def test_awq_single_projection_is_q_part(oracle_mod):
    x, projs = synth.int4_awq(2, 256, (64, 16, 16), 128, seed=46)
    outs = oracle_mod.int4_awq_qkv(x, [(p.qweight, p.scales, p.zeros) for p in projs], 128)
    single = oracle_mod.int4_awq_gemm(x, projs[0].qweight, projs[0].scales, projs[0].zeros, 128)
    np.testing.assert_array_equal(outs[0][0], single[0])
