"""Pins for the oracle's W8A8 pieces (metrale_model_layers w8a8_decode.rs).

Activation/weight quantization: the absmax element encodes to +-448, the
floor for zero rows, g128 == row when every group shares its maximum, and the
reconstruction error stays within half an E4M3 step.  The product reference:
brute force in exact rationals on tiny shapes, segment invariance, blk128 with
uniform scales == rowscale, integer codes with unit scales == numpy integer
matmul, and row independence.
"""
from fractions import Fraction

import numpy as np
import pytest

from kv_quantization_amd import synth


def _e4m3_step(v):
    """Spacing of E4M3 values around |v| (v already divided by the scale)."""
    a = np.abs(v.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 2.0 ** (e - 3)


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("silu,with_up", [(False, False), (True, False), (True, True)])
def test_act_quant_properties(oracle_mod, kind, silu, with_up):
    rows, k = 5, 512
    inp = synth.w8a8(rows, k, (128,), seed=21, with_up=with_up)
    x = inp.x_bf16
    q, s = oracle_mod.act_quant(kind, x, k, silu=silu, up_bf16=inp.up_bf16)
    v = oracle_mod.bf16_to_f32(x).astype(np.float32)
    if silu:
        v = oracle_mod.silu(v)
    if with_up:
        v = (v * oracle_mod.bf16_to_f32(inp.up_bf16)).astype(np.float32)
    table = oracle_mod.e4m3_decode_table().astype(np.float64)
    span = k if kind == 0 else 128
    vg = v.reshape(rows, k // span, span).astype(np.float64)
    qg = q.reshape(rows, k // span, span)
    sg = s.reshape(rows, k // span, 1).astype(np.float64)
    amax = np.abs(vg).max(axis=2, keepdims=True)
    assert np.all(np.abs(sg - np.maximum(amax / 448.0, 1e-8)) <= 2.0 ** -23 * sg)
    # the group's absmax element encodes to +-448
    idx = np.abs(vg).argmax(axis=2)
    top = np.take_along_axis(qg, idx[..., None], axis=2)
    assert np.all((top & 0x7F) == 0x7E)
    # reconstruction within half an E4M3 step (plus the quotient rounding)
    rec = table[qg] * sg
    assert np.all(np.abs(rec - vg) <= sg * (_e4m3_step(vg / sg) / 2 * (1 + 2.0 ** -20) + 2.0 ** -22 * np.abs(vg / sg)))
    # codes keep the sign of the value
    nz = vg != 0
    assert np.all((np.signbit(table[qg]) == np.signbit(vg))[nz & (table[qg] != 0)])


def test_act_quant_zero_row_and_g128_equals_row(oracle_mod):
    k = 384
    x = np.zeros((2, k), np.float32)
    # row 1: every 128-group has the same absmax (ones with a +-7 spike)
    rng = np.random.default_rng(5)
    x[1] = rng.uniform(-3, 3, k).astype(np.float32)
    x[1, [5, 130, 300]] = [7.0, -7.0, 7.0]
    xb = oracle_mod.f32_to_bf16(x)
    q0, s0 = oracle_mod.act_quant(0, xb, k)
    q1, s1 = oracle_mod.act_quant(1, xb, k)
    assert s0[0] == np.float32(1e-8) and np.all(q0[0] == 0)
    assert np.all(s1[0] == np.float32(1e-8))
    np.testing.assert_array_equal(q0[1], q1[1])
    assert np.all(s1[1] == s0[1])


def test_act_quant_ldx_padding_ignored(oracle_mod):
    inp = synth.w8a8(3, 256, (128,), seed=23)
    xpad = np.zeros((3, 264), np.uint16)
    xpad[:, :256] = inp.x_bf16
    xpad[:, 256:] = 0x7F7F      # garbage past k must not be read
    for kind in (0, 1):
        a = oracle_mod.act_quant(kind, inp.x_bf16, 256)
        b = oracle_mod.act_quant(kind, xpad, 256)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("kind", [0, 1])
def test_weight_quant_properties(oracle_mod, kind):
    n, k = 300, 384           # ragged last 128-block band (300 = 2*128 + 44)
    w = synth.w8a8(1, k, (n,), seed=24).weights[0]
    q, s = oracle_mod.weight_quant(kind, w)
    table = oracle_mod.e4m3_decode_table().astype(np.float64)
    if kind == 0:
        sfull = np.repeat(s[:, None], k, axis=1).astype(np.float64)
    else:
        assert s.shape == (3, 3)
        sfull = np.repeat(np.repeat(s, 128, axis=0)[:n], 128, axis=1).astype(np.float64)
    w64 = w.astype(np.float64)
    rec = table[q] * sfull
    assert np.all(np.abs(rec - w64) <= sfull * (_e4m3_step(w64 / sfull) / 2 * (1 + 2.0 ** -20) + 2.0 ** -22 * np.abs(w64 / sfull)))
    # each scale's block holds an element encoded to +-448
    if kind == 0:
        assert np.all(((q & 0x7F) == 0x7E).any(axis=1))
    else:
        for jb in range(3):
            for cb in range(3):
                blk = q[jb * 128:(jb + 1) * 128, cb * 128:(cb + 1) * 128]
                assert ((blk & 0x7F) == 0x7E).any()


# ------------------------------------------------------------ the product --

def _frac_e4m3(c):
    sign = -1 if c & 0x80 else 1
    e, m = (c >> 3) & 15, c & 7
    if e == 0:
        return sign * Fraction(m, 8) * Fraction(1, 64)
    return sign * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def test_gemv_brute_force_rationals(oracle_mod):
    rng = np.random.default_rng(31)
    k, m = 256, 2
    segs_n = (16, 8)
    qa = rng.integers(0, 256, (m, k), dtype=np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x3C               # no NaN codes
    for kind in (0, 1):
        sa = rng.uniform(0.5, 2, (m,) if kind == 0 else (m, k // 128)).astype(np.float32)
        segs = []
        for n in segs_n:
            qw = rng.integers(0, 256, (n, k), dtype=np.uint8)
            qw[(qw & 0x7F) == 0x7F] = 0x41
            sw = rng.uniform(0.5, 2, (n,) if kind == 0 else ((n + 127) // 128, k // 128)).astype(np.float32)
            segs.append((qw, sw))
        ref, bound = oracle_mod.w8a8_gemv(kind, qa, sa, segs)
        col = 0
        for qw, sw in segs:
            for j in range(qw.shape[0]):
                for r in range(m):
                    tot, ab = Fraction(0), Fraction(0)
                    for c in range(k):
                        a_s = Fraction(float(sa[r])) if kind == 0 else Fraction(float(sa[r, c // 128]))
                        w_s = Fraction(float(sw[j])) if kind == 0 else Fraction(float(sw[j // 128, c // 128]))
                        t = _frac_e4m3(int(qa[r, c])) * a_s * _frac_e4m3(int(qw[j, c])) * w_s
                        tot += t
                        ab += abs(t)
                    assert abs(ref[r, col + j] - float(tot)) <= 1e-12 * float(ab) + 1e-300
                    assert abs(bound[r, col + j] - float(ab)) <= 1e-12 * float(ab)
            col += qw.shape[0]


def test_gemv_segment_invariance_and_rows(oracle_mod):
    inp = synth.w8a8(6, 512, (256, 128, 64), seed=32)
    for kind in (0, 1):
        q, sa = oracle_mod.act_quant(kind, inp.x_bf16, 512)
        segs = [oracle_mod.weight_quant(kind, w) for w in inp.weights]
        ref3, _ = oracle_mod.w8a8_gemv(kind, q, sa, segs)
        allw = np.concatenate(inp.weights, axis=0)
        if kind == 0:
            # per-row scales do not depend on the split
            one = [oracle_mod.weight_quant(0, allw)]
            ref1, _ = oracle_mod.w8a8_gemv(0, q, sa, one)
            np.testing.assert_allclose(ref1, ref3, rtol=0, atol=1e-12)
        # row independence: each row alone gives the same outputs
        for r in range(6):
            rr, _ = oracle_mod.w8a8_gemv(kind, q[r:r + 1], sa[r:r + 1], segs)
            np.testing.assert_allclose(rr[0], ref3[r], rtol=0, atol=1e-12)
        # sampled evaluation agrees with the full one
        rows = np.array([0, 5, 3, 2]); cols = np.array([0, 300, 383, 447])
        sr, sb = oracle_mod.w8a8_gemv_sampled(kind, q, sa, segs, rows, cols)
        np.testing.assert_allclose(sr, ref3[rows, cols], rtol=0, atol=1e-12)


def test_gemv_blk128_uniform_scales_equals_rowscale(oracle_mod):
    rng = np.random.default_rng(33)
    m, n, k = 3, 256, 384
    qa = rng.integers(0, 0x7E, (m, k), dtype=np.uint8) | (rng.integers(0, 2, (m, k), dtype=np.uint8) << 7)
    qw = rng.integers(0, 0x7E, (n, k), dtype=np.uint8)
    sa_row = rng.uniform(0.1, 1, m).astype(np.float32)
    sw_band = rng.uniform(0.1, 1, n // 128).astype(np.float32)
    sw_row = np.repeat(sw_band, 128)
    r_row, _ = oracle_mod.w8a8_gemv(0, qa, sa_row, [(qw, sw_row)])
    r_blk, _ = oracle_mod.w8a8_gemv(1, qa, np.repeat(sa_row[:, None], k // 128, axis=1),
                                     [(qw, np.repeat(sw_band[:, None], k // 128, axis=1))])
    np.testing.assert_allclose(r_blk, r_row, rtol=1e-14, atol=1e-12)


def test_gemv_integer_codes_unit_scales_is_int_matmul(oracle_mod):
    # codes for the integers -8..8 (exact in E4M3): 0x38 + ... built from the table
    table = oracle_mod.e4m3_decode_table()
    ints = {int(v): c for c, v in enumerate(table[:0x7F]) if np.isfinite(v) and v == int(v) and abs(v) <= 8}
    ints.update({-int(v): c | 0x80 for v, c in list(ints.items())})
    vals = np.array(sorted(ints))
    rng = np.random.default_rng(34)
    m, n, k = 4, 40, 256
    ia = rng.choice(vals, (m, k)); iw = rng.choice(vals, (n, k))
    qa = np.vectorize(ints.get)(ia).astype(np.uint8)
    qw = np.vectorize(ints.get)(iw).astype(np.uint8)
    ref, _ = oracle_mod.w8a8_gemv(0, qa, np.ones(m, np.float32), [(qw, np.ones(n, np.float32))])
    np.testing.assert_array_equal(ref, (ia.astype(np.int64) @ iw.T.astype(np.int64)).astype(np.float64))
