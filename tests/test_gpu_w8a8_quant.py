"""GPU parity: W8A8 activation quantization, weight quantization and the
E4M3 encoder vs the oracle, bit for bit, through the C ABI."""
import numpy as np
import pytest
import torch

from conftest import print_case
from gpu_util import assert_bits_equal, assert_canary, dev, host, poisoned
from kv_quantization_amd import api, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _bind_oracle(oracle_mod):
    global _oracle
    _oracle = oracle_mod


def _act_case(x_bf16, k, kind, silu=False, up=None):
    rows, ldx = x_bf16.shape
    q, raw_q = poisoned((rows, k), torch.uint8)
    sshape = (rows,) if kind == 0 else (rows, k // 128)
    s, raw_s = poisoned(sshape, torch.float32)
    api.act_quant(dev(x_bf16), k, kind, silu, None if up is None else dev(up), q, s)
    rq, rs = _oracle.act_quant(kind, x_bf16, k, silu=silu, up_bf16=up)
    torch.cuda.synchronize()
    assert_bits_equal(host(q), rq, "act codes")
    assert_bits_equal(host(s), rs, "act scales")
    assert_canary(raw_q, rows * k)
    assert_canary(raw_s, int(np.prod(sshape)) * 4)


@pytest.mark.parametrize("m", [1, 8, 32])
def test_act_quant_rowscale_qkv_shape(m):
    print_case("act row qkv", m)
    inp = synth.w8a8_qkv()
    _act_case(inp.x_bf16[:m], 4096, 0)


@pytest.mark.parametrize("m", [64, 128, 256])
@pytest.mark.parametrize("with_up", [False, True])
def test_act_quant_g128_silu_down_shape(m, with_up):
    print_case("act g128 silu down", m, with_up)
    inp = synth.w8a8_down(with_up=with_up)
    _act_case(inp.x_bf16[:m], 14336, 1, silu=True, up=None if inp.up_bf16 is None else inp.up_bf16[:m])


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("silu,with_up", [(False, False), (True, False), (True, True)])
@pytest.mark.parametrize("rows,k,ldx", [(1, 128, 128), (3, 384, 392), (256, 256, 256), (5, 2176, 2176), (2, 14336, 14344)])
def test_act_quant_edges(kind, silu, with_up, rows, k, ldx):
    print_case("act edges", kind, silu, with_up, rows, k, ldx)
    inp = synth.w8a8(rows, ldx, (128,), seed=rows + k + ldx, with_up=with_up)
    x = inp.x_bf16.copy()
    if rows >= 3:
        x[1] = 0                                  # zero row -> floor scale
        x[2, : k // 2] = _oracle.f32_to_bf16(np.full(k // 2, 30.0, np.float32))   # large SiLU inputs
    _act_case(x, k, kind, silu, inp.up_bf16)


def test_act_quant_extreme_silu_inputs():
    print_case("act silu extremes")
    v = np.array([0, -0.0, 1e-30, -1e-30, 87, -87, 88, -88, 89, -89, 100, -100, 3e38, -3e38, 0.5, -0.5] * 8,
                 np.float32)
    x = _oracle.f32_to_bf16(v.reshape(1, 128))
    for kind in (0, 1):
        _act_case(x, 128, kind, silu=True)
        _act_case(x, 128, kind, silu=False)


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("n,k", [(6144, 4096), (300, 384), (1, 128), (129, 256)])
def test_weight_quant(kind, n, k):
    print_case("weight quant", kind, n, k)
    w = synth.w8a8(1, k, (n,), seed=n + k).weights[0]
    rq, rs = _oracle.weight_quant(kind, w)
    q, s = api.weight_quant(dev(w), kind)
    torch.cuda.synchronize()
    assert_bits_equal(host(q), rq, "weight codes")
    assert_bits_equal(host(s), rs, "weight scales")


def test_weight_quant_down_blk128_full():
    print_case("weight quant down blk128")
    w = synth.w8a8_down().weights[0]
    rq, rs = _oracle.weight_quant(1, w)
    q, s = api.weight_quant(dev(w), 1)
    torch.cuda.synchronize()
    assert_bits_equal(host(q), rq, "weight codes")
    assert_bits_equal(host(s), rs, "weight scales")


def test_e4m3_encoder_all_finite_fp32():
    """Every finite fp32 bit pattern through the device encoder, vs the oracle."""
    print_case("e4m3 exhaustive")
    chunk = 1 << 27
    for start in range(0, 1 << 32, chunk):
        bits = np.arange(chunk, dtype=np.uint32) + np.uint32(start)
        x = bits.view(np.float32)
        fin = np.isfinite(x)
        if not fin.all():
            x = x[fin]
        ref = _oracle.e4m3_encode(x)
        got = host(api.f32_to_e4m3(dev(x)))
        if not np.array_equal(got, ref):
            bad = np.nonzero(got != ref)[0][:5]
            raise AssertionError(f"chunk {start:#x}: {int((got != ref).sum())} mismatches, e.g. "
                                 f"{[(float(x[i]), hex(x[i:i+1].view(np.uint32)[0]), int(got[i]), int(ref[i])) for i in bad]}")


@pytest.mark.parametrize("n", [1, 3, 5, 1000, 4099])
def test_e4m3_encoder_ragged(n):
    print_case("e4m3 ragged", n)
    x = np.random.default_rng(n).normal(0, 100, n).astype(np.float32)
    out, raw = poisoned((n,), torch.uint8)
    api.f32_to_e4m3(dev(x), out)
    torch.cuda.synchronize()
    assert_bits_equal(host(out), _oracle.e4m3_encode(x), "e4m3")
    assert_canary(raw, n)


def _wide_range(rows, k, seed):
    """Rows whose magnitudes span many binades (log-uniform 2^-40 .. 2^40 per
    row, elements log-uniform over 2^-30 of that, random signs, some exact
    zeros and row maxima): quotients v / s land on every E4M3 code boundary."""
    rng = np.random.default_rng(seed)
    top = np.exp2(rng.uniform(-40, 40, (rows, 1)))
    x = top * np.exp2(-rng.uniform(0, 30, (rows, k))) * rng.choice([-1.0, 1.0], (rows, k))
    x[rng.random((rows, k)) < 0.01] = 0.0
    x[:, 0] = top[:, 0]
    return synth.to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("kind", [0, 1])
def test_act_quant_wide_range_codes(kind):
    # the encoders divide by the scale with a reciprocal and one correction
    # step; codes must still equal those of an IEEE division (the oracle's)
    print_case("act wide range", kind)
    _act_case(_wide_range(256, 8192, 77 + kind), 8192, kind)
