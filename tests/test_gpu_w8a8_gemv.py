"""GPU parity: W8A8 FP8 GEMV/GEMM (w8a8_gemv, w8a8_proj) vs the oracle's fp64
definition, |gpu - ref| <= 1e-3 * sum|a||w| per output, through the C ABI.

The activations and weights given to both sides are the oracle's quantized
codes (their bit-exact parity with the HIP quantizers is tested separately)."""
import numpy as np
import pytest
import torch

from conftest import print_case
from gpu_util import assert_canary, dev, host, poisoned
from kv_quantization_amd import _lib, api, synth

pytestmark = pytest.mark.gpu
RTOL = 1e-3


@pytest.fixture(autouse=True, scope="module")
def _bind_oracle(oracle_mod):
    global _oracle
    _oracle = oracle_mod


def _weights(kind, ws):
    segs = [_oracle.weight_quant(kind, w) for w in ws]
    return segs, api.W8a8Weight(kind, [(dev(q), dev(s)) for q, s in segs])


def _half_ulp_bf16(v):
    """Half a bf16 ulp at |v| (8 significant bits): the rounding any bf16 output carries."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 8)


def _check(out_bf16, ref, bound, what, strict=False):
    """|gpu - ref| <= 1e-3 * sum|a||w| + half a bf16 ulp of the result (the output
    format's own rounding).  strict: also without the bf16 allowance, which holds
    at the workload shapes (large K, |y| << sum|a||w|)."""
    got = _oracle.bf16_to_f32(out_bf16).astype(np.float64)
    err = np.abs(got - ref)
    ratio = err / np.maximum(bound, 1e-300)
    worst = float(ratio.max())
    print(f"{what}: max |err|/sum|a||w| = {worst:.3e}", flush=True)
    over = err > RTOL * bound + _half_ulp_bf16(ref)
    assert not over.any(), f"{what}: {int(over.sum())} outputs beyond tolerance, worst ratio {worst:.3e}"
    if strict:
        assert worst <= RTOL, f"{what}: {int((ratio > RTOL).sum())} outputs beyond 1e-3, worst {worst:.3e}"


def _expect_invalid(call, text):
    with pytest.raises(_lib.KvqError) as e:
        call()
    assert e.value.status == _lib.KVQ_E_INVALID and text in str(e.value), str(e.value)


def _case(kind, x_bf16, k, ws, rows, silu=False, up=None, ldc_pad=0, what="", strict=False):
    segs, weight = _weights(kind, ws)
    q, sa = _oracle.act_quant(kind, x_bf16[:rows], k, silu=silu, up_bf16=None if up is None else up[:rows])
    ref, bound = _oracle.w8a8_gemv(kind, q, sa, segs)
    n = ref.shape[1]
    ldc = n + ldc_pad
    out, raw = poisoned((rows, ldc), torch.bfloat16)
    api.gemv(dev(q), dev(sa), weight, out=out, ldc=ldc)
    torch.cuda.synchronize()
    o = host(out)
    _check(o[:, :n], ref, bound, what, strict)
    if ldc_pad:
        assert np.all(o[:, n:].view(np.uint8) == 0xAA), "columns past N were written"
    assert_canary(raw, rows * ldc * 2)
    return o[:, :n]


@pytest.mark.parametrize("m", [1, 8, 32])
def test_rowscale_fused_qkv(m):
    print_case("w8a8 rowscale qkv", m)
    inp = synth.w8a8_qkv()
    _case(0, inp.x_bf16, 4096, inp.weights, m, what=f"qkv M={m}", strict=True)


_down = {}


def _down_inputs():
    if not _down:
        inp = synth.w8a8_down()
        segs, weight = _weights(1, inp.weights)
        _down.update(inp=inp, segs=segs, weight=weight)
    return _down


@pytest.mark.parametrize("m", [64, 128, 256])
def test_blk128_down_proj(m):
    print_case("w8a8 blk128 down", m)
    d = _down_inputs()
    q, sa = _oracle.act_quant(1, d["inp"].x_bf16[:m], 14336, silu=True)
    ref, bound = _oracle.w8a8_gemv(1, q, sa, d["segs"])
    out = api.gemv(dev(q), dev(sa), d["weight"])
    torch.cuda.synchronize()
    _check(host(out), ref, bound, f"down M={m}", strict=True)


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("rows", [1, 3, 4, 5, 8, 16, 17, 32, 33, 63, 64, 65, 100, 255, 256])
def test_row_counts(kind, rows):
    print_case("w8a8 rows", kind, rows)
    seg_n = (48, 32, 21) if kind == 0 else (128, 256, 77)
    inp = synth.w8a8(256, 384, seg_n, seed=300 + rows)
    _case(kind, inp.x_bf16, 384, inp.weights, rows, ldc_pad=8, what=f"kind={kind} rows={rows}")


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("seg_n,k", [((1,), 128), ((7,), 256), ((16, 1), 128), ((128,), 128), ((64, 64, 64), 512),
                                     ((2048,), 1024)])
def test_segment_shapes(kind, seg_n, k):
    print_case("w8a8 segments", kind, seg_n, k)
    inp = synth.w8a8(70, k, seg_n, seed=400 + k + sum(seg_n))
    if kind == 1 and any(n % 128 for n in seg_n[:-1]):
        # block scales cover 128 weight rows: a non-last segment that is not a
        # multiple of 128 rows is refused on the host, before any launch
        _expect_invalid(lambda: _case(kind, inp.x_bf16, k, inp.weights, 9), "not a multiple of 128")
        return
    for rows in (1, 9, 70):
        _case(kind, inp.x_bf16, k, inp.weights, rows, what=f"kind={kind} segs={seg_n} rows={rows}")


def test_segment_invariance_rowscale():
    """Three segments give the same bits as one concatenated segment."""
    print_case("w8a8 segment invariance")
    inp = synth.w8a8(8, 512, (256, 128, 64), seed=500)
    q, sa = _oracle.act_quant(0, inp.x_bf16, 512)
    segs3, w3 = _weights(0, inp.weights)
    w1 = api.W8a8Weight(0, [(dev(np.concatenate([s[0] for s in segs3])), dev(np.concatenate([s[1] for s in segs3])))])
    a = host(api.gemv(dev(q), dev(sa), w3))
    b = host(api.gemv(dev(q), dev(sa), w1))
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("kind,silu,with_up", [(0, False, False), (1, True, False), (1, True, True), (0, True, True)])
def test_proj_equals_act_quant_then_gemv(kind, silu, with_up):
    print_case("w8a8 proj", kind, silu, with_up)
    inp = synth.w8a8(40, 1024, (256, 128), seed=600, with_up=with_up)
    _, weight = _weights(kind, inp.weights)
    x = dev(inp.x_bf16)
    up = None if inp.up_bf16 is None else dev(inp.up_bf16)
    q, sa = api.act_quant(x, 1024, kind, silu, up)
    a = host(api.gemv(q, sa, weight))
    b = host(api.proj(x, weight, silu=silu, up=up))
    np.testing.assert_array_equal(a, b)
    # and the proj output against the oracle chain
    qo, so = _oracle.act_quant(kind, inp.x_bf16, 1024, silu=silu, up_bf16=inp.up_bf16)
    np.testing.assert_array_equal(host(q), qo)
    ref, bound = _oracle.w8a8_gemv(kind, qo, so, [_oracle.weight_quant(kind, w) for w in inp.weights])
    _check(b, ref, bound, "proj")


def test_shared_workspace_across_calls():
    """One workspace serves split-K calls of every kind in turn: the counters
    each call leaves at zero sit in a fixed area that no partial sum reaches."""
    print_case("w8a8 shared workspace")
    a = synth.w8a8(70, 512, (48, 32, 21), seed=601)     # N % 4 != 0: separate reduction kernel
    b = synth.w8a8(70, 512, (64, 64, 64), seed=602)     # N % 4 == 0: sums inside the GEMM
    x4, projs = synth.int4_awq(64, 1024, (256, 64, 64), 128, seed=603)
    for _ in range(2):
        for inp, what in ((a, "reduce kernel"), (b, "in-GEMM sums")):
            _case(0, inp.x_bf16, 512, inp.weights, 70, what=f"shared workspace, {what}")
        outs = api.int4_awq_qkv(dev(x4), [(dev(p.qweight.view(np.int32)), dev(p.scales), dev(p.zeros)) for p in projs],
                                128)
        torch.cuda.synchronize()
        refs = _oracle.int4_awq_qkv(x4, [(p.qweight, p.scales, p.zeros) for p in projs], 128)
        for o, (r, bnd) in zip(outs, refs):
            assert np.all(np.abs(host(o).astype(np.float64) - r) <= 1e-3 * bnd), "int4 with shared workspace"


# w8a8_proj with <= 8 rows is one launch (the GEMV quantizes its activations);
# its output must equal act_quant + gemv bit for bit, its scratch must hold the
# oracle's codes and scales, and the output must meet the oracle's bound.
@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("silu,with_up", [(False, False), (True, False), (True, True)])
@pytest.mark.parametrize("rows,k,seg_n", [(1, 128, (16,)), (3, 384, (48, 32, 21)), (4, 1152, (256, 128, 77)),
                                          (5, 4096, (128, 256)), (8, 4096, (1024, 256, 100)),
                                          (2, 4736, (256, 31)), (8, 14336, (256,)), (6, 8192, (128, 128))])
def test_proj_single_launch(kind, silu, with_up, rows, k, seg_n):
    print_case("w8a8 proj fused", kind, silu, with_up, rows, k, seg_n)
    inp = synth.w8a8(rows, k + 8, seg_n, seed=700 + rows + k, with_up=with_up)
    xb = inp.x_bf16.copy()
    if rows >= 3:
        xb[1] = 0                                   # zero row: floor scale
    segs = [_oracle.weight_quant(kind, w[:, :k].copy()) for w in inp.weights]
    weight = api.W8a8Weight(kind, [(dev(q), dev(s)) for q, s in segs])
    x = dev(xb)                                     # ldx = k + 8
    up = None if inp.up_bf16 is None else dev(inp.up_bf16)
    if kind == 1 and any(n % 128 for n in seg_n[:-1]):
        # refused on the host (block scales cover 128 weight rows), nothing launched
        _expect_invalid(lambda: api.proj(x, weight, silu=silu, up=up), "not a multiple of 128")
        return
    sshape = (rows,) if kind == 0 else (rows, k // 128)
    q, raw_q = poisoned((rows, k), torch.uint8)
    sa, raw_s = poisoned(sshape, torch.float32)
    b = host(api.proj(x, weight, silu=silu, up=up, scratch=(q, sa)))
    q2, sa2 = api.act_quant(x, k, kind, silu, up)
    a = host(api.gemv(q2, sa2, weight))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.view(np.uint16), b.view(np.uint16))
    qo, so = _oracle.act_quant(kind, xb, k, silu=silu, up_bf16=inp.up_bf16)
    np.testing.assert_array_equal(host(q), qo)
    np.testing.assert_array_equal(host(sa).view(np.uint32), so.view(np.uint32))
    assert_canary(raw_q, rows * k)
    assert_canary(raw_s, int(np.prod(sshape)) * 4)
    ref, bound = _oracle.w8a8_gemv(kind, qo, so, segs)
    _check(b, ref, bound, "proj fused")


@pytest.mark.parametrize("m", [1, 4, 8])
def test_proj_single_launch_qkv_shape(m):
    print_case("w8a8 proj fused qkv", m)
    inp = synth.w8a8_qkv()
    segs, weight = _weights(0, inp.weights)
    x = dev(inp.x_bf16[:m])
    b = host(api.proj(x, weight))
    qo, so = _oracle.act_quant(0, inp.x_bf16[:m], 4096)
    ref, bound = _oracle.w8a8_gemv(0, qo, so, segs)
    _check(b, ref, bound, f"proj qkv M={m}", strict=True)
