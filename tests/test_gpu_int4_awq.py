"""GPU parity: INT4 AWQ fused Q/K/V GEMV/GEMM vs the oracle's fp64 definition,
|gpu - ref| <= 1e-3 * sum|x||w| per output, through the C ABI."""
import numpy as np
import pytest
import torch

from conftest import print_case
from gpu_util import assert_canary, dev, host, poisoned
from kv_quantization_amd import api, synth

pytestmark = pytest.mark.gpu
RTOL = 1e-3


@pytest.fixture(autouse=True, scope="module")
def _bind_oracle(oracle_mod):
    global _oracle
    _oracle = oracle_mod


def _run(x, projs, gs, use_workspace=True):
    m = x.shape[0]
    outs, raws = [], []
    for p in projs:
        n = p.qweight.shape[1] * 8
        o, raw = poisoned((m, n), torch.float32)
        outs.append(o)
        raws.append((raw, m * n * 4))
    api.int4_awq_qkv(dev(x), [(dev(p.qweight), dev(p.scales), dev(p.zeros)) for p in projs], gs, outs=outs,
                     use_workspace=use_workspace)
    torch.cuda.synchronize()
    for raw, nb in raws:
        assert_canary(raw, nb)
    return [host(o) for o in outs]


def _check(x, projs, gs, got, what):
    refs = _oracle.int4_awq_qkv(x, [(p.qweight, p.scales, p.zeros) for p in projs], gs)
    worst = 0.0
    for (ref, bound), g in zip(refs, got):
        ratio = np.abs(g.astype(np.float64) - ref) / np.maximum(bound, 1e-300)
        worst = max(worst, float(ratio.max()))
    print(f"{what}: max |err|/sum|x||w| = {worst:.3e}", flush=True)
    assert worst <= RTOL, what


def test_single_projection_512():
    print_case("int4 single 512")
    x, projs = synth.int4_gemv_512()
    _check(x, projs, 128, _run(x, projs, 128), "C1")


@pytest.mark.parametrize("m", [1, 16, 128])
def test_fused_qkv_8b(m):
    print_case("int4 qkv 8b", m)
    x, projs = synth.int4_qkv()
    _check(x[:m], projs, 128, _run(x[:m], projs, 128), f"qkv M={m}")


@pytest.mark.parametrize("m", [1, 2, 5, 16, 17, 31, 32, 33, 64, 100, 256])
@pytest.mark.parametrize("gs", [32, 64, 128, 256])
def test_shapes(m, gs):
    print_case("int4 shapes", m, gs)
    k = 512
    x, projs = synth.int4_awq(m, k, (136, 24, 24), gs, seed=700 + m + gs)
    _check(x, projs, gs, _run(x, projs, gs), f"m={m} gs={gs}")


@pytest.mark.parametrize("m", [33, 64, 100, 129, 256])
@pytest.mark.parametrize("gs", [32, 64, 128, 256])
def test_shapes_wide_m(m, gs):
    # m > 32 (several row chunks per column tile), a partial last column tile
    # (n = 96) and several K slices, with and without the workspace
    print_case("int4 wide-m shapes", m, gs)
    k = 1024
    x, projs = synth.int4_awq(m, k, (256, 96, 96), gs, seed=1700 + m + gs)
    _check(x, projs, gs, _run(x, projs, gs), f"m={m} gs={gs}")
    _check(x, projs, gs, _run(x, projs, gs, use_workspace=False), f"nows m={m} gs={gs}")


@pytest.mark.parametrize("m", [1, 16, 40])
def test_without_workspace_same_bits_order_independent(m):
    print_case("int4 workspace vs none", m)
    x, projs = synth.int4_awq(m, 2048, (1024, 256, 256), 128, seed=800 + m)
    a = _run(x, projs, 128, use_workspace=True)
    b = _run(x, projs, 128, use_workspace=False)
    _check(x, projs, 128, a, f"ws m={m}")
    _check(x, projs, 128, b, f"nows m={m}")
    # repeated calls reuse the workspace (left zero-filled): same bits again
    c = _run(x, projs, 128, use_workspace=True)
    for u, v in zip(a, c):
        np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("m,k,ns", [(33, 2048, (8192, 1024, 1024)), (128, 4096, (4096, 1024, 1024)),
                                    (256, 1024, (2048, 512, 512))])
def test_no_k_split_workspace_holds_the_scaled_copy(m, k, ns):
    """These shapes have more than 128 (tile, row chunk) units, so no call
    splits K across workgroups: the workspace holds the counter area (left
    zero), the per-row power-of-two scaled fp16 copy of the activations and
    the row scales.  Without a workspace the product kernel rounds the
    activations itself, unscaled; both pass."""
    print_case("int4 no split-K", m, k)
    x, projs = synth.int4_awq(m, k, ns, 128, seed=1900 + m)
    r256 = lambda b: (b + 255) // 256 * 256
    assert api.int4_workspace_bytes(m, k, 128, sum(ns)) == 4096 + r256(m * k * 2) + r256(m * 4)
    _check(x, projs, 128, _run(x, projs, 128, use_workspace=True), f"scaled copy m={m}")
    _check(x, projs, 128, _run(x, projs, 128, use_workspace=False), f"in-kernel rounding m={m}")


@pytest.mark.parametrize("m,k,ns,gs", [
    (64, 4096, (512,), 128),              # 4 tiles x 2 row chunks: K slices over the waves and workgroups
    (100, 2048, (1152, 128, 128), 64),    # 11 tiles (a pair across projections), 4 ragged row chunks
    (300, 1024, (512, 256, 256), 32),     # 10 row chunks, 32-row groups
    (129, 1536, (2048, 512, 512), 256),   # 5 row chunks (the last one row), 6 groups
    (64, 512, (16384,), 128),             # 128 tiles
    (96, 1088, (256, 64, 64), 32),        # 34 groups of 32 (odd)
    (80, 544, (256, 64, 64), 32),         # 17 groups of 32
])
def test_matrix_core_more_shapes(m, k, ns, gs):
    """The matrix-core ring on ragged shapes: parity with and without a
    workspace, the same bits on a second call, and fp16 / bf16 activations
    bit-identical to the fp32 call on their values."""
    print_case("int4 matrix-core shapes", m, k, ns, gs)
    x, projs = synth.int4_awq(m, k, ns, gs, seed=3100 + m + gs)
    a = _run(x, projs, gs)
    _check(x, projs, gs, a, f"m={m} k={k} gs={gs}")
    for u, v in zip(a, _run(x, projs, gs)):
        np.testing.assert_array_equal(u.view(np.uint32), v.view(np.uint32))
    _check(x, projs, gs, _run(x, projs, gs, use_workspace=False), f"nows m={m} k={k} gs={gs}")
    for dt in (1, 2):
        xb = _oracle.narrow16(x, dt)
        xw = _oracle.widen16(xb, dt)
        got16 = _run16(xb, dt, projs, gs)
        _check(xw, projs, gs, got16, f"dt={dt} m={m}")
        for u, v in zip(got16, _run(xw, projs, gs)):
            np.testing.assert_array_equal(u.view(np.uint32), v.view(np.uint32))


@pytest.mark.parametrize("m", [16, 40, 128])
@pytest.mark.parametrize("kind", ["tiny", "huge", "mixed"])
def test_matrix_core_activation_range(m, kind):
    """From 16 rows the activations reach the matrix cores as fp16, each row
    scaled by a power of two that puts its absmax in [2^14, 2^15): rows of
    1e-6 keep 11 bits per term and rows of 1e5 (past fp16's 65504) do not
    overflow.  Mixed: rows alternate 1e-6, 1e5, exact zeros and N(0, 1)."""
    print_case("int4 matrix-core activation range", m, kind)
    x, projs = synth.int4_awq(m, 1024, (256, 64, 64), 128, seed=2400 + m)
    if kind == "tiny":
        x = (x * 1e-6).astype(np.float32)
    elif kind == "huge":
        x = (x * 1e5).astype(np.float32)
    else:
        f = np.array([1e-6, 1e5, 0.0, 1.0], dtype=np.float64)[np.arange(m) % 4]
        x = (x * f[:, None]).astype(np.float32)
    _check(x, projs, 128, _run(x, projs, 128), f"{kind} m={m}")


def test_large_call_then_split_k_calls():
    """A call without K split (128 rows) followed, on the same workspace, by
    calls that count K slices through the counter area (1, 5 and 16 rows):
    every counter is back at zero after each call."""
    print_case("int4 large call then split-K")
    x5, projs = _qkv_inputs()
    _check(x5[:128], projs, 128, _run(x5[:128], projs, 128), "qkv M=128")
    for m in (1, 5, 16):
        x, small = synth.int4_awq(m, 512, (136, 24, 24), 32, seed=2000 + m)
        _check(x, small, 32, _run(x, small, 32), f"after the large call m={m}")
        _check(x, small, 32, _run(x, small, 32), f"again m={m}")


def test_single_is_q_part_of_fused():
    print_case("int4 single vs fused")
    x, projs = synth.int4_awq(3, 256, (64, 16, 16), 128, seed=900)
    fused = _run(x, projs, 128)
    single = _run(x, projs[:1], 128)
    np.testing.assert_array_equal(fused[0], single[0])


def test_degenerate_scales_zeros():
    print_case("int4 degenerate")
    rng = np.random.default_rng(901)
    x, projs = synth.int4_awq(4, 256, (64,), 64, seed=902)
    p = projs[0]
    codes = _oracle.awq_unpack(p.qweight, 64)
    # zero == code within each group -> exactly zero output
    z = codes.reshape(4, 64, 64)[:, 0, :].astype(np.float32)
    codes[:] = np.repeat(z.astype(np.uint8), 64, axis=0)
    p.qweight = _oracle.awq_pack(codes)
    p.zeros = z
    got = _run(x, [p], 64)
    # The kernel sums s * (P - z*X) with P = sum x~ q and X = sum x~ in fp32, so
    # a cancellation leaves a residual bounded by a few ulps of
    # s * (sum |x~| q + |z| sum |x~|) per group (not by sum |x||w|, which is 0).
    xa = np.abs(x.astype(np.float16).astype(np.float64))
    per_group = [(xa[:, g * 64:(g + 1) * 64] @ codes[g * 64:(g + 1) * 64].astype(np.float64)
                  + xa[:, g * 64:(g + 1) * 64].sum(axis=1, keepdims=True) * np.abs(z[g]))
                 * p.scales[g].astype(np.float64) for g in range(4)]
    cancel_bound = 2.0 ** -24 * 70 * np.sum(per_group, axis=0)
    assert np.all(np.abs(got[0]) <= cancel_bound)
    # unit scales, zero offsets, small-integer x: exact integer results
    xi = rng.integers(-8, 8, (4, 256)).astype(np.float32)
    p.scales = np.ones_like(p.scales)
    p.zeros = np.zeros_like(p.zeros)
    got = _run(xi, [p], 64)
    np.testing.assert_array_equal(got[0], (xi.astype(np.int64) @ codes.astype(np.int64)).astype(np.float32))


# ------------------------------------------- M = 2..15 and 16-bit activations --

_qkv = {}


def _qkv_inputs():
    if not _qkv:
        x5, projs = synth.int4_qkv(seed=5)
        _qkv.update(x=x5, projs=projs)
    return _qkv["x"], _qkv["projs"]


@pytest.mark.parametrize("m", [2, 3, 4, 7, 8, 12, 15])
def test_fused_qkv_small_m(m):
    """The fused QKV workload between the M=1 and M=16 configurations."""
    print_case("int4 qkv small m", m)
    x5, projs = _qkv_inputs()
    x = x5[:m]
    _check(x, projs, 128, _run(x, projs, 128), f"qkv M={m}")


def _run16(x16_bits, dt, projs, gs):
    tdt = {1: torch.float16, 2: torch.bfloat16}[dt]
    xd = torch.from_numpy(np.ascontiguousarray(x16_bits).view(np.int16)).cuda().view(tdt)
    outs = api.int4_awq_qkv(xd, [(dev(p.qweight), dev(p.scales), dev(p.zeros)) for p in projs], gs)
    torch.cuda.synchronize()
    return [host(o) for o in outs]


@pytest.mark.parametrize("dt", [1, 2])
@pytest.mark.parametrize("m", [1, 5, 16, 40, 128])
def test_16bit_activations(dt, m):
    """fp16/bf16 x: within the bound of the oracle on the exact (widened)
    values, and bit-identical to the fp32 call on those values (both reach
    the matrix cores as the same fp16 operands)."""
    print_case("int4 16-bit x", dt, m)
    x5, projs = _qkv_inputs()
    xb = _oracle.narrow16(x5[:m], dt)
    xw = _oracle.widen16(xb, dt)
    got16 = _run16(xb, dt, projs, 128)
    _check(xw, projs, 128, got16, f"qkv M={m} dt={dt}")
    got32 = _run(xw, projs, 128)
    for a, b in zip(got16, got32):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------ fp32 GEMV below 16 rows --
# Below 16 rows the products are fp32 on the vector ALUs (the page's
# arithmetic): no rounding of x, so the error against the fp64 definition is
# fp32 summation error only, far under the 1e-3 contract.  FP32_RTOL pins
# that: fp16 activations alone would exceed it (2^-11 per term).
FP32_RTOL = 2e-5


def _ratio(x, projs, gs, got):
    refs = _oracle.int4_awq_qkv(x, [(p.qweight, p.scales, p.zeros) for p in projs], gs)
    worst = 0.0
    for (ref, bound), g in zip(refs, got):
        worst = max(worst, float((np.abs(g.astype(np.float64) - ref) / np.maximum(bound, 1e-300)).max()))
    return worst


@pytest.mark.parametrize("gs", [32, 64, 128, 256])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 9, 13, 15])
def test_gemv_fp32_rows_below_16(m, gs):
    # n = 512 / 96 / 96: 32-column lanes (96 % 32 == 0), partial 256-column
    # tiles; K = 2048 splits each tile's groups over several workgroups
    print_case("int4 gemv fp32", m, gs)
    x, projs = synth.int4_awq(m, 2048, (512, 96, 96), gs, seed=3000 + 16 * m + gs)
    got = _run(x, projs, gs)
    worst = _ratio(x, projs, gs, got)
    print(f"gemv m={m} gs={gs}: max |err|/sum|x||w| = {worst:.3e}", flush=True)
    assert worst <= FP32_RTOL
    nows = _run(x, projs, gs, use_workspace=False)
    assert _ratio(x, projs, gs, nows) <= FP32_RTOL


@pytest.mark.parametrize("m", [1, 4, 8, 15])
def test_gemv_fp32_qkv_workload(m):
    print_case("int4 gemv fp32 qkv", m)
    x5, projs = _qkv_inputs()
    worst = _ratio(x5[:m], projs, 128, _run(x5[:m], projs, 128))
    print(f"qkv M={m}: max |err|/sum|x||w| = {worst:.3e}", flush=True)
    assert worst <= FP32_RTOL


@pytest.mark.parametrize("sigma", [1e-6, 1e5])
@pytest.mark.parametrize("m", [1, 4, 15])
def test_gemv_fp32_activation_range(m, sigma):
    """Activations far outside fp16's range (tiny: 1e-6, subnormal in fp16;
    large: |x| ~ 1e5, past fp16's 65504) stay within the fp32 bound."""
    print_case("int4 gemv range", m, sigma)
    x, projs = synth.int4_awq(m, 1024, (256, 64, 64), 128, seed=3100 + m)
    xs = (x * np.float32(sigma)).astype(np.float32)
    worst = _ratio(xs, projs, 128, _run(xs, projs, 128))
    print(f"range m={m} sigma={sigma}: max |err|/sum|x||w| = {worst:.3e}", flush=True)
    assert worst <= FP32_RTOL


def test_gemv_single_projection_fp32():
    # the 512 x 512 single projection at M=1 runs the fp32 path too
    print_case("int4 gemv single 512")
    x, projs = synth.int4_gemv_512()
    worst = _ratio(x, projs, 128, _run(x, projs, 128))
    assert worst <= FP32_RTOL
