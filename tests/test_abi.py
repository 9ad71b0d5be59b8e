"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects every contract violation on the host before any
HIP call (so these run without a GPU)."""
import ctypes
import re
from pathlib import Path

import pytest

from kv_quantization_amd import _lib

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "kvq.h"

# Every call below breaks the contract, so it returns before any HIP call and
# the fake addresses are never used on a device.
FAKE = 0x10000          # 16-byte aligned, never dereferenced: validation fails first
MISALIGNED = 0x10004


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_parses_and_library_exports_every_symbol(lib):
    names = declared_functions()
    assert len(names) >= 17, names
    for n in names:
        assert hasattr(lib, n), f"libkvq.so does not export {n}"
    assert set(names) == set(_lib.SIGNATURES) | {"kvq_last_error", "kvq_abi_version"}
    assert lib.kvq_abi_version() == 100


def _err(lib, name, *args):
    st = getattr(lib, name)(*args)
    return st, lib.kvq_last_error().decode()


@pytest.mark.parametrize("args,frag", [
    ((0, FAKE, FAKE, 4, 8, None), "null"),
    ((MISALIGNED, FAKE, FAKE, 4, 8, None), "aligned"),
    ((FAKE, FAKE, FAKE, 0, 8, None), "num_tokens=0"),
    ((FAKE, FAKE, FAKE, 4, 0, None), "head_dim=0"),
])
def test_kv_int8_validation(lib, args, frag):
    for fn in ("kvq_quant_int8_token", "kvq_dequant_int8_token", "kvq_quant_fp8_token", "kvq_dequant_fp8_token"):
        st, msg = _err(lib, fn, *args)
        assert st == _lib.KVQ_E_INVALID and frag in msg, (fn, msg)


# Only invalid argument sets here: a valid one would launch on fake pointers.
@pytest.mark.parametrize("t,d,gs", [(4, 8, 3), (4, 8, 0), (3, 5, 4), (3, 6, 4), (1, 1, 2)])
def test_kv_int4_group_validation(lib, t, d, gs):
    st, msg = _err(lib, "kvq_quant_int4_group", FAKE, FAKE, FAKE, FAKE, t, d, gs, None)
    assert st == _lib.KVQ_E_INVALID and "group_size" in msg


def test_kv_int4_null_and_alignment(lib):
    assert _err(lib, "kvq_dequant_int4_group", FAKE, FAKE, 0, FAKE, 4, 8, 4, None)[0] == _lib.KVQ_E_INVALID
    assert _err(lib, "kvq_dequant_int4_group", FAKE, FAKE, MISALIGNED, FAKE, 4, 8, 4, None)[0] == _lib.KVQ_E_INVALID


@pytest.mark.parametrize("kind,silu,up,ldx,rows,k,frag", [
    (0, 0, 0, 128, 0, 128, "rows"),
    (0, 0, 0, 128, 257, 128, "rows"),
    (1, 0, 0, 256, 4, 200, "K=200"),
    (0, 0, 0, 120, 4, 128, "ldx=120"),
    (0, 0, 0, 132, 4, 128, "ldx=132"),
    (0, 0, FAKE, 128, 4, 128, "up is only used with silu"),
    (2, 0, 0, 128, 4, 128, "scale kind"),
])
def test_act_quant_validation(lib, kind, silu, up, ldx, rows, k, frag):
    st, msg = _err(lib, "w8a8_act_quant", kind, silu, FAKE, up or None, ldx, rows, k, FAKE, FAKE, None)
    assert st == _lib.KVQ_E_INVALID and frag in msg, msg


def test_scratch_bytes_follow_the_scratch_rule(lib):
    qb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.w8a8_scratch_bytes(0, 256, 4096, ctypes.byref(qb), ctypes.byref(sb)) == 0
    assert (qb.value, sb.value) == (256 * 4096, 256 * 4)
    assert lib.w8a8_scratch_bytes(1, 64, 14336, ctypes.byref(qb), ctypes.byref(sb)) == 0
    assert (qb.value, sb.value) == (64 * 14336, 64 * 112 * 4)


def test_weight_quant_and_cast_validation(lib):
    assert _err(lib, "w8a8_weight_quant", 0, FAKE, 16, 100, FAKE, FAKE, None)[0] == _lib.KVQ_E_INVALID
    assert _err(lib, "w8a8_weight_quant", 1, FAKE, 0, 128, FAKE, FAKE, None)[0] == _lib.KVQ_E_INVALID
    assert _err(lib, "kvq_f32_to_e4m3", FAKE, FAKE, 0, None)[0] == _lib.KVQ_E_INVALID
    assert _err(lib, "kvq_f32_to_e4m3", MISALIGNED, FAKE, 8, None)[0] == _lib.KVQ_E_INVALID


def _segs(*specs):
    arr = (_lib.W8a8Segment * 3)()
    for i, (w, s, n) in enumerate(specs):
        arr[i].w, arr[i].scale, arr[i].n = w, s, n
    return arr


@pytest.mark.parametrize("kind,rows,k,specs,nseg,ldc,frag", [
    (0, 0, 128, [(FAKE, FAKE, 16)], 1, 16, "rows"),
    (0, 257, 128, [(FAKE, FAKE, 16)], 1, 16, "rows"),
    (0, 4, 100, [(FAKE, FAKE, 16)], 1, 16, "K=100"),
    (0, 4, 128, [(FAKE, FAKE, 16)], 0, 16, "segments"),
    (0, 4, 128, [(FAKE, FAKE, 16)] * 3, 4, 64, "segments"),
    (0, 4, 128, [(FAKE, FAKE, 0)], 1, 16, "empty"),
    (0, 4, 128, [(0, FAKE, 16)], 1, 16, "empty"),
    (0, 4, 128, [(FAKE, FAKE, 24), (FAKE, FAKE, 16)], 2, 64, "not a multiple of 16"),
    (1, 4, 128, [(FAKE, FAKE, 64), (FAKE, FAKE, 128)], 2, 256, "not a multiple of 128"),
    (0, 4, 128, [(FAKE, FAKE, 32), (FAKE, FAKE, 16)], 2, 40, "ldc=40"),
    (0, 4, 128, [(MISALIGNED, FAKE, 16)], 1, 16, "aligned"),
])
def test_gemv_validation(lib, kind, rows, k, specs, nseg, ldc, frag):
    st, msg = _err(lib, "w8a8_gemv", kind, FAKE, FAKE, rows, k, _segs(*specs), nseg, FAKE, ldc, None, 0, None)
    assert st == _lib.KVQ_E_INVALID and frag in msg, msg


def _proj(qw=FAKE, s=FAKE, z=FAKE, o=FAKE, n=64):
    p = _lib.Int4AwqProj()
    p.qweight, p.scales, p.zeros, p.out, p.n = qw, s, z, o, n
    return p


@pytest.mark.parametrize("m,k,gs,q,kv,frag", [
    (0, 256, 128, _proj(), None, "m == 0"),
    (1, 256, 96, _proj(), None, "group_size"),
    (1, 200, 128, _proj(), None, "K=200"),
    (1, 256, 128, _proj(n=60), None, "n=60"),
    (1, 256, 128, _proj(qw=0), None, "null"),
    (1, 256, 128, _proj(o=MISALIGNED), None, "aligned"),
    (1, 256, 128, _proj(), (_proj(n=32), _proj(n=64)), "differ"),
    (1, 256, 128, _proj(), (_proj(), None), "both"),
])
def test_int4_validation(lib, m, k, gs, q, kv, frag):
    kp = ctypes.byref(kv[0]) if kv and kv[0] is not None else None
    vp = ctypes.byref(kv[1]) if kv and kv[1] is not None else None
    st, msg = _err(lib, "int4_awq_qkv_gemm", FAKE, m, k, gs, ctypes.byref(q), kp, vp, None, 0, None)
    assert st == _lib.KVQ_E_INVALID and frag in msg, msg


def test_workspace_sizes(lib):
    b = ctypes.c_size_t()
    assert lib.int4_awq_workspace_bytes(1, 4096, 128, 6144, ctypes.byref(b)) == 0
    assert b.value > 0          # small M slices K across workgroups
    assert lib.int4_awq_workspace_bytes(1, 512, 128, 512, ctypes.byref(b)) == 0
    assert b.value == 0         # tiny problem: one workgroup per tile
    # 16 rows and more (matrix cores): the counter area and partial tiles
    # when K is split (up to two extra tiles for any split of n into three
    # projections); when a wave's K range does not fit its ring, also the
    # per-row power-of-two scaled fp16 copy of the activations and the row
    # scales, each rounded up to 256 bytes
    counters = 4096
    r256 = lambda v: (v + 255) // 256 * 256
    # 16 rows x 6144 columns: 5 K slices (4, then one more while 48-50 tiles
    # x 5 stay within 256 workgroups) of 16 x 128 fp32 tiles; at most one
    # group per wave, scaled inside the wave
    assert lib.int4_awq_workspace_bytes(16, 4096, 128, 6144, ctypes.byref(b)) == 0
    assert b.value == counters + (6144 // 128 + 2) * 5 * 16 * 128 * 4
    # 128 rows x 6144 columns: K is not split, 4 groups per wave: the copy
    assert lib.int4_awq_workspace_bytes(128, 4096, 128, 6144, ctypes.byref(b)) == 0
    assert b.value == counters + 128 * 4096 * 2 + 512
    assert lib.int4_awq_workspace_bytes(17, 96, 32, 8, ctypes.byref(b)) == 0
    assert b.value == 0         # one tile, 3 groups of 32: fits the rings, no split
    assert lib.int4_awq_workspace_bytes(16, 96, 32, 8, ctypes.byref(b)) == 0
    assert b.value == 0
    assert lib.w8a8_gemv_workspace_bytes(0, 8, 4096, 6144, ctypes.byref(b)) == 0


@pytest.mark.parametrize("args,frag", [
    ((0, FAKE, FAKE, 4, 8), "null"),
    ((MISALIGNED, FAKE, FAKE, 4, 8), "aligned"),
    ((FAKE, FAKE, FAKE, 0, 8), "num_tokens=0"),
    ((FAKE, FAKE, FAKE, 4, 0), "head_dim=0"),
])
def test_kv_int8_tensor_validation(lib, args, frag):
    st, msg = _err(lib, "kvq_quant_int8_tensor", *args, FAKE, 1 << 20, None)
    assert st == _lib.KVQ_E_INVALID and frag in msg, msg
    st, msg = _err(lib, "kvq_dequant_int8_tensor", *args, None)
    assert st == _lib.KVQ_E_INVALID and frag in msg, msg


def test_kv_int8_tensor_workspace_rules(lib):
    need = _lib.INT8_TENSOR_WORKSPACE_BYTES
    text = HEADER.read_text()
    counter = int(re.search(r"#define KVQ_WORKSPACE_COUNTER_BYTES (\d+)u", text).group(1))
    extra = int(re.search(r"#define KVQ_INT8_TENSOR_WORKSPACE_BYTES \(KVQ_WORKSPACE_COUNTER_BYTES \+ (\d+)u\)",
                          text).group(1))
    assert need == counter + extra
    for ws, nbytes in ((None, need), (FAKE, need - 1), (MISALIGNED, need)):
        st, msg = _err(lib, "kvq_quant_int8_tensor", FAKE, FAKE, FAKE, 4, 8, ws, nbytes, None)
        assert st == _lib.KVQ_E_INVALID and "workspace" in msg, msg


@pytest.mark.parametrize("dt", [3, -1])
def test_kv_dtype_validation(lib, dt):
    for fn, args in (("kvq_quant_int8_token_dt", (FAKE, dt, FAKE, FAKE, 4, 8, None)),
                     ("kvq_dequant_int8_token_dt", (FAKE, FAKE, FAKE, dt, 4, 8, None)),
                     ("kvq_quant_int4_group_dt", (FAKE, dt, FAKE, FAKE, FAKE, 4, 8, 4, None)),
                     ("kvq_dequant_int4_group_dt", (FAKE, FAKE, FAKE, FAKE, dt, 4, 8, 4, None))):
        st, msg = _err(lib, fn, *args)
        assert st == _lib.KVQ_E_INVALID and "dtype" in msg, (fn, msg)


def test_kv_dtype_calls_share_the_fp32_checks(lib):
    st, msg = _err(lib, "kvq_quant_int8_token_dt", FAKE, 1, FAKE, FAKE, 0, 8, None)
    assert st == _lib.KVQ_E_INVALID and "num_tokens=0" in msg
    st, msg = _err(lib, "kvq_quant_int4_group_dt", FAKE, 2, FAKE, FAKE, FAKE, 4, 8, 3, None)
    assert st == _lib.KVQ_E_INVALID and "group_size" in msg


# decode attention: q, Hq, Hkv, T, D, k codes, k scales, v codes, v scales, scale, out, ws, ws bytes, stream
def _attn(hq=32, hkv=8, t=4096, d=128, q=FAKE, kc=FAKE, ks=FAKE, vc=FAKE, vs=FAKE, scale=0.088, out=FAKE):
    return (q, hq, hkv, t, d, kc, ks, vc, vs, ctypes.c_float(scale), out, None, 0, None)


@pytest.mark.parametrize("args,frag", [
    (_attn(hq=0), "num_q_heads=0"),
    (_attn(hkv=0), "num_kv_heads=0"),
    (_attn(t=0), "num_tokens=0"),
    (_attn(hq=12, hkv=8), "not 1..8 times"),
    (_attn(hq=72, hkv=8), "not 1..8 times"),
    (_attn(d=96), "head_dim=96"),
    (_attn(d=512), "head_dim=512"),
    (_attn(t=1 << 21, hkv=8), "2 GiB"),
    (_attn(hq=1 << 23, hkv=1 << 20, t=1), "queries larger than 2 GiB"),
    (_attn(q=0), "null"),
    (_attn(vs=0), "null"),
    (_attn(kc=MISALIGNED), "aligned"),
    (_attn(scale=float("inf")), "softmax_scale"),
    (_attn(scale=float("nan")), "softmax_scale"),
])
def test_attn_decode_validation(lib, args, frag):
    st, msg = _err(lib, "kvq_attn_decode_int8", *args)
    assert st == _lib.KVQ_E_INVALID and frag in msg, msg


def test_attn_decode_workspace_sizes(lib):
    b = ctypes.c_size_t()
    # 4096 tokens, 8 KV heads: 32 blocks of 128 tokens per head, one chunk
    # each (256 workgroups), records of 4 heads x (128 outputs, max, sum, 2 pad)
    assert lib.kvq_attn_decode_workspace_bytes(32, 8, 4096, 128, ctypes.byref(b)) == 0
    assert b.value == 4096 + 8 * 32 * 4 * 132 * 4
    # one block per head: no chunks to merge, no workspace
    assert lib.kvq_attn_decode_workspace_bytes(32, 8, 128, 128, ctypes.byref(b)) == 0
    assert b.value == 0
    # 6 query heads per KV head are padded to 8 in the records
    assert lib.kvq_attn_decode_workspace_bytes(48, 8, 1000, 128, ctypes.byref(b)) == 0
    assert b.value == 4096 + 8 * 8 * 8 * 132 * 4
    assert lib.kvq_attn_decode_workspace_bytes(32, 8, 0, 128, ctypes.byref(b)) == _lib.KVQ_E_INVALID
    # the record holds head_dim outputs, max, sum and two pad floats
    assert lib.kvq_attn_decode_workspace_bytes(16, 2, 4096, 256, ctypes.byref(b)) == 0
    assert b.value == 4096 + 2 * 32 * 8 * 260 * 4


def test_attn_decode_int4_validation(lib):
    f = ctypes.c_float(0.088)
    ok = (FAKE, 32, 8, 4096, 128)
    cache = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    for gs in (16, 96, 256):
        st, msg = _err(lib, "kvq_attn_decode_int4", *ok, gs, *cache, f, FAKE, None, 0, None)
        assert st == _lib.KVQ_E_INVALID and f"group_size={gs}" in msg, msg
    st, msg = _err(lib, "kvq_attn_decode_int4", *ok, 32, FAKE, FAKE, 0, FAKE, FAKE, FAKE, f, FAKE, None, 0, None)
    assert st == _lib.KVQ_E_INVALID and "null" in msg, msg
    st, msg = _err(lib, "kvq_attn_decode_int4", FAKE, 32, 8, 4096, 32, 32, *cache, f, FAKE, None, 0, None)
    assert st == _lib.KVQ_E_INVALID and "head_dim=32" in msg, msg
    # a group may not span two rows
    st, msg = _err(lib, "kvq_attn_decode_int4", FAKE, 32, 8, 4096, 64, 128, *cache, f, FAKE, None, 0, None)
    assert st == _lib.KVQ_E_INVALID and "group_size=128" in msg, msg


def test_attn_decode_varlen_validation(lib):
    f = ctypes.c_float(0.088)
    cache8 = (FAKE, FAKE, FAKE, FAKE)

    def call(batch=4, hq=32, hkv=8, d=128, seq=FAKE, total=1000, tmax=500):
        return _err(lib, "kvq_attn_decode_int8_varlen", FAKE, batch, hq, hkv, d, seq, total, tmax, *cache8, f, FAKE,
                    None, 0, None)
    for kw, frag in [(dict(batch=0), "batch=0"), (dict(hq=12), "not 1..8 times"), (dict(d=96), "head_dim=96"),
                     (dict(seq=0), "seq_start"), (dict(seq=FAKE + 2), "seq_start"),
                     (dict(tmax=1001), "exceeds total_tokens")]:
        st, msg = call(**kw)
        assert st == _lib.KVQ_E_INVALID and frag in msg, (kw, msg)
    b = ctypes.c_size_t()
    # 4 sequences x 8 KV heads = 32 units over up to 4096 tokens (32 blocks):
    # chunks of at most 2 blocks, 16 per unit
    assert lib.kvq_attn_decode_varlen_workspace_bytes(4, 32, 8, 4096, 128, ctypes.byref(b)) == 0
    assert b.value == 4096 + 4 * 8 * 16 * 4 * 132 * 4
    assert lib.kvq_attn_decode_varlen_workspace_bytes(64, 32, 8, 4096, 128, ctypes.byref(b)) == 0
    assert b.value == 4096 + 64 * 8 * 16 * 4 * 132 * 4
    # 64 sequences of at most 256 tokens x 8 heads: one workgroup each, nothing to merge
    assert lib.kvq_attn_decode_varlen_workspace_bytes(64, 32, 8, 256, 128, ctypes.byref(b)) == 0
    assert b.value == 0


def test_int4_noalloc_rejects_a_plan_beyond_its_scratch(lib):
    # 32 rows x K=4096 x 16384 columns: 128 tiles in 2 K slices of 32 x 128
    # fp32 partials need 4 MiB behind the 4 KiB counter area; the call
    # refuses on the host, before any HIP call
    p = _lib.Int4AwqProj(FAKE, FAKE, FAKE, FAKE, 16384)
    st, msg = _err(lib, "int4_awq_qkv_gemm_noalloc", FAKE, 32, 4096, 128, ctypes.byref(p), None, None, None)
    assert st == _lib.KVQ_E_INVALID and "scratch" in msg
    st, msg = _err(lib, "int4_awq_qkv_gemm_noalloc", FAKE, 0, 16384, 128, ctypes.byref(p), None, None, None)
    assert st == _lib.KVQ_E_INVALID and "m == 0" in msg
