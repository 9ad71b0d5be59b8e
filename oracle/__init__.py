"""CPU oracle for the quantized-decode hot path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the product package
``kv_quantization_amd``.  It shares no code with the HIP library.

The quantizers are encodings, so they live in plain C (``oracle.c``, fp32
operations one at a time, ``-ffp-contract=off``) and must agree bit for bit.
The two matrix products are plain definitions, written here as fp64 sums with
``numpy.matmul`` as the summation primitive:

* W8A8 (metrale_model_layers ``w8a8_decode.rs``, ``w8a8_gemv`` over the
  ``W8a8Weight`` segments): ``out[m, j] = sum_k (dec(qa[m,k]) * sa) *
  (dec(qw[j,k]) * sw)`` where the scales are per row, or per 128x128 weight
  block and per 128-column activation group.
* INT4 AWQ (boostr ``fused_int4_qkv.rs``, ``fused_int4_qkv_q/k/v``):
  ``out[m, j] = sum_k x[m,k] * (q[k,j] - z[k/gs, j]) * s[k/gs, j]`` with q
  unpacked in the ``QKV_AWQ_SHIFTS`` nibble order.

* Decode attention over the quantized cache (a reading: the pages define
  the cache and its dequantization, not the attention that reads it):
  textbook scaled-dot-product attention for one new token, ``out_h =
  sum_t softmax_t(scale * q_h . k_t) v_t`` over the dequantized keys and
  values, query head h reading KV head ``h // (Hq // Hkv)``; the bound is
  ``sum_t p_t |v_t|``.

Every function returns, next to the reference value, the bound
``sum_k |a_k| |w_k|`` of the operands actually multiplied, which the parity
tests scale by the 1e-3 relative tolerance.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_DIR = Path(__file__).resolve().parent
_SRC = _DIR / "oracle.c"
_LIB = _DIR / "liboracle.so"

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11"]


def build(force: bool = False) -> Path:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (no SIMD intrinsics)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(f".so.tmp{os.getpid()}")
        subprocess.run(["gcc", *CFLAGS, str(_SRC), "-o", str(tmp), "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(str(build()))
        i64 = ctypes.c_int64
        p = ctypes.c_void_p
        sig = {
            "oracle_num_threads": ([], ctypes.c_int),
            "oracle_set_num_threads": ([ctypes.c_int], None),
            "oracle_kv_int8_quant": ([p, p, p, i64, i64], None),
            "oracle_kv_int8_dequant": ([p, p, p, i64, i64], None),
            "oracle_kv_int8_quant_tensor": ([p, p, p, i64], None),
            "oracle_kv_int8_dequant_tensor": ([p, ctypes.c_float, p, i64], None),
            "oracle_kv_fp8_quant": ([p, p, p, i64, i64], None),
            "oracle_kv_fp8_dequant": ([p, p, p, i64, i64], None),
            "oracle_kv_int4_quant": ([p, p, p, p, i64, i64, i64], None),
            "oracle_kv_int4_dequant": ([p, p, p, p, i64, i64, i64], None),
            "oracle_bf16_to_f32": ([ctypes.c_uint16], ctypes.c_float),
            "oracle_f32_to_bf16": ([ctypes.c_float], ctypes.c_uint16),
            "oracle_e4m3_decode": ([ctypes.c_uint8], ctypes.c_float),
            "oracle_e4m3_encode": ([ctypes.c_float], ctypes.c_uint8),
            "oracle_exp": ([ctypes.c_float], ctypes.c_float),
            "oracle_silu": ([ctypes.c_float], ctypes.c_float),
            "oracle_act_quant": ([ctypes.c_int, ctypes.c_int, p, p, i64, i64, i64, p, p], None),
            "oracle_weight_quant": ([ctypes.c_int, p, i64, i64, p, p], None),
            "oracle_awq_unpack": ([p, p, i64, i64], None),
            "oracle_awq_pack": ([p, p, i64, i64], None),
            "oracle_awq_dequant_f64": ([p, p, p, p, i64, i64, i64], None),
            "oracle_e4m3_dequant_f64": ([ctypes.c_int, p, p, p, i64, i64], None),
            "oracle_e4m3_encode_array": ([p, p, i64], None),
            "oracle_f32_to_bf16_array": ([p, p, i64], None),
            "oracle_exp_array": ([p, p, i64], None),
            "oracle_silu_array": ([p, p, i64], None),
        }
        for name, (args, res) in sig.items():
            fn = getattr(_lib, name)
            fn.argtypes = args
            fn.restype = res
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the oracle's parallel loops from now on (timing only)."""
    lib().oracle_set_num_threads(int(n))


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def _finite(x: np.ndarray) -> None:
    if not np.all(np.isfinite(x)):
        raise ValueError("oracle inputs must be finite (NaN/Inf are outside the method's contract)")


# --------------------------------------------------------------------------
# KV cache codecs (boostr kv_cache_quant.wgsl)

def kv_int8_quant(x: np.ndarray):
    """Per-token symmetric INT8 (section "INT8 Per-Token Quantization").

    x: float32 [T, D] -> (codes int8 [T, D], scales float32 [T])."""
    x = _c(x, np.float32)
    _finite(x)
    t, d = x.shape
    codes = np.empty((t, d), np.int8)
    scales = np.empty(t, np.float32)
    lib().oracle_kv_int8_quant(_p(x), _p(codes), _p(scales), t, d)
    return codes, scales


def kv_int8_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Section "INT8 Per-Token Dequantization": float(code) * scale."""
    codes = _c(codes, np.int8)
    scales = _c(scales, np.float32)
    t, d = codes.shape
    y = np.empty((t, d), np.float32)
    lib().oracle_kv_int8_dequant(_p(codes), _p(scales), _p(y), t, d)
    return y


def kv_int8_quant_tensor(x: np.ndarray):
    """Per-tensor symmetric INT8: the declared ``mode = 0`` of the page's
    parameter block, read as the per-token rule over the whole tensor.

    x: float32, any shape -> (codes int8, same shape; scale float32 [1])."""
    x = _c(x, np.float32)
    _finite(x)
    codes = np.empty(x.shape, np.int8)
    scale = np.empty(1, np.float32)
    lib().oracle_kv_int8_quant_tensor(_p(x), _p(codes), _p(scale), x.size)
    return codes, scale


def kv_int8_dequant_tensor(codes: np.ndarray, scale) -> np.ndarray:
    """float(code) * scale with the tensor's one scale."""
    codes = _c(codes, np.int8)
    y = np.empty(codes.shape, np.float32)
    lib().oracle_kv_int8_dequant_tensor(_p(codes), float(np.float32(np.asarray(scale).reshape(-1)[0])), _p(y),
                                        codes.size)
    return y


def kv_fp8_quant(x: np.ndarray):
    """Section "FP8 Per-Token Quantization" (an integer /127 code, same bytes as INT8)."""
    x = _c(x, np.float32)
    _finite(x)
    t, d = x.shape
    codes = np.empty((t, d), np.int8)
    scales = np.empty(t, np.float32)
    lib().oracle_kv_fp8_quant(_p(x), _p(codes), _p(scales), t, d)
    return codes, scales


def kv_fp8_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.int8)
    scales = _c(scales, np.float32)
    t, d = codes.shape
    y = np.empty((t, d), np.float32)
    lib().oracle_kv_fp8_dequant(_p(codes), _p(scales), _p(y), t, d)
    return y


def kv_int4_quant(x: np.ndarray, group_size: int):
    """Per-group asymmetric INT4 (section "INT4 Per-Group Quantization").

    x: float32 [T, D]; groups of ``group_size`` over the flattened array.
    -> (packed uint8 [T*D/2], scales float32 [G], zeros float32 [G])."""
    x = _c(x, np.float32)
    _finite(x)
    t, d = x.shape
    if group_size < 2 or group_size % 2 or (t * d) % group_size:
        raise ValueError("group_size must be even and divide num_tokens*head_dim")
    g = t * d // group_size
    packed = np.empty(t * d // 2, np.uint8)
    scales = np.empty(g, np.float32)
    zeros = np.empty(g, np.float32)
    lib().oracle_kv_int4_quant(_p(x), _p(packed), _p(scales), _p(zeros), t, d, group_size)
    return packed, scales, zeros


def kv_int4_dequant(packed, scales, zeros, num_tokens: int, head_dim: int, group_size: int):
    """Section "INT4 Per-Group Dequantization": code*scale - zero*scale."""
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.float32)
    zeros = _c(zeros, np.float32)
    y = np.empty((num_tokens, head_dim), np.float32)
    lib().oracle_kv_int4_dequant(_p(packed), _p(scales), _p(zeros), _p(y), num_tokens, head_dim, group_size)
    return y


# --------------------------------------------------------------------------
# Number formats

def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits (uint16), round to nearest even; element by element in C."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_bf16_array(_p(x), _p(out), x.size)
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bits -> fp32 (exact: the bits become the top half)."""
    return (_c(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


# 16-bit value formats of the KV codecs: 1 = fp16, 2 = bf16 (0 = fp32).

def widen16(bits: np.ndarray, dtype: int) -> np.ndarray:
    """fp16 or bf16 bits (uint16) -> fp32, exact (every 16-bit value is an fp32)."""
    bits = _c(bits, np.uint16)
    if dtype == 1:
        return bits.view(np.float16).astype(np.float32)
    if dtype == 2:
        return bf16_to_f32(bits)
    raise ValueError("dtype must be 1 (fp16) or 2 (bf16)")


def narrow16(x: np.ndarray, dtype: int) -> np.ndarray:
    """fp32 -> fp16 or bf16 bits, round to nearest even (numpy's IEEE cast for
    fp16, the C routine above for bf16)."""
    x = _c(x, np.float32)
    if dtype == 1:
        with np.errstate(over="ignore"):
            return x.astype(np.float16).view(np.uint16)
    if dtype == 2:
        return f32_to_bf16(x)
    raise ValueError("dtype must be 1 (fp16) or 2 (bf16)")


def kv_int8_quant_dt(x_bits: np.ndarray, dtype: int):
    """INT8 per token of a 16-bit cache: the fp32 codec on the exactly widened values."""
    return kv_int8_quant(widen16(x_bits, dtype))


def kv_int8_dequant_dt(codes, scales, dtype: int) -> np.ndarray:
    """fp32 dequantization, then rounding to the 16-bit type."""
    return narrow16(kv_int8_dequant(codes, scales), dtype)


def kv_int4_quant_dt(x_bits: np.ndarray, group_size: int, dtype: int):
    return kv_int4_quant(widen16(x_bits, dtype), group_size)


def kv_int4_dequant_dt(packed, scales, zeros, num_tokens: int, head_dim: int, group_size: int, dtype: int):
    return narrow16(kv_int4_dequant(packed, scales, zeros, num_tokens, head_dim, group_size), dtype)


def e4m3_encode(x) -> np.ndarray:
    """fp32 -> E4M3FN codes (RNE, saturating, sign kept), element by element in C."""
    x = _c(np.atleast_1d(x), np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().oracle_e4m3_encode_array(_p(x), _p(out), x.size)
    return out


def e4m3_decode_table() -> np.ndarray:
    """float32 [256]: the value of every E4M3FN code (NaN for 0x7F/0xFF)."""
    f = lib().oracle_e4m3_decode
    return np.array([f(c) for c in range(256)], np.float32)


def exp_k(y) -> np.ndarray:
    """The pinned SiLU exponential (Cody-Waite + degree-7 Taylor), fp32."""
    y = _c(np.atleast_1d(y), np.float32)
    out = np.empty(y.shape, np.float32)
    lib().oracle_exp_array(_p(y), _p(out), y.size)
    return out


def silu(v) -> np.ndarray:
    """v / (1 + exp_k(-v)) in fp32."""
    v = _c(np.atleast_1d(v), np.float32)
    out = np.empty(v.shape, np.float32)
    lib().oracle_silu_array(_p(v), _p(out), v.size)
    return out


# --------------------------------------------------------------------------
# W8A8 FP8 decode (metrale_model_layers w8a8_decode.rs)

ROWSCALE = 0  # W8a8Scale::PerRow
BLK128 = 1    # W8a8Scale::Block128


def act_quant(kind: int, x_bf16: np.ndarray, k: int, silu: bool = False, up_bf16=None):
    """Activation quantization (w8a8_act_quant / w8a8_act_quant_silu).

    x_bf16: uint16 [rows, ldx]; up_bf16 the same shape or None.
    -> (q uint8 [rows, k], scales float32 [rows] or [rows, k/128])."""
    x = _c(x_bf16, np.uint16)
    rows, ldx = x.shape
    _finite(bf16_to_f32(x[:, :k]))
    if k % 128 or ldx < k:
        raise ValueError("k must be a multiple of 128 and ldx >= k")
    up = None if up_bf16 is None else _c(up_bf16, np.uint16)
    if up is not None and (up.shape != x.shape or not silu):
        raise ValueError("up must match x and is only used with silu")
    q = np.empty((rows, k), np.uint8)
    scales = np.empty((rows,) if kind == ROWSCALE else (rows, k // 128), np.float32)
    lib().oracle_act_quant(kind, int(silu), _p(x), 0 if up is None else _p(up), ldx, rows, k, _p(q), _p(scales))
    return q, scales


def weight_quant(kind: int, w: np.ndarray):
    """E4M3 weight quantization with the activation rule, per weight row
    (ROWSCALE) or per 128x128 block (BLK128).  w: float32 [n, k]."""
    w = _c(w, np.float32)
    _finite(w)
    n, k = w.shape
    if k % 128:
        raise ValueError("k must be a multiple of 128")
    q = np.empty((n, k), np.uint8)
    scales = np.empty((n,) if kind == ROWSCALE else ((n + 127) // 128, k // 128), np.float32)
    lib().oracle_weight_quant(kind, _p(w), n, k, _p(q), _p(scales))
    return q, scales


def e4m3_dequant_f64(mode: int, q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """mode 0: per-row scale; 1: 128x128 weight blocks; 2: activation 128-groups."""
    q = _c(q, np.uint8)
    scales = _c(scales, np.float32)
    n, k = q.shape
    out = np.empty((n, k), np.float64)
    lib().oracle_e4m3_dequant_f64(mode, _p(q), _p(scales), _p(out), n, k)
    return out


def w8a8_gemv(kind: int, q: np.ndarray, a_scales: np.ndarray, segments):
    """Reference for ``w8a8_gemv`` over 1..3 concatenated weight segments.

    q: uint8 [M, K] activation codes; a_scales [M] or [M, K/128];
    segments: list of (codes uint8 [n_i, K], scales [n_i] or [ceil(n_i/128), K/128]).
    Output column j belongs to the first segment whose running row total
    exceeds j (the W8a8Weight boundaries).
    -> (ref float64 [M, N] unrounded, bound float64 [M, N])."""
    a = e4m3_dequant_f64(0 if kind == ROWSCALE else 2, q, a_scales)
    ws = [e4m3_dequant_f64(0 if kind == ROWSCALE else 1, wq, ws) for wq, ws in segments]
    w = np.concatenate(ws, axis=0)            # [N, K]
    ref = np.matmul(a, w.T)
    bound = np.matmul(np.abs(a), np.abs(w).T)
    return ref, bound


def w8a8_gemv_sampled(kind: int, q, a_scales, segments, rows_idx, cols_idx):
    """The same definition evaluated only at the (row, col) pairs given, one
    dot product per pair, for full-size spot checks."""
    rows_idx = np.asarray(rows_idx)
    cols_idx = np.asarray(cols_idx)
    bounds_n = np.cumsum([0] + [s[0].shape[0] for s in segments])
    ref = np.empty(rows_idx.size, np.float64)
    bnd = np.empty(rows_idx.size, np.float64)
    arow_cache = {}
    for i, (m, j) in enumerate(zip(rows_idx.tolist(), cols_idx.tolist())):
        if m not in arow_cache:
            arow_cache[m] = e4m3_dequant_f64(0 if kind == ROWSCALE else 2, q[m:m + 1],
                                             a_scales[m:m + 1])[0]
        a = arow_cache[m]
        si = int(np.searchsorted(bounds_n, j, side="right") - 1)
        wq, wsc = segments[si]
        jj = j - bounds_n[si]
        if kind == ROWSCALE:
            w = e4m3_dequant_f64(0, wq[jj:jj + 1], wsc[jj:jj + 1])[0]
        else:
            # rebuild the row with its 128-block band of scales
            band = wsc[jj // 128: jj // 128 + 1]
            w = e4m3_dequant_f64(1, wq[jj:jj + 1], band)[0]
        ref[i] = float(np.dot(a, w))
        bnd[i] = float(np.dot(np.abs(a), np.abs(w)))
    return ref, bnd


# --------------------------------------------------------------------------
# INT4 AWQ (boostr fused_int4_qkv.rs)

AWQ_SHIFTS = (0, 16, 4, 20, 8, 24, 12, 28)


def awq_unpack(qweight: np.ndarray, n: int) -> np.ndarray:
    """u32 [K, n/8] -> codes uint8 [K, n] (unpack_awq_qkv for every column)."""
    qw = _c(qweight, np.uint32)
    k = qw.shape[0]
    codes = np.empty((k, n), np.uint8)
    lib().oracle_awq_unpack(_p(qw), _p(codes), k, n)
    return codes


def awq_pack(codes: np.ndarray) -> np.ndarray:
    c = _c(codes, np.uint8)
    k, n = c.shape
    qw = np.empty((k, n // 8), np.uint32)
    lib().oracle_awq_pack(_p(c), _p(qw), k, n)
    return qw


def awq_dequant_f64(qweight, scales, zeros, group_size: int) -> np.ndarray:
    """[K, n] fp64 weights (q - z) * s, per the fused_int4_qkv kernels."""
    qw = _c(qweight, np.uint32)
    s = _c(scales, np.float32)
    z = _c(zeros, np.float32)
    k, n8 = qw.shape
    n = n8 * 8
    if k % group_size:
        raise ValueError("K must be a multiple of group_size")
    w = np.empty((k, n), np.float64)
    lib().oracle_awq_dequant_f64(_p(qw), _p(s), _p(z), _p(w), k, n, group_size)
    return w


def int4_awq_gemm(x: np.ndarray, qweight, scales, zeros, group_size: int):
    """One projection of fused_int4_qkv: x float32 [M, K] -> (ref fp64 [M, n], bound)."""
    x64 = _c(x, np.float32).astype(np.float64)
    w = awq_dequant_f64(qweight, scales, zeros, group_size)
    return np.matmul(x64, w), np.matmul(np.abs(x64), np.abs(w))


def int4_awq_qkv(x, projections, group_size: int):
    """Q, K, V (or a single projection): list of (ref, bound) per projection."""
    return [int4_awq_gemm(x, qw, s, z, group_size) for (qw, s, z) in projections]


# --------------------------------------------------------------------------
# Decode attention over the quantized cache.  The pages define the cache and
# its dequantization but not the attention that reads it; the reading taken
# is textbook scaled-dot-product attention for one new token per query head,
# with consecutive query heads sharing a KV head (grouped queries).

def attn_decode(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, softmax_scale: float):
    """q float32 [Hq, D]; k_hat, v_hat float32 [T, Hkv, D], the cache as the
    pages' dequantization gives it; Hq a multiple of Hkv, and query head h
    reads KV head h // (Hq // Hkv).  In fp64: s_t = softmax_scale * (q_h .
    k_t); p = softmax(s), computed as exp(s - max s) / sum; out_h = sum_t
    p_t v_t.  Returns (out fp64 [Hq, D], bound fp64 [Hq, D] = sum_t p_t |v_t|),
    the bound of the weighted sum the parity tests scale by 1e-3."""
    q64 = _c(q, np.float32).astype(np.float64)
    k64 = _c(k_hat, np.float32).astype(np.float64)
    v64 = _c(v_hat, np.float32).astype(np.float64)
    hq, d = q64.shape
    t, hkv, dk = k64.shape
    if dk != d or v64.shape != k64.shape or t < 1 or hkv < 1 or hq % hkv:
        raise ValueError("attn_decode: shapes do not match")
    sc = float(np.float32(softmax_scale))      # the fp32 value a caller passes
    grp = hq // hkv
    out = np.empty((hq, d))
    bound = np.empty((hq, d))
    for h in range(hq):
        g = h // grp
        s = sc * np.matmul(k64[:, g, :], q64[h])
        p = np.exp(s - s.max())
        p /= p.sum()
        out[h] = np.matmul(p, v64[:, g, :])
        bound[h] = np.matmul(p, np.abs(v64[:, g, :]))
    return out, bound


def attn_decode_int8(q, k_codes, k_scales, v_codes, v_scales, softmax_scale: float):
    """Keys and values as per-token INT8: codes int8 [T, Hkv, D], one scale
    per (token, head) row, float32 [T, Hkv], dequantized by the INT8 section."""
    t, hkv, d = np.shape(k_codes)
    kh = kv_int8_dequant(np.reshape(k_codes, (t * hkv, d)), np.reshape(k_scales, t * hkv)).reshape(t, hkv, d)
    vh = kv_int8_dequant(np.reshape(v_codes, (t * hkv, d)), np.reshape(v_scales, t * hkv)).reshape(t, hkv, d)
    return attn_decode(q, kh, vh, softmax_scale)


def attn_decode_int4(q, k_packed, k_scales, k_zeros, v_packed, v_scales, v_zeros, num_tokens: int,
                     num_kv_heads: int, head_dim: int, group_size: int, softmax_scale: float):
    """Keys and values as per-group INT4 over the flattened [T, Hkv, D] cache
    (group_size divides D, so no group spans two rows), dequantized by the
    INT4 section."""
    rows = num_tokens * num_kv_heads
    kh = kv_int4_dequant(k_packed, k_scales, k_zeros, rows, head_dim, group_size)
    vh = kv_int4_dequant(v_packed, v_scales, v_zeros, rows, head_dim, group_size)
    shp = (num_tokens, num_kv_heads, head_dim)
    return attn_decode(q, kh.reshape(shp), vh.reshape(shp), softmax_scale)


def attn_decode_varlen(q, seq_start, k_hat, v_hat, softmax_scale: float):
    """A batch: q float32 [B, Hq, D]; sequence b reads cache rows
    seq_start[b] .. seq_start[b+1]-1 of k_hat, v_hat [T_total, Hkv, D]; a
    sequence with no tokens has output 0 (and bound 0).  Returns (out, bound)
    fp64 [B, Hq, D]."""
    q = _c(q, np.float32)
    bsz, hq, d = q.shape
    out = np.zeros((bsz, hq, d))
    bound = np.zeros((bsz, hq, d))
    for b in range(bsz):
        s0, s1 = int(seq_start[b]), int(seq_start[b + 1])
        if s1 > s0:
            out[b], bound[b] = attn_decode(q[b], k_hat[s0:s1], v_hat[s0:s1], softmax_scale)
    return out, bound
