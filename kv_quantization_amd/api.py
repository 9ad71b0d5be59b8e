"""PyTorch-facing wrappers over the libkvq.so C ABI.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind include/kvq.h.  torch provides device memory and the current
stream; tensors must live on a ROCm device, be contiguous and have the dtype
each function states.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import W8A8_BLK128, W8A8_ROWSCALE, Int4AwqProj, W8a8Segment

ROWSCALE = W8A8_ROWSCALE
BLK128 = W8A8_BLK128


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, dtype, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _empty(shape, dtype, like: torch.Tensor):
    return torch.empty(shape, dtype=dtype, device=like.device)


# ------------------------------------------------------------ workspace ----

_workspaces: dict = {}
# Buffers replaced by a larger one.  They are never freed: a HIP graph
# captured while one was current keeps its address and may be replayed later.
_retired: list = []


def workspace(device: torch.device, nbytes: int, stream: int) -> torch.Tensor:
    """A zero-filled device buffer of at least nbytes, cached per (device,
    stream).  The kernels leave the counter area at its start zero-filled and
    put partial results only behind it, so reuse by calls ordered on one
    stream is safe.  A buffer is created or grown only outside graph capture
    (the zero fill must run before the first kernel reads the counters);
    inside a capture a call that needs a new or larger buffer raises: make
    one eager call of that shape on the stream first."""
    key = (torch.device(device), stream)
    buf = _workspaces.get(key)
    if buf is None or buf.numel() < nbytes:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError(
                f"kv_quantization_amd: this call needs a workspace of {nbytes} bytes on stream {stream:#x}, "
                "which cannot be allocated and zero-filled during graph capture; make one eager call of the "
                "same shape on this stream before capturing")
        if buf is not None:
            _retired.append(buf)
        # zero fill enqueued on the current stream, the one the kernels use
        buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = buf
    return buf


# ----------------------------------------------------------- KV cache ------

# value dtypes of the KV codecs (kvq_dtype_t)
_KV_DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


def _kv_dt(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _KV_DT:
        raise TypeError(f"{name} must be float32, float16 or bfloat16, got {t.dtype}")
    return _KV_DT[t.dtype]


def quant_int8_token(x: torch.Tensor, codes=None, scales=None):
    """x fp32/fp16/bf16 [T, D] -> (codes int8 [T, D], scales fp32 [T])."""
    t, d = x.shape
    codes = _empty((t, d), torch.int8, x) if codes is None else codes
    scales = _empty((t,), torch.float32, x) if scales is None else scales
    dt = _kv_dt(x, "x")
    if dt == 0:
        _lib.call("kvq_quant_int8_token", _dev(x, torch.float32, "x"), _dev(codes, torch.int8, "codes"),
                  _dev(scales, torch.float32, "scales"), t, d, _stream(x))
    else:
        _lib.call("kvq_quant_int8_token_dt", _dev(x, x.dtype, "x"), dt, _dev(codes, torch.int8, "codes"),
                  _dev(scales, torch.float32, "scales"), t, d, _stream(x))
    return codes, scales


def dequant_int8_token(codes: torch.Tensor, scales: torch.Tensor, out=None, dtype=torch.float32):
    """-> y [T, D] of `dtype` (or of out's dtype): fp32 value, 16-bit rounded to nearest even."""
    t, d = codes.shape
    out = _empty((t, d), dtype, codes) if out is None else out
    dt = _kv_dt(out, "out")
    if dt == 0:
        _lib.call("kvq_dequant_int8_token", _dev(codes, torch.int8, "codes"),
                  _dev(scales, torch.float32, "scales"), _dev(out, torch.float32, "out"), t, d, _stream(codes))
    else:
        _lib.call("kvq_dequant_int8_token_dt", _dev(codes, torch.int8, "codes"),
                  _dev(scales, torch.float32, "scales"), _dev(out, out.dtype, "out"), dt, t, d, _stream(codes))
    return out


def quant_int8_tensor(x: torch.Tensor, codes=None, scale=None):
    """Per-tensor INT8 (the KV page's declared per-tensor mode): x fp32 [T, D]
    -> (codes int8 [T, D], scale fp32 [1]).  Two launches; uses the shared
    workspace for the partial maxima."""
    t, d = x.shape
    codes = _empty((t, d), torch.int8, x) if codes is None else codes
    scale = _empty((1,), torch.float32, x) if scale is None else scale
    stream = _stream(x)
    nbytes = _lib.INT8_TENSOR_WORKSPACE_BYTES
    ws = workspace(x.device, nbytes, stream)
    _lib.call("kvq_quant_int8_tensor", _dev(x, torch.float32, "x"), _dev(codes, torch.int8, "codes"),
              _dev(scale, torch.float32, "scale"), t, d, ws.data_ptr(), nbytes, stream)
    return codes, scale


def dequant_int8_tensor(codes: torch.Tensor, scale: torch.Tensor, out=None):
    t, d = codes.shape
    out = _empty((t, d), torch.float32, codes) if out is None else out
    _lib.call("kvq_dequant_int8_tensor", _dev(codes, torch.int8, "codes"), _dev(scale, torch.float32, "scale"),
              _dev(out, torch.float32, "out"), t, d, _stream(codes))
    return out


def quant_int4_group(x: torch.Tensor, group_size: int, packed=None, scales=None, zeros=None):
    """x fp32/fp16/bf16 [T, D] -> (packed uint8 [T*D/2], scales fp32 [G], zeros fp32 [G])."""
    t, d = x.shape
    total = t * d
    g = total // group_size if group_size else 0
    packed = _empty((total // 2,), torch.uint8, x) if packed is None else packed
    scales = _empty((g,), torch.float32, x) if scales is None else scales
    zeros = _empty((g,), torch.float32, x) if zeros is None else zeros
    dt = _kv_dt(x, "x")
    args = (_dev(packed, torch.uint8, "packed"), _dev(scales, torch.float32, "scales"),
            _dev(zeros, torch.float32, "zeros"), t, d, group_size, _stream(x))
    if dt == 0:
        _lib.call("kvq_quant_int4_group", _dev(x, torch.float32, "x"), *args)
    else:
        _lib.call("kvq_quant_int4_group_dt", _dev(x, x.dtype, "x"), dt, *args)
    return packed, scales, zeros


def dequant_int4_group(packed, scales, zeros, num_tokens: int, head_dim: int, group_size: int, out=None,
                       dtype=torch.float32):
    out = _empty((num_tokens, head_dim), dtype, packed) if out is None else out
    dt = _kv_dt(out, "out")
    head = (_dev(packed, torch.uint8, "packed"), _dev(scales, torch.float32, "scales"),
            _dev(zeros, torch.float32, "zeros"))
    if dt == 0:
        _lib.call("kvq_dequant_int4_group", *head, _dev(out, torch.float32, "out"), num_tokens, head_dim,
                  group_size, _stream(packed))
    else:
        _lib.call("kvq_dequant_int4_group_dt", *head, _dev(out, out.dtype, "out"), dt, num_tokens, head_dim,
                  group_size, _stream(packed))
    return out


# --------------------------------------------------------------- W8A8 ------

def scratch_bytes(kind: int, rows: int, k: int):
    qb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _lib.call("w8a8_scratch_bytes", kind, rows, k, ctypes.byref(qb), ctypes.byref(sb))
    return qb.value, sb.value


def act_quant(x: torch.Tensor, k: int | None = None, kind: int = ROWSCALE, silu: bool = False,
              up: torch.Tensor | None = None, q=None, scales=None):
    """x bf16 [rows, ldx] (gate when silu) -> (q uint8 [rows, k], scales fp32)."""
    rows, ldx = x.shape
    k = ldx if k is None else k
    q = _empty((rows, k), torch.uint8, x) if q is None else q
    if scales is None:
        scales = _empty((rows,) if kind == ROWSCALE else (rows, k // 128), torch.float32, x)
    up_ptr = 0 if up is None else _dev(up, torch.bfloat16, "up")
    if up is not None and up.shape != x.shape:
        raise ValueError("up must have the shape of x")
    _lib.call("w8a8_act_quant", kind, int(silu), _dev(x, torch.bfloat16, "x"), up_ptr, ldx, rows, k,
              _dev(q, torch.uint8, "q"), _dev(scales, torch.float32, "scales"), _stream(x))
    return q, scales


def weight_quant(w: torch.Tensor, kind: int = ROWSCALE):
    """w fp32 [n, k] -> (codes uint8 [n, k], scales fp32 [n] or [ceil(n/128), k/128])."""
    n, k = w.shape
    q = _empty((n, k), torch.uint8, w)
    s = _empty((n,) if kind == ROWSCALE else ((n + 127) // 128, k // 128), torch.float32, w)
    _lib.call("w8a8_weight_quant", kind, _dev(w, torch.float32, "w"), n, k, _dev(q, torch.uint8, "q"),
              _dev(s, torch.float32, "scales"), _stream(w))
    return q, s


def f32_to_e4m3(x: torch.Tensor, out=None):
    out = _empty(x.shape, torch.uint8, x) if out is None else out
    _lib.call("kvq_f32_to_e4m3", _dev(x, torch.float32, "x"), _dev(out, torch.uint8, "out"), x.numel(), _stream(x))
    return out


@dataclass
class W8a8Weight:
    """1..3 E4M3 weight segments sharing K (metrale W8a8Weight)."""
    kind: int
    segments: list  # [(codes uint8 [n_i, k], scales fp32), ...]

    @property
    def k(self) -> int:
        return int(self.segments[0][0].shape[1])

    @property
    def n(self) -> int:
        return int(sum(int(c.shape[0]) for c, _ in self.segments))

    def c_segments(self):
        arr = (W8a8Segment * 3)()
        for i, (c, s) in enumerate(self.segments):
            arr[i].w = _dev(c, torch.uint8, f"segment {i} codes")
            arr[i].scale = _dev(s, torch.float32, f"segment {i} scales")
            arr[i].n = int(c.shape[0])
        return arr


def gemv_workspace_bytes(kind: int, rows: int, k: int, n_total: int) -> int:
    b = ctypes.c_size_t()
    _lib.call("w8a8_gemv_workspace_bytes", kind, rows, k, n_total, ctypes.byref(b))
    return b.value


def gemv(q: torch.Tensor, a_scales: torch.Tensor, weight: W8a8Weight, out=None, ldc: int | None = None,
         use_workspace: bool = True):
    """(q, a_scales) from act_quant, W8a8Weight -> out bf16 [rows, ldc]."""
    rows, k = q.shape
    n = weight.n
    ldc = n if ldc is None else ldc
    out = _empty((rows, ldc), torch.bfloat16, q) if out is None else out
    stream = _stream(q)
    ws_ptr, ws_bytes = 0, 0
    if use_workspace:
        ws_bytes = gemv_workspace_bytes(weight.kind, rows, k, n)
        if ws_bytes:
            ws_ptr = workspace(q.device, ws_bytes, stream).data_ptr()
    _lib.call("w8a8_gemv", weight.kind, _dev(q, torch.uint8, "q"), _dev(a_scales, torch.float32, "a_scales"), rows,
              k, weight.c_segments(), len(weight.segments), _dev(out, torch.bfloat16, "out"), ldc, ws_ptr, ws_bytes,
              stream)
    return out


def proj(x: torch.Tensor, weight: W8a8Weight, silu: bool = False, up=None, out=None, scratch=None):
    """act_quant + gemv in one call (metrale w8a8_proj); one launch for <= 8
    rows.  scratch: optional (codes uint8 [rows, k], scales fp32) that receive
    the activation codes and scales."""
    rows, ldx = x.shape
    k = weight.k
    if scratch is None:
        q = _empty((rows, k), torch.uint8, x)
        sa = _empty((rows,) if weight.kind == ROWSCALE else (rows, k // 128), torch.float32, x)
    else:
        q, sa = scratch
        _dev(q, torch.uint8, "scratch codes")
        _dev(sa, torch.float32, "scratch scales")
        if q.numel() < rows * k or sa.numel() < rows * (1 if weight.kind == ROWSCALE else k // 128):
            raise ValueError("scratch buffers too small for rows x k")
    n = weight.n
    out = _empty((rows, n), torch.bfloat16, x) if out is None else out
    stream = _stream(x)
    ws_bytes = gemv_workspace_bytes(weight.kind, rows, k, n)
    ws_ptr = workspace(x.device, ws_bytes, stream).data_ptr() if ws_bytes else 0
    up_ptr = 0 if up is None else _dev(up, torch.bfloat16, "up")
    _lib.call("w8a8_proj", weight.kind, int(silu), _dev(x, torch.bfloat16, "x"), up_ptr, ldx, rows, k,
              weight.c_segments(), len(weight.segments), _dev(out, torch.bfloat16, "out"), out.shape[1],
              q.data_ptr(), sa.data_ptr(), ws_ptr, ws_bytes, stream)
    return out


# ------------------------------------------------------------ INT4 AWQ -----

def int4_workspace_bytes(m: int, k: int, group_size: int, n_total: int) -> int:
    b = ctypes.c_size_t()
    _lib.call("int4_awq_workspace_bytes", m, k, group_size, n_total, ctypes.byref(b))
    return b.value


def int4_awq_qkv(x: torch.Tensor, projections, group_size: int, outs=None, use_workspace: bool = True):
    """x fp32/fp16/bf16 [m, k]; projections: 1 or 3 of (qweight int32/uint32 [k, n/8],
    scales fp32 [k/gs, n], zeros fp32 [k/gs, n]) -> list of fp32 [m, n]."""
    m, k = x.shape
    if len(projections) not in (1, 3):
        raise ValueError("need 1 (single) or 3 (Q, K, V) projections")
    structs, res = [], []
    for i, (qw, sc, zr) in enumerate(projections):
        n = int(qw.shape[1]) * 8
        o = _empty((m, n), torch.float32, x) if outs is None else outs[i]
        p = Int4AwqProj()
        if qw.dtype not in (torch.int32, torch.uint32):
            raise TypeError("qweight must be int32/uint32")
        p.qweight = _dev(qw, qw.dtype, "qweight")
        p.scales = _dev(sc, torch.float32, "scales")
        p.zeros = _dev(zr, torch.float32, "zeros")
        p.out = _dev(o, torch.float32, "out")
        p.n = n
        structs.append(p)
        res.append(o)
    stream = _stream(x)
    n_total = sum(s.n for s in structs)
    ws_ptr, ws_bytes = 0, 0
    if use_workspace:
        ws_bytes = int4_workspace_bytes(m, k, group_size, n_total)
        if ws_bytes:
            ws_ptr = workspace(x.device, ws_bytes, stream).data_ptr()
    kp = ctypes.byref(structs[1]) if len(structs) == 3 else None
    vp = ctypes.byref(structs[2]) if len(structs) == 3 else None
    xdt = _kv_dt(x, "x")
    if xdt == 0:
        _lib.call("int4_awq_qkv_gemm", _dev(x, torch.float32, "x"), m, k, group_size, ctypes.byref(structs[0]), kp,
                  vp, ws_ptr, ws_bytes, stream)
    else:
        _lib.call("int4_awq_qkv_gemm_dt", _dev(x, x.dtype, "x"), xdt, m, k, group_size, ctypes.byref(structs[0]),
                  kp, vp, ws_ptr, ws_bytes, stream)
    return res


def int4_awq_qkv_noalloc(x: torch.Tensor, projections, group_size: int, outs=None):
    """int4_awq_qkv through int4_awq_qkv_gemm_noalloc: the library's own
    per-GPU scratch instead of a workspace (nothing is allocated for it).
    x fp32 [m, k]; projections and outputs as int4_awq_qkv."""
    m, k = x.shape
    if len(projections) not in (1, 3):
        raise ValueError("need 1 (single) or 3 (Q, K, V) projections")
    structs, res = [], []
    for i, (qw, sc, zr) in enumerate(projections):
        n = int(qw.shape[1]) * 8
        o = _empty((m, n), torch.float32, x) if outs is None else outs[i]
        p = Int4AwqProj()
        if qw.dtype not in (torch.int32, torch.uint32):
            raise TypeError("qweight must be int32/uint32")
        p.qweight = _dev(qw, qw.dtype, "qweight")
        p.scales = _dev(sc, torch.float32, "scales")
        p.zeros = _dev(zr, torch.float32, "zeros")
        p.out = _dev(o, torch.float32, "out")
        p.n = n
        structs.append(p)
        res.append(o)
    kp = ctypes.byref(structs[1]) if len(structs) == 3 else None
    vp = ctypes.byref(structs[2]) if len(structs) == 3 else None
    _lib.call("int4_awq_qkv_gemm_noalloc", _dev(x, torch.float32, "x"), m, k, group_size, ctypes.byref(structs[0]),
              kp, vp, _stream(x))
    return res


# ---------------------------------------------------- decode attention ----

def attn_decode_workspace_bytes(num_q_heads: int, num_kv_heads: int, num_tokens: int, head_dim: int) -> int:
    b = ctypes.c_size_t()
    _lib.call("kvq_attn_decode_workspace_bytes", num_q_heads, num_kv_heads, num_tokens, head_dim, ctypes.byref(b))
    return b.value


def attn_decode_int8(q: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, v_codes: torch.Tensor,
                     v_scales: torch.Tensor, softmax_scale: float = None, out: torch.Tensor = None,
                     use_workspace: bool = True) -> torch.Tensor:
    """q fp32 [Hq, D]; k/v codes int8 [T, Hkv, D]; k/v scales fp32 [T, Hkv]
    -> out fp32 [Hq, D] (softmax_scale defaults to 1/sqrt(D))."""
    hq, d = q.shape
    t, hkv, dk = k_codes.shape
    if dk != d or tuple(v_codes.shape) != (t, hkv, d):
        raise ValueError("q, k_codes and v_codes shapes do not match")
    if tuple(k_scales.shape) != (t, hkv) or tuple(v_scales.shape) != (t, hkv):
        raise ValueError("scales must be [T, Hkv]")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    o = _empty((hq, d), torch.float32, q) if out is None else out
    stream = _stream(q)
    ws_ptr, ws_bytes = 0, 0
    if use_workspace:
        ws_bytes = attn_decode_workspace_bytes(hq, hkv, t, d)
        if ws_bytes:
            ws_ptr = workspace(q.device, ws_bytes, stream).data_ptr()
    _lib.call("kvq_attn_decode_int8", _dev(q, torch.float32, "q"), hq, hkv, t, d,
              _dev(k_codes, torch.int8, "k_codes"), _dev(k_scales, torch.float32, "k_scales"),
              _dev(v_codes, torch.int8, "v_codes"), _dev(v_scales, torch.float32, "v_scales"), scale,
              _dev(o, torch.float32, "out"), ws_ptr, ws_bytes, stream)
    return o


def attn_decode_int4(q: torch.Tensor, group_size: int, k_packed: torch.Tensor, k_scales: torch.Tensor,
                     k_zeros: torch.Tensor, v_packed: torch.Tensor, v_scales: torch.Tensor, v_zeros: torch.Tensor,
                     softmax_scale: float = None, out: torch.Tensor = None, use_workspace: bool = True) -> torch.Tensor:
    """q fp32 [Hq, D]; k/v packed uint8 [T, Hkv, D/2]; k/v scales and zeros
    fp32 [T, Hkv, D/group_size] -> out fp32 [Hq, D]."""
    hq, d = q.shape
    t, hkv, half = k_packed.shape
    ng = d // group_size if group_size else 0
    if half * 2 != d or tuple(v_packed.shape) != (t, hkv, half):
        raise ValueError("q, k_packed and v_packed shapes do not match")
    for a in (k_scales, k_zeros, v_scales, v_zeros):
        if tuple(a.shape) != (t, hkv, ng):
            raise ValueError("scales and zeros must be [T, Hkv, D/group_size]")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    o = _empty((hq, d), torch.float32, q) if out is None else out
    stream = _stream(q)
    ws_ptr, ws_bytes = 0, 0
    if use_workspace:
        ws_bytes = attn_decode_workspace_bytes(hq, hkv, t, d)
        if ws_bytes:
            ws_ptr = workspace(q.device, ws_bytes, stream).data_ptr()
    f = lambda a, n: _dev(a, torch.float32, n)
    _lib.call("kvq_attn_decode_int4", _dev(q, torch.float32, "q"), hq, hkv, t, d, group_size,
              _dev(k_packed, torch.uint8, "k_packed"), f(k_scales, "k_scales"), f(k_zeros, "k_zeros"),
              _dev(v_packed, torch.uint8, "v_packed"), f(v_scales, "v_scales"), f(v_zeros, "v_zeros"), scale,
              _dev(o, torch.float32, "out"), ws_ptr, ws_bytes, stream)
    return o


def attn_decode_varlen_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, max_seq_tokens: int,
                                       head_dim: int) -> int:
    b = ctypes.c_size_t()
    _lib.call("kvq_attn_decode_varlen_workspace_bytes", batch, num_q_heads, num_kv_heads, max_seq_tokens, head_dim,
              ctypes.byref(b))
    return b.value


def _varlen_common(q, seq_start, softmax_scale, out):
    bsz, hq, d = q.shape
    if seq_start.dtype not in (torch.int32, torch.uint32) or tuple(seq_start.shape) != (bsz + 1,):
        raise ValueError("seq_start must be int32/uint32 [batch + 1]")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    o = _empty((bsz, hq, d), torch.float32, q) if out is None else out
    return bsz, hq, d, scale, o


def attn_decode_int8_varlen(q: torch.Tensor, seq_start: torch.Tensor, max_seq_tokens: int, k_codes: torch.Tensor,
                            k_scales: torch.Tensor, v_codes: torch.Tensor, v_scales: torch.Tensor,
                            softmax_scale: float = None, out: torch.Tensor = None,
                            use_workspace: bool = True) -> torch.Tensor:
    """q fp32 [B, Hq, D]; seq_start device int32 [B + 1]; k/v codes int8
    [T_total, Hkv, D], scales fp32 [T_total, Hkv] -> out fp32 [B, Hq, D]."""
    t, hkv, d = k_codes.shape
    bsz, hq, d, scale, o = _varlen_common(q, seq_start, softmax_scale, out)
    stream = _stream(q)
    ws_ptr, ws_bytes = 0, 0
    if use_workspace:
        ws_bytes = attn_decode_varlen_workspace_bytes(bsz, hq, hkv, max_seq_tokens, d)
        if ws_bytes:
            ws_ptr = workspace(q.device, ws_bytes, stream).data_ptr()
    _lib.call("kvq_attn_decode_int8_varlen", _dev(q, torch.float32, "q"), bsz, hq, hkv, d,
              _dev(seq_start, seq_start.dtype, "seq_start"), t, max_seq_tokens,
              _dev(k_codes, torch.int8, "k_codes"), _dev(k_scales, torch.float32, "k_scales"),
              _dev(v_codes, torch.int8, "v_codes"), _dev(v_scales, torch.float32, "v_scales"), scale,
              _dev(o, torch.float32, "out"), ws_ptr, ws_bytes, stream)
    return o


def attn_decode_int4_varlen(q: torch.Tensor, seq_start: torch.Tensor, max_seq_tokens: int, group_size: int,
                            k_packed: torch.Tensor, k_scales: torch.Tensor, k_zeros: torch.Tensor,
                            v_packed: torch.Tensor, v_scales: torch.Tensor, v_zeros: torch.Tensor,
                            softmax_scale: float = None, out: torch.Tensor = None,
                            use_workspace: bool = True) -> torch.Tensor:
    """q fp32 [B, Hq, D]; seq_start device int32 [B + 1]; k/v packed uint8
    [T_total, Hkv, D/2], scales and zeros fp32 [T_total, Hkv, D/group_size]."""
    t, hkv, half = k_packed.shape
    bsz, hq, d, scale, o = _varlen_common(q, seq_start, softmax_scale, out)
    stream = _stream(q)
    ws_ptr, ws_bytes = 0, 0
    if use_workspace:
        ws_bytes = attn_decode_varlen_workspace_bytes(bsz, hq, hkv, max_seq_tokens, d)
        if ws_bytes:
            ws_ptr = workspace(q.device, ws_bytes, stream).data_ptr()
    f = lambda a, n: _dev(a, torch.float32, n)
    _lib.call("kvq_attn_decode_int4_varlen", _dev(q, torch.float32, "q"), bsz, hq, hkv, d, group_size,
              _dev(seq_start, seq_start.dtype, "seq_start"), t, max_seq_tokens,
              _dev(k_packed, torch.uint8, "k_packed"), f(k_scales, "k_scales"), f(k_zeros, "k_zeros"),
              _dev(v_packed, torch.uint8, "v_packed"), f(v_scales, "v_scales"), f(v_zeros, "v_zeros"), scale,
              _dev(o, torch.float32, "out"), ws_ptr, ws_bytes, stream)
    return o


# ---------------------------------------------------------- measurement ----

def stream_read(buf: torch.Tensor, nbytes: int, sink: torch.Tensor) -> None:
    """Read nbytes of buf on the device (the empirical read ceiling)."""
    if not buf.is_cuda or not buf.is_contiguous() or buf.numel() * buf.element_size() < nbytes:
        raise ValueError("buf must be a contiguous device tensor of at least nbytes")
    _lib.call("kvq_stream_read", buf.data_ptr(), nbytes, _dev(sink, torch.int32, "sink"), _stream(buf))
