"""ctypes view of libkvq.so: the C ABI declared in include/kvq.h.

Loading fails loudly when the library has not been built; there is no CPU or
PyTorch fallback anywhere in this package.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libkvq.so"

KVQ_OK, KVQ_E_INVALID, KVQ_E_UNSUPPORTED, KVQ_E_LAUNCH = 0, 1, 2, 3
W8A8_ROWSCALE, W8A8_BLK128 = 0, 1


class W8a8Segment(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("n", ctypes.c_uint32)]


class Int4AwqProj(ctypes.Structure):
    _fields_ = [("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("n", ctypes.c_uint32)]


_p = ctypes.c_void_p
_u32 = ctypes.c_uint32
_u64 = ctypes.c_uint64
_i = ctypes.c_int
_sz = ctypes.c_size_t
_psz = ctypes.POINTER(ctypes.c_size_t)

# name -> argtypes (all return int status, except the two noted)
SIGNATURES = {
    "kvq_quant_int8_token": [_p, _p, _p, _u32, _u32, _p],
    "kvq_dequant_int8_token": [_p, _p, _p, _u32, _u32, _p],
    "kvq_quant_fp8_token": [_p, _p, _p, _u32, _u32, _p],
    "kvq_dequant_fp8_token": [_p, _p, _p, _u32, _u32, _p],
    "kvq_quant_int8_tensor": [_p, _p, _p, _u32, _u32, _p, _sz, _p],
    "kvq_quant_int8_token_dt": [_p, _i, _p, _p, _u32, _u32, _p],
    "kvq_dequant_int8_token_dt": [_p, _p, _p, _i, _u32, _u32, _p],
    "kvq_quant_int4_group_dt": [_p, _i, _p, _p, _p, _u32, _u32, _u32, _p],
    "kvq_dequant_int4_group_dt": [_p, _p, _p, _p, _i, _u32, _u32, _u32, _p],
    "kvq_dequant_int8_tensor": [_p, _p, _p, _u32, _u32, _p],
    "kvq_quant_int4_group": [_p, _p, _p, _p, _u32, _u32, _u32, _p],
    "kvq_dequant_int4_group": [_p, _p, _p, _p, _u32, _u32, _u32, _p],
    "w8a8_act_quant": [_i, _i, _p, _p, _u32, _u32, _u32, _p, _p, _p],
    "w8a8_scratch_bytes": [_i, _u32, _u32, _psz, _psz],
    "w8a8_gemv": [_i, _p, _p, _u32, _u32, ctypes.POINTER(W8a8Segment), _u32, _p, _u32, _p, _sz, _p],
    "w8a8_gemv_workspace_bytes": [_i, _u32, _u32, _u32, _psz],
    "w8a8_proj": [_i, _i, _p, _p, _u32, _u32, _u32, ctypes.POINTER(W8a8Segment), _u32, _p, _u32, _p, _p, _p,
                  _sz, _p],
    "w8a8_weight_quant": [_i, _p, _u32, _u32, _p, _p, _p],
    "kvq_f32_to_e4m3": [_p, _p, _u64, _p],
    "int4_awq_qkv_gemm": [_p, _u32, _u32, _u32, ctypes.POINTER(Int4AwqProj), ctypes.POINTER(Int4AwqProj),
                          ctypes.POINTER(Int4AwqProj), _p, _sz, _p],
    "int4_awq_workspace_bytes": [_u32, _u32, _u32, _u32, _psz],
    "int4_awq_qkv_gemm_dt": [_p, _i, _u32, _u32, _u32, ctypes.POINTER(Int4AwqProj), ctypes.POINTER(Int4AwqProj),
                             ctypes.POINTER(Int4AwqProj), _p, _sz, _p],
    "int4_awq_qkv_gemm_noalloc": [_p, _u32, _u32, _u32, ctypes.POINTER(Int4AwqProj), ctypes.POINTER(Int4AwqProj),
                                  ctypes.POINTER(Int4AwqProj), _p],
    "kvq_stream_read": [_p, _sz, _p, _p],
    "kvq_attn_decode_int8": [_p, _u32, _u32, _u32, _u32, _p, _p, _p, _p, ctypes.c_float, _p, _p, _sz, _p],
    "kvq_attn_decode_workspace_bytes": [_u32, _u32, _u32, _u32, _psz],
    "kvq_attn_decode_varlen_workspace_bytes": [_u32, _u32, _u32, _u32, _u32, _psz],
    "kvq_attn_decode_int8_varlen": [_p, _u32, _u32, _u32, _u32, _p, _u32, _u32, _p, _p, _p, _p, ctypes.c_float, _p,
                                    _p, _sz, _p],
    "kvq_attn_decode_int4_varlen": [_p, _u32, _u32, _u32, _u32, _u32, _p, _u32, _u32, _p, _p, _p, _p, _p, _p,
                                    ctypes.c_float, _p, _p, _sz, _p],
    "kvq_attn_decode_int4": [_p, _u32, _u32, _u32, _u32, _u32, _p, _p, _p, _p, _p, _p, ctypes.c_float, _p, _p, _sz,
                             _p],
}

# include/kvq.h: KVQ_INT8_TENSOR_WORKSPACE_BYTES (counter area + 512 partials)
INT8_TENSOR_WORKSPACE_BYTES = 4096 + 2048
# include/kvq.h: KVQ_INT4_NOALLOC_SCRATCH_BYTES (the library's own scratch per GPU)
INT4_NOALLOC_SCRATCH_BYTES = 4 << 20

_lib = None


def load() -> ctypes.CDLL:
    """Load libkvq.so (built by kv_quantization_amd.build) and bind every symbol."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise ImportError(f"{LIB_PATH} is missing: build it with `python kv_quantization_amd/build.py` "
                          "(hipcc, gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(str(LIB_PATH))
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.kvq_last_error.argtypes = []
    lib.kvq_last_error.restype = ctypes.c_char_p
    lib.kvq_abi_version.argtypes = []
    lib.kvq_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


class KvqError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} -> status {status}: {msg}")
        self.status = status


def check(status: int, fn: str) -> None:
    if status != KVQ_OK:
        raise KvqError(status, fn, load().kvq_last_error().decode())


def call(name: str, *args) -> None:
    check(getattr(load(), name)(*args), name)
