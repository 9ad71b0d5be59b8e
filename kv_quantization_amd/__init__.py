"""kv_quantization_amd: quantized-decode kernels for AMD MI355X (gfx950).

The compute lives in libkvq.so (hand-written HIP, C ABI in include/kvq.h);
this package is its thin Python binding over torch device memory and streams.

    from kv_quantization_amd import api
    codes, scales = api.quant_int8_token(x)          # KV cache INT8 per token
    packed, s, z = api.quant_int4_group(x, 32)       # KV cache INT4 per group
    q, sa = api.act_quant(x_bf16, kind=api.ROWSCALE) # W8A8 activation quant
    out = api.gemv(q, sa, api.W8a8Weight(...))       # W8A8 FP8 GEMV/GEMM
    q, k, v = api.int4_awq_qkv(x, projs, 128)        # INT4 AWQ fused QKV
"""
from ._lib import KvqError, load  # noqa: F401

__all__ = ["load", "KvqError", "api", "synth", "build"]
