"""Workload for HBM-traffic counters (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE).

Runs, each 5 times: a plain device copy of COPY_MIB MiB (calibration: its
FETCH_SIZE and WRITE_SIZE per dispatch should read COPY_MIB MiB), and the
dominant call of the benchmark step, the 128x128 block-scaled W8A8 GEMM at
M=256, K=14336, N=4096 (w8a8_wide + w8a8_reduce), on rotating weight copies
so that every call reads its weights from HBM.
"""
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from kv_quantization_amd import api, synth  # noqa: E402

COPY_MIB = 256


def main():
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    src = torch.empty(COPY_MIB << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    down = synth.w8a8_down(seed=4)
    seg = [api.weight_quant(dev(w), api.BLK128) for w in down.weights]
    weights = [api.W8a8Weight(api.BLK128, [tuple(t.clone() for t in s) for s in seg]) for _ in range(5)]
    x = dev(down.x_bf16.view(np.int16)).view(torch.bfloat16)
    q, sa = api.act_quant(x[:256], 14336, api.BLK128, True)
    for w in weights:
        api.gemv(q, sa, w)
    torch.cuda.synchronize()
    print("done", flush=True)


if __name__ == "__main__":
    main()
