"""The measurement helper (streaming read) runs through the C ABI, rejects
bad sizes on the host and writes nothing for ordinary data."""
import pytest
import torch

from conftest import print_case
from kv_quantization_amd import _lib, api

pytestmark = pytest.mark.gpu


def test_stream_read_runs_and_leaves_sink():
    print_case("stream read")
    buf = torch.randint(0, 255, (64 << 20,), dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for n in (16, 4096, 1 << 20, (64 << 20) - 16, 64 << 20):
        api.stream_read(buf, n, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    with pytest.raises(_lib.KvqError):
        api.stream_read(buf, 17, sink)
