"""GPU: the binding's per-stream workspace cache under HIP graph capture and
with two streams.  Split-K calls (INT4 AWQ exchanges partial tiles and
counters through the workspace, the W8A8 GEMM above 32 rows writes partial
sums into it) must give the oracle's results when a captured graph is
replayed after the cache has moved to a larger buffer, and when two streams
each run their own calls at the same time."""
import numpy as np
import pytest
import torch

from conftest import print_case
from gpu_util import dev, host
from kv_quantization_amd import api, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _bind_oracle(oracle_mod):
    global _oracle
    _oracle = oracle_mod


def _awq_inputs(m, seed):
    x, projs = synth.int4_awq(m, 1024, (256, 64, 64), 128, seed=seed)
    dp = [(dev(p.qweight.view(np.int32)), dev(p.scales), dev(p.zeros)) for p in projs]
    refs = _oracle.int4_awq_qkv(x, [(p.qweight, p.scales, p.zeros) for p in projs], 128)
    return dev(x), dp, refs


def _awq_ok(outs, refs, what):
    for o, (r, b) in zip(outs, refs):
        err = np.abs(host(o).astype(np.float64) - r)
        assert np.all(err <= 1e-3 * b), what


def _w8a8_inputs(rows, seed):
    inp = synth.w8a8(rows, 512, (256, 128, 128), seed=seed)
    q, sa = _oracle.act_quant(0, inp.x_bf16, 512)
    segs = [_oracle.weight_quant(0, w) for w in inp.weights]
    ref, bound = _oracle.w8a8_gemv(0, q, sa, segs)
    weight = api.W8a8Weight(0, [(dev(c), dev(s)) for c, s in segs])
    return dev(q), dev(sa), weight, ref, bound


def _w8a8_ok(out, ref, bound, what):
    got = _oracle.bf16_to_f32(host(out)).astype(np.float64)
    half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 8)
    assert np.all(np.abs(got - ref) <= 1e-3 * bound + half_ulp), what


def test_graph_replay_after_the_workspace_grows():
    print_case("workspace: graph replay after growth")
    s = torch.cuda.Stream()
    x1, p1, r1 = _awq_inputs(1, 901)
    outs1 = [torch.empty((1, n), dtype=torch.float32, device="cuda") for n in (256, 64, 64)]
    with torch.cuda.stream(s):
        api.int4_awq_qkv(x1, p1, 128, outs=outs1)           # eager: creates the stream's small workspace
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            api.int4_awq_qkv(x1, p1, 128, outs=outs1)
    torch.cuda.synchronize()
    # a call that needs a larger workspace on the same stream: the cache moves
    q, sa, weight, ref, bound = _w8a8_inputs(200, 902)
    with torch.cuda.stream(s):
        out = api.gemv(q, sa, weight)
    torch.cuda.synchronize()
    _w8a8_ok(out, ref, bound, "eager W8A8 after growth")
    for i in range(3):
        for o in outs1:
            o.fill_(float("nan"))
        with torch.cuda.stream(s):
            g.replay()
            out2 = api.gemv(q, sa, weight)                   # eager work between replays
        torch.cuda.synchronize()
        _awq_ok(outs1, r1, f"replay {i} of the graph captured before growth")
        _w8a8_ok(out2, ref, bound, f"eager W8A8 after replay {i}")


def test_capture_refuses_to_create_a_workspace():
    print_case("workspace: capture without a prior eager call")
    s = torch.cuda.Stream()
    x1, p1, _ = _awq_inputs(1, 903)
    g = torch.cuda.CUDAGraph()
    with pytest.raises(RuntimeError, match="graph capture"):
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                api.int4_awq_qkv(x1, p1, 128)
    torch.cuda.synchronize()


def test_two_streams_run_split_k_calls_together():
    print_case("workspace: two streams")
    a = _awq_inputs(16, 904)
    b = _awq_inputs(1, 905)
    wa = _w8a8_inputs(100, 906)
    wb = _w8a8_inputs(64, 907)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for it in range(3):
        with torch.cuda.stream(s1):
            oa = api.int4_awq_qkv(a[0], a[1], 128)
            ga = api.gemv(wa[0], wa[1], wa[2])
        with torch.cuda.stream(s2):
            ob = api.int4_awq_qkv(b[0], b[1], 128)
            gb = api.gemv(wb[0], wb[1], wb[2])
        torch.cuda.synchronize()
        _awq_ok(oa, a[2], f"stream 1 INT4, pass {it}")
        _awq_ok(ob, b[2], f"stream 2 INT4, pass {it}")
        _w8a8_ok(ga, wa[3], wa[4], f"stream 1 W8A8, pass {it}")
        _w8a8_ok(gb, wb[3], wb[4], f"stream 2 W8A8, pass {it}")
