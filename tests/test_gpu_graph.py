"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph):
they launch kernels only -- no allocation, memset or host synchronisation --
so a serving loop can capture them once and replay them.  The graph holds
the fused NVFP4 quantize (4/6 + dequant, and a ragged group range), the
standalone dequant and the MXFP4 Rollout-ResQ call; it is replayed several
times, each time after eager work that writes a new input into the captured
buffer, and every replay's outputs must equal an eager call's bit for bit
(the first replay is also checked against the oracle)."""
import numpy as np
import pytest
import torch

import fp4_block_quantization_amd as fq
import workloads
from gpuutil import assert_same, bits_of, host, oracle_mx, oracle_nvfp4, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fq.lib()


def _alloc_nv(R, H):
    kw = dict(device="cuda")
    return (torch.empty((R, H // 2), dtype=torch.uint8, **kw),
            torch.empty((R, H // 16), dtype=torch.uint8, **kw),
            torch.empty((R,), dtype=torch.float32, **kw),
            torch.empty((R, H), dtype=torch.bfloat16, **kw))


def _alloc_mx(R, H):
    kw = dict(dtype=torch.uint8, device="cuda")
    return (torch.empty((R, H // 2), **kw), torch.empty((R, H // 32), **kw),
            torch.empty((R, H // 4), **kw), torch.empty((R, H // 8), **kw),
            torch.empty((R, H // 32), **kw))


def test_captured_calls_replay_bit_exact():
    R, H = 96, 7168
    inputs = [workloads.random_rows(100 + i, R, H, dist=1, row_gain_sigma=1.0) for i in range(4)]
    offs = torch.tensor([8, 20, 20, 77], dtype=torch.int64, device="cuda")
    x = to_dev(inputs[0])
    nv, ragged, mx = _alloc_nv(R, H), _alloc_nv(R, H), _alloc_mx(R, H)
    back = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    for t in ragged:
        t.zero_()

    def calls():
        fq.nvfp4_quantize(x, True, out=nv)
        fq.nvfp4_quantize(x, True, offsets=offs, out=ragged)
        fq.nvfp4_dequantize(nv[0], nv[1], nv[2], out=back)
        fq.mxfp4_resq_quantize(x, out=mx)

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    for i, bits in enumerate(inputs + inputs[:1]):
        x.copy_(to_dev(bits))  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        e_nv = fq.nvfp4_quantize(x, True)
        e_mx = fq.mxfp4_resq_quantize(x)
        torch.cuda.synchronize()
        for g, w in zip(nv, e_nv):
            assert torch.equal(g.view(torch.uint8), w.view(torch.uint8)), ("replay", i)
        assert torch.equal(back.view(torch.int16), nv[3].view(torch.int16)), ("dequant", i)
        lo, hi = 8, 77
        for g, w in zip(ragged, e_nv):
            assert torch.equal(g[lo:hi].view(torch.uint8), w[lo:hi].view(torch.uint8)), ("ragged", i)
        for g, w in zip(mx, e_mx):
            assert torch.equal(g, w), ("mx", i)
        if i == 0:
            want = oracle_nvfp4(bits, True)
            assert_same(host(nv[0]), want[0], "graph codes")
            assert_same(host(nv[1]), want[1], "graph block_scales")
            assert_same(host(nv[2])[:, None], want[2][:, None], "graph token_scales")
            assert_same(bits_of(nv[3]), want[3], "graph dequant")
            for g, w in zip(mx, oracle_mx(bits)):
                assert_same(host(g), w, "graph mx")
    # rows outside the ragged range were never written by any replay
    for t in ragged:
        assert (t[:8].view(torch.uint8) == 0).all() and (t[77:].view(torch.uint8) == 0).all()
