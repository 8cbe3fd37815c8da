"""The library's calls inside a captured HIP graph: every path is captured once, replayed
several times with other eager work of the library and synchronizations in between, and
each replay's outputs are compared bit for bit with the same calls run eagerly on the same
inputs. The library allocates nothing and clears its counters with kernels, so a replay
has to reproduce the eager launches exactly; the static quantizer's counter and the
delayed-scaling history are state carried from replay to replay, checked against the eager
sequence of the same steps."""

import pytest
import torch

import fp4_w8a8_quantized_amd as w8
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _x(shape, seed, scale=1.0):
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda:0") * scale).to(torch.bfloat16)


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    a, b = a.contiguous(), b.contiguous()
    return a.dtype == b.dtype and a.shape == b.shape and torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def _capture(fn):
    """Capture fn() on a side stream; returns (graph, outputs captured)."""
    side = torch.cuda.Stream(device="cuda:0")
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            out = fn()
    torch.cuda.synchronize()
    return g, out


def _noise():
    """Eager library work between replays (other shapes, other buffers)."""
    xq, sx = w8.quantize_per_token(_x((64, 1024), 99))
    wq, sw = w8.quantize_weight_per_channel(_x((256, 1024), 98, 0.02))
    w8.gemm(xq, sx, wq, sw)
    torch.cuda.synchronize()


@pytest.mark.parametrize("fmt", ["e4m3fn", "int8"])
@pytest.mark.parametrize("M,N,K", [(300, 1000, 4096), (8, 4096, 4096), (1, 2048, 4096), (2048, 4096, 1024)])
def test_quantize_gemm_in_graph(fmt, M, N, K):
    need_gpu()
    x = _x((M, K), M + N + K)
    wq, sw = w8.quantize_weight_per_channel(_x((N, K), 7, 0.02), fmt)

    def step():
        xq, sx = w8.quantize_per_token(x, fmt)
        y = w8.gemm(xq, sx, wq, sw)
        yl = w8.linear(x, wq, sw)
        return xq, sx, y, yl

    ref = step()
    torch.cuda.synchronize()
    ref = tuple(t.clone() for t in ref)
    g, out = _capture(step)
    for r in range(REPLAYS):
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert _same(a, b), f"replay {r}"
        _noise()


def test_epilogue_fp8_out_in_graph():
    need_gpu()
    M, N, K = 2048, 6144, 4096
    xq, sx = w8.quantize_per_token(_x((M, K), 3))
    wq, sw = w8.quantize_weight_per_channel(_x((N, K), 4, 0.02))
    bias = _x((N,), 5)

    def step():
        return w8.gemm_ex(xq, sx, wq, sw, bias=bias, act="silu", out_scale=0.05)

    ref = step().clone()
    g, out = _capture(step)
    for r in range(REPLAYS):
        g.replay()
        torch.cuda.synchronize()
        assert _same(out, ref), f"replay {r}"
        _noise()


def test_static_quantizer_state_across_replays():
    """The saturation counter and the running amax accumulate over replays exactly as over
    eager calls, and the delayed-scaling update (captured with a fixed step) writes the same
    history slot and scale each time."""
    need_gpu()
    x = _x((512, 4096), 11, 3.0)
    amax0 = float(x.float().abs().max())
    scale = torch.tensor([amax0 / 448.0 / 4], dtype=torch.float32, device="cuda:0")   # saturates
    hist_shape = (4,)

    def run(n, sat, amax, hist, sc):
        outs = []
        for _ in range(n):
            q = w8.quantize_static(x, sc, saturated=sat, amax=amax)
            outs.append(q.clone())
            w8.delayed_scale_update(hist, amax, 2, sc)
        return outs

    # eager reference: REPLAYS + 1 steps from the same start
    def fresh():
        return (torch.zeros((1,), dtype=torch.int32, device="cuda:0"),
                torch.zeros((1,), dtype=torch.float32, device="cuda:0"),
                torch.zeros(hist_shape, dtype=torch.float32, device="cuda:0"),
                scale.clone())

    e_sat, e_amax, e_hist, e_sc = fresh()
    e_q = run(REPLAYS + 1, e_sat, e_amax, e_hist, e_sc)
    torch.cuda.synchronize()

    g_sat, g_amax, g_hist, g_sc = fresh()
    side = torch.cuda.Stream(device="cuda:0")
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            q = w8.quantize_static(x, g_sc, saturated=g_sat, amax=g_amax)
            w8.delayed_scale_update(g_hist, g_amax, 2, g_sc)
    torch.cuda.synchronize()
    # capture does not run the work: reset the state and replay REPLAYS + 1 times
    g_sat.zero_(); g_amax.zero_(); g_hist.zero_(); g_sc.copy_(scale)
    torch.cuda.synchronize()
    for r in range(REPLAYS + 1):
        graph.replay()
        torch.cuda.synchronize()
        assert _same(q, e_q[r]), f"codes, replay {r}"
        _noise()
    assert int(g_sat.item()) == int(e_sat.item()) and int(e_sat.item()) > 0
    assert _same(g_amax, e_amax) and _same(g_hist, e_hist) and _same(g_sc, e_sc)


def test_low_bit_formats_in_graph():
    """Block-scaled FP8, MXFP4, NVFP4 (tensor scale computed: four launches, one of them
    the kernel that clears the amax slot) and W4A16."""
    need_gpu()
    M, N, K = 512, 1024, 2048
    x = _x((M, K), 21)
    w = _x((N, K), 22, 0.02)
    wbq, wbs = w8.quantize_weight_block(w)
    wmq, wms = w8.quantize_mxfp4(w)
    wnq, wns, wng = w8.quantize_nvfp4(w)
    w4q, w4s = w8.quantize_int4(w)

    def step():
        xq, sx = w8.quantize_per_token_group(x)
        yb = w8.gemm_blockscaled(xq, sx, wbq, wbs)
        mq, ms = w8.quantize_mxfp4(x)
        ym = w8.gemm_mxfp4(mq, ms, wmq, wms)
        nq, ns, ng = w8.quantize_nvfp4(x)
        yn = w8.gemm_nvfp4(nq, ns, ng, wnq, wns, wng)
        y4 = w8.gemm_w4a16(x[:8].contiguous(), w4q, w4s)
        return xq, sx, yb, mq, ms, ym, nq, ns, ng, yn, y4

    ref = tuple(t.clone() for t in step())
    torch.cuda.synchronize()
    g, out = _capture(step)
    for r in range(REPLAYS):
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(out, ref)):
            assert _same(a, b), f"output {i}, replay {r}"
        _noise()
