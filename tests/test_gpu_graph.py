"""The library's launches captured in a HIP graph: every replay, with eager
work and synchronisations in between, equals the eager result bit for bit.
(The kernels enqueue no memset nodes; this checks capture and replay.)"""
import numpy as np
import pytest
import torch

import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    return gu.lib_or_skip()


@pytest.mark.parametrize("G,M", [(128, 1), (64, 16), (32, 200)])
def test_graph_replays_match_eager(w4, G, M):
    N, K = 320, 1024 + 128
    W = gu.to_dev_bf16(workloads.random_bf16((N, K), 0.02, G + M))
    x = gu.to_dev_bf16(workloads.random_bf16((M, K), 1.0, G + M + 1))
    c_e, s_e, z_e = w4.quantize_int4_grouped(W, G)
    y_e = w4.w4a16_linear(x, c_e, s_e, z_e, G)
    torch.cuda.synchronize()
    ref = [t.view(torch.uint8).cpu().numpy().copy() for t in (c_e, s_e, z_e, y_e)]

    c = torch.empty_like(c_e)
    s = torch.empty_like(s_e)
    z = torch.empty_like(z_e)
    y = torch.empty_like(y_e)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        w4.quantize_int4_grouped(W, G, c, s, z)
        w4.w4a16_linear(x, c, s, z, G, out=y)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (c, s, z, y):
            t.view(torch.uint8).fill_(0xEE)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.view(torch.uint8).cpu().numpy() for t in (c, s, z, y)]
        for a, b, name in zip(got, ref, ("codes", "scales", "zeros", "y")):
            assert np.array_equal(a, b), f"replay {rep}: {name} differs from eager"


def _replays_equal(g, outs, ref, names):
    for rep in range(4):
        for t in outs:
            t.view(torch.uint8).fill_(0xEE)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, b, name in zip(outs, ref, names):
            assert np.array_equal(t.view(torch.uint8).cpu().numpy(), b), \
                f"replay {rep}: {name} differs from eager"


@pytest.mark.parametrize("G,M", [(128, 1), (32, 16), (64, 200)])
def test_graph_int8_weight_only(w4, G, M):
    N, K = 320, 1024 + 128
    W = gu.to_dev_bf16(workloads.random_bf16((N, K), 0.02, 7 * G + M))
    x = gu.to_dev_bf16(workloads.random_bf16((M, K), 1.0, 7 * G + M + 1))
    q_e, s_e = w4.quantize_int8_grouped(W, G)
    y_e = w4.w8a16_linear(x, q_e, s_e, G)
    torch.cuda.synchronize()
    ref = [t.view(torch.uint8).cpu().numpy().copy() for t in (q_e, s_e, y_e)]
    q, s, y = torch.empty_like(q_e), torch.empty_like(s_e), torch.empty_like(y_e)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        w4.quantize_int8_grouped(W, G, q, s)
        w4.w8a16_linear(x, q, s, G, out=y)
    torch.cuda.synchronize()
    _replays_equal(g, (q, s, y), ref, ("codes8", "scales", "y"))


@pytest.mark.parametrize("G", [128, 32])
def test_graph_w4a8_and_preshuffled(w4, G):
    N, K, M = 320, 1024 + 128, 130
    W = gu.to_dev_bf16(workloads.random_bf16((N, K), 0.02, 11 * G))
    x = gu.to_dev_bf16(workloads.random_bf16((M, K), 1.0, 11 * G + 1))
    c, s, z = w4.quantize_int4_grouped(W, G)
    x8_e, sx_e = w4.quantize_act_int8(x)
    y8_e = w4.w4a8_linear(x8_e, sx_e, c, s, z, G)
    cp_e, sz_e = w4.repack_int4_preshuffled(c, s, z, G)
    yp_e = w4.w4a16_linear_preshuffled(x, cp_e, sz_e, G)
    torch.cuda.synchronize()
    outs_e = (x8_e, sx_e, y8_e, cp_e, sz_e, yp_e)
    ref = [t.view(torch.uint8).cpu().numpy().copy() for t in outs_e]
    x8, sx, y8, cp, sz, yp = (torch.empty_like(t) for t in outs_e)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        w4.quantize_act_int8(x, x8=x8, sx=sx)
        w4.w4a8_linear(x8, sx, c, s, z, G, out=y8)
        w4.repack_int4_preshuffled(c, s, z, G, codes_ps=cp, sz=sz)
        w4.w4a16_linear_preshuffled(x, cp, sz, G, out=yp)
    torch.cuda.synchronize()
    _replays_equal(g, (x8, sx, y8, cp, sz, yp), ref, ("x8", "sx", "y_w4a8", "codes_ps", "sz", "y_ps"))
