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
