"""Seeded random shapes through every path, against the oracle: the
quantizer bit-exact, the linear on the plain and pre-shuffled layouts
(automatic dispatch and both forced kernels) within the accuracy bar, with
guard bands around every output. The shapes are drawn once from a fixed
seed: ragged N and M, K any multiple of G, with and without bias."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _cases(n=40, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([32, 64, 128]))
        K = G * int(rng.integers(1, 8192 // G + 8))
        N = int(rng.integers(1, 700))
        M = int(rng.choice([1, 2, 3, int(rng.integers(4, 17)), int(rng.integers(17, 300))]))
        path = ["AUTO", "GEMV", "GEMM"][i % 3]
        if path == "GEMV" and M > 16:
            path = "AUTO"
        out.append((i, M, N, K, G, path, bool(rng.integers(0, 2))))
    return out


@pytest.fixture(scope="module")
def w4():
    return gu.lib_or_skip()


@pytest.mark.parametrize("i,M,N,K,G,path,bias", _cases())
def test_random_shape(w4, i, M, N, K, G, path, bias):
    seed = 1000 + i
    W = workloads.random_bf16((N, K), 0.02, seed)
    x = workloads.random_bf16((M, K), 1.0, seed + 1)
    b = workloads.random_bf16((1, N), 1.0, seed + 2)[0] if bias else None
    gu.log(f"random case {i}: M={M} N={N} K={K} G={G} path={path} bias={bias}")
    ref = oracle.quantize_ref(W, G)
    cd, sd, zd = w4.quantize_int4_grouped(gu.to_dev_bf16(W), G)
    gu.assert_quant_equal((cd.cpu().numpy(), gu.to_host_bits(sd), gu.to_host_bits(zd)), ref,
                          f"quantize case {i}")
    codes, s, z = ref
    y_ref = oracle.linear_ref(x, codes, s, z, G, b)
    bound = gu.abs_bound(x, codes, s, z, G)
    p = getattr(w4.W4Path, path)
    bd = gu.to_dev_bf16(b) if bias else None
    y = gu.Guarded((M, N), torch.bfloat16)
    w4.w4a16_linear(gu.to_dev_bf16(x), cd, sd, zd, G, bias=bd, out=y.tensor, path=p)
    torch.cuda.synchronize()
    y.check_guards()
    gu.check_linear(gu.to_host_bits(y.tensor), y_ref, bound, what=f"plain case {i}")
    cp, sz = w4.repack_int4_preshuffled(cd, sd, zd, G)
    yp = gu.Guarded((M, N), torch.bfloat16)
    w4.w4a16_linear_preshuffled(gu.to_dev_bf16(x), cp, sz, G, bias=bd, out=yp.tensor, path=p)
    torch.cuda.synchronize()
    yp.check_guards()
    gu.check_linear(gu.to_host_bits(yp.tensor), y_ref, bound, what=f"pre-shuffled case {i}")
