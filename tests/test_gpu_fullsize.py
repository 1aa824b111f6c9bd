"""Parity at the full workload sizes, with the kernels launched as the
benchmark launches them (automatic dispatch). Where the oracle cannot
afford every output, it checks seeded samples of rows/columns."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    return gu.lib_or_skip()


def quant_full(w4, cfg, layer, G):
    W = workloads.weight_bits(cfg, layer)
    gu.log(f"full quantize config={cfg} layer={layer} shape={W.shape} G={G}")
    cd, sd, zd = w4.quantize_int4_grouped(gu.to_dev_bf16(W), G)
    torch.cuda.synchronize()
    ref = oracle.quantize_ref(W, G)
    gu.assert_quant_equal((cd.cpu().numpy(), gu.to_host_bits(sd), gu.to_host_bits(zd)), ref,
                          f"config {cfg} {layer}")
    return (cd, sd, zd), ref


@pytest.mark.parametrize("layer", sorted(workloads.LLAMA3_8B))
def test_llama3_8b_decode_m1(w4, layer):
    N, K = workloads.LLAMA3_8B[layer]
    (cd, sd, zd), (c, s, z) = quant_full(w4, 2, layer, 128)
    x = workloads.activation_bits(2, 1, K)
    y = w4.w4a16_linear(gu.to_dev_bf16(x), cd, sd, zd, 128)
    torch.cuda.synchronize()
    y_ref = oracle.linear_ref(x, c, s, z, 128)
    gu.check_linear(gu.to_host_bits(y), y_ref, gu.abs_bound(x, c, s, z, 128),
                    what=f"llama {layer} M=1", strict=True)


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("layer", sorted(workloads.LLAMA3_8B))
def test_llama3_8b_m16_outliers(w4, layer, G):
    N, K = workloads.LLAMA3_8B[layer]
    (cd, sd, zd), (c, s, z) = quant_full(w4, 3, layer, G)
    x = workloads.activation_bits(3, 16, K)
    y = w4.w4a16_linear(gu.to_dev_bf16(x), cd, sd, zd, G)
    torch.cuda.synchronize()
    y_ref = oracle.linear_ref(x, c, s, z, G)
    gu.check_linear(gu.to_host_bits(y), y_ref, gu.abs_bound(x, c, s, z, G),
                    what=f"llama {layer} M=16 G={G}", strict=True)


@pytest.mark.parametrize("layer", ["o", "down"])
def test_llama3_8b_fake_quant_g32(w4, layer):
    W = workloads.weight_bits(2, layer)
    gu.log(f"full fake quant layer={layer} shape={W.shape} G=32")
    got = gu.to_host_bits(w4.fake_quant_int4_grouped(gu.to_dev_bf16(W), 32))
    torch.cuda.synchronize()
    ref = oracle.fake_quant_ref(W, 32)
    assert np.array_equal(got, ref), f"{layer}: {int((got != ref).sum())} elements differ"


@pytest.mark.parametrize("M", [1, 4])
@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("layer", sorted(workloads.LLAMA3_8B))
def test_llama3_8b_small_m_repeat(w4, layer, G, M):
    # Several (tile, K segment) items per wave on the wide layers; two calls
    # must agree bit for bit (a register hazard once made them differ) and
    # match the oracle.
    N, K = workloads.LLAMA3_8B[layer]
    (cd, sd, zd), (c, s, z) = quant_full(w4, 2, layer, G)
    x = workloads.activation_bits(5, M, K)
    xd = gu.to_dev_bf16(x)
    y1 = w4.w4a16_linear(xd, cd, sd, zd, G)
    y2 = w4.w4a16_linear(xd, cd, sd, zd, G)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), f"llama {layer} M={M} G={G}: two calls differ"
    y_ref = oracle.linear_ref(x, c, s, z, G)
    gu.check_linear(gu.to_host_bits(y1), y_ref, gu.abs_bound(x, c, s, z, G),
                    what=f"llama {layer} M={M} G={G}", strict=True)


@pytest.mark.parametrize("layer", sorted(workloads.GEMMA3_12B))
def test_gemma3_12b_prefill_m2048(w4, layer):
    N, K = workloads.GEMMA3_12B[layer]
    (cd, sd, zd), (c, s, z) = quant_full(w4, 4, layer, 128)
    x = workloads.activation_bits(4, 2048, K)
    y = w4.w4a16_linear(gu.to_dev_bf16(x), cd, sd, zd, 128)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, 1, 127, 128, 1023, 2047,
                           np.random.default_rng(N + K).integers(0, 2048, 10)])
    y_ref = oracle.linear_rows_ref(x, rows, c, s, z, 128)
    yb = gu.to_host_bits(y)[rows]
    gu.check_linear(yb, y_ref, gu.abs_bound(x, c, s, z, 128, rows=rows),
                    what=f"gemma {layer} M=2048 rows {len(rows)}", strict=True)


@pytest.fixture(scope="module")
def square(w4):
    N, K, G = 32768, 32768, 64
    W = workloads.weight_bits(5, "square")
    gu.log("square 32768^2: quantize on the GPU")
    Wd = gu.to_dev_bf16(W)
    cd, sd, zd = w4.quantize_int4_grouped(Wd, G)
    torch.cuda.synchronize()
    del Wd
    # oracle on three seeded row blocks (first, a middle one, last)
    blocks = [(0, 256), (16384 + 512, 16384 + 768), (N - 256, N)]
    refs = [oracle.quantize_ref(W[a:b], G) for a, b in blocks]
    return dict(W=W, dev=(cd, sd, zd), blocks=blocks, refs=refs, G=G, K=K)


def test_square_quantize_sampled_rows(w4, square):
    cd, sd, zd = square["dev"]
    for (a, b), ref in zip(square["blocks"], square["refs"]):
        got = (cd[a:b].cpu().numpy(), gu.to_host_bits(sd[a:b]), gu.to_host_bits(zd[a:b]))
        gu.assert_quant_equal(got, ref, f"square rows {a}:{b}")


def test_square_quantize_all_rows(w4, square):
    """The whole 32768 x 32768 quantize pass against the oracle, bit for bit,
    in blocks of 1024 rows on the host's cores."""
    import concurrent.futures
    cd, sd, zd = square["dev"]
    W, G = square["W"], square["G"]
    got_c, got_s, got_z = cd.cpu().numpy(), gu.to_host_bits(sd), gu.to_host_bits(zd)
    N = W.shape[0]
    step = 1024

    def block(a):
        ref = oracle.quantize_ref(W[a:a + step], G)
        gu.assert_quant_equal((got_c[a:a + step], got_s[a:a + step], got_z[a:a + step]), ref,
                              f"square rows {a}:{a + step}")
        return a

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        for i, a in enumerate(ex.map(block, range(0, N, step))):
            if i % 8 == 7:
                gu.log(f"square quantize: rows below {a + step} match")


def _square_cols(square):
    cols = np.concatenate([np.arange(a, b) for a, b in square["blocks"]])
    c = np.concatenate([r[0] for r in square["refs"]])
    s = np.concatenate([r[1] for r in square["refs"]])
    z = np.concatenate([r[2] for r in square["refs"]])
    return cols, c, s, z


def test_square_m1(w4, square):
    cd, sd, zd = square["dev"]
    K, G = square["K"], square["G"]
    x = workloads.activation_bits(5, 1, K)
    gu.log("square M=1 linear")
    y = w4.w4a16_linear(gu.to_dev_bf16(x), cd, sd, zd, G)
    torch.cuda.synchronize()
    cols, c, s, z = _square_cols(square)
    y_ref = oracle.linear_ref(x, c, s, z, G)
    gu.check_linear(gu.to_host_bits(y)[:, cols], y_ref, gu.abs_bound(x, c, s, z, G),
                    what="square M=1 sampled columns", strict=True)


def test_square_m32768(w4, square):
    cd, sd, zd = square["dev"]
    K, G = square["K"], square["G"]
    M = 32768
    x = workloads.activation_bits(5, M, K)
    gu.log("square M=32768 linear")
    y = w4.w4a16_linear(gu.to_dev_bf16(x), cd, sd, zd, G)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, 255, 256, 16383, M - 1,
                           np.random.default_rng(77).integers(0, M, 3)])
    cols, c, s, z = _square_cols(square)
    y_ref = oracle.linear_ref(x[rows], c, s, z, G)
    yb = gu.to_host_bits(y)[np.ix_(rows, cols)]
    gu.check_linear(yb, y_ref, gu.abs_bound(x[rows], c, s, z, G),
                    what="square M=32768 sampled rows/columns", strict=True)
