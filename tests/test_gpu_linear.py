"""W4A16 linear on the GPU against the oracle (small seeded shapes that span
several tiles and ragged tails, both kernels, bias, edge cases)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import gpu_util as gu
from tests import pins

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    return gu.lib_or_skip()


def run_case(w4, M, N, K, G, bias, path, seed, wstd=0.02, outliers=False):
    W = workloads.random_bf16((N, K), wstd, seed)
    if outliers:
        cols = workloads.outlier_columns(K, seed)
        W = workloads.normal_bf16_rows(N, K, wstd, seed, outlier_cols=cols)
    x = workloads.random_bf16((M, K), 1.0, seed + 1)
    b = workloads.random_bf16((1, N), 1.0, seed + 2)[0] if bias else None
    codes, s, z = oracle.quantize_ref(W, G)
    gu.log(f"linear M={M} N={N} K={K} G={G} bias={bias} path={path.name} seed={seed}")
    # the GPU quantizes for itself; its output is checked bit-exact first
    Wd = gu.to_dev_bf16(W)
    cd, sd, zd = w4.quantize_int4_grouped(Wd, G)
    gu.assert_quant_equal((cd.cpu().numpy(), gu.to_host_bits(sd), gu.to_host_bits(zd)),
                          (codes, s, z), "quantize")
    y = gu.Guarded((M, N), torch.bfloat16)
    w4.w4a16_linear(gu.to_dev_bf16(x), cd, sd, zd, G,
                    bias=gu.to_dev_bf16(b) if bias else None, out=y.tensor, path=path)
    torch.cuda.synchronize()
    y.check_guards()
    y_ref = oracle.linear_ref(x, codes, s, z, G, b)
    bound = gu.abs_bound(x, codes, s, z, G)
    return gu.check_linear(gu.to_host_bits(y.tensor), y_ref, bound,
                           what=f"M={M} N={N} K={K} G={G}")


def test_tiny_config_auto(w4):
    # nn.Linear(512, 512), group size 32, one input row
    W = workloads.weight_bits(1, "linear")
    x = workloads.activation_bits(1, 1, 512)
    codes, s, z = oracle.quantize_ref(W, 32)
    cd, sd, zd = w4.quantize_int4_grouped(gu.to_dev_bf16(W), 32)
    y = w4.w4a16_linear(gu.to_dev_bf16(x), cd, sd, zd, 32)
    torch.cuda.synchronize()
    y_ref = oracle.linear_ref(x, codes, s, z, 32)
    gu.check_linear(gu.to_host_bits(y), y_ref, gu.abs_bound(x, codes, s, z, 32), what="tiny",
                    strict=True)


GEMV_SHAPES = [(16, 128), (33, 256), (100, 96), (48, 320), (200, 1024), (17, 4096 + 128)]


def _with_groups(cases, groups=(32, 64, 128)):
    """(G, *case) for every group size that divides the case's K (the last
    element of the case)."""
    return [(G, *c) for c in cases for G in groups if c[-1] % G == 0]


@pytest.mark.parametrize("G,M,N,K", _with_groups(
    [(M, N, K) for M in (1, 2, 3, 4, 5, 8, 15, 16) for N, K in GEMV_SHAPES]))
def test_gemv(w4, G, M, N, K):
    run_case(w4, M, N, K, G, bias=(M % 2 == 1), path=gu_path(w4, "GEMV"), seed=N + K + M)


# Edge shapes every path must take: the smallest legal K (one group of 32,
# a single partial chunk), and fewer output rows than one 16-row tile or
# one row group of the M = 1 kernel.
EDGE_CASES = [(M, N, K) for M in (1, 3, 16, 17) for N, K in ((1, 32), (7, 32), (15, 64), (1, 160), (7, 4096))]


@pytest.mark.parametrize("path,G,M,N,K", [
    (path, *c) for c in _with_groups(EDGE_CASES) for path in ("GEMV", "GEMM")
    if path == "GEMM" or c[1] <= 16])           # the GEMV serves M <= 16
def test_edge_shapes(w4, path, G, M, N, K):
    run_case(w4, M, N, K, G, bias=(N % 2 == 1), path=gu_path(w4, path), seed=11 * N + K + M)


# Long rows: x of M rows no longer fits in LDS for the larger M, which
# moves the decode path to the kernels that read x fragments from L2 (K a
# multiple of 128) or stage it in phases (otherwise).
LONG_K_CASES = [(16, 40, 10240, 32), (16, 40, 10240, 64), (16, 40, 10240, 128),
                (16, 40, 10016, 32), (16, 40, 10048, 64), (6, 72, 16384, 128),
                (4, 40, 16512, 128), (2, 24, 32768, 64), (9, 33, 12288, 32),
                # M = 1: x through the per-wave LDS slab once a row spans more
                # than two 2048-wide segments; past 16 segments a wave takes
                # several (K = 40960: 20 segments)
                (1, 40, 10240, 32), (1, 19, 10048, 64), (1, 24, 14336, 128),
                (1, 20, 40960, 64), (1, 9, 6144 + 96, 32),
                # M = 2 on the same kernel: both x rows through the slab, one
                # at a time (K = 36864: 18 segments, so some waves take two)
                (2, 21, 14336, 128), (2, 11, 36864, 128),
                # M = 3, 4 with long rows on the split and direct kernels
                (3, 17, 18432, 32), (4, 20, 40960, 64), (4, 13, 6144 + 64, 64)]


# Two activation rows with a bias: every row of y gets the bias (the other
# parametrisations give odd M the bias), on both x paths of the M <= 2
# kernel (direct loads at K <= 4096, the LDS slab beyond) and both layouts'
# group sizes.
@pytest.mark.parametrize("G,N,K", [(32, 37, 2048), (128, 64, 4096), (64, 21, 10240), (128, 9, 14336)])
def test_gemv_two_rows_with_bias(w4, G, N, K):
    run_case(w4, 2, N, K, G, bias=True, path=gu_path(w4, "GEMV"), seed=3 * N + K)


@pytest.mark.parametrize("M,N,K,G", LONG_K_CASES)
def test_gemv_long_k(w4, M, N, K, G):
    run_case(w4, M, N, K, G, bias=(K % 3 == 1), path=gu_path(w4, "GEMV"), seed=M + N + K)


@pytest.mark.parametrize("K", [1 << 24, (1 << 24) + 128])
def test_auto_dispatch_at_the_gemv_k_limit(w4, K):
    # K = 2^24 is the largest the decode GEMV takes (its waves loop over 8192
    # segments); one group more and AUTO hands the call to the GEMM
    assert w4.GEMV_MAX_K == 1 << 24
    run_case(w4, 1, 8, K, 128, bias=True, path=gu_path(w4, "AUTO"), seed=K % 1000)


GEMM_SHAPES = [(16, 64), (130, 320), (257, 512), (64, 96)]


@pytest.mark.parametrize("G,M,N,K", _with_groups(
    [(M, N, K) for M in (1, 16, 17, 33, 127, 128, 129, 257) for N, K in GEMM_SHAPES]))
def test_gemm(w4, G, M, N, K):
    run_case(w4, M, N, K, G, bias=(M % 2 == 0), path=gu_path(w4, "GEMM"), seed=3 * N + K + M)


# Shapes with enough 128 x 256 tiles to fill a 256-unit chip (at least 240)
# run the eight-wave 128 x 256 GEMM block (G >= 64): ragged M and N, a
# one-column tail, bias on half; the last one has several blocks per unit.
WIDE_SHAPES = [(2000, 4000, 256), (2048, 3840, 384), (2047, 4097, 128), (4000, 2048, 256),
               (3000, 6000, 128)]


@pytest.mark.parametrize("M,N,K", WIDE_SHAPES)
@pytest.mark.parametrize("G", [64, 128])
def test_gemm_wide_blocks(w4, G, M, N, K):
    run_case(w4, M, N, K, G, bias=(N % 2 == 0), path=gu_path(w4, "GEMM"), seed=N + K + G)


# M > 16 on a layer with few output tiles: AUTO runs the decode GEMV on
# 16-row slices (a ragged last slice included, with and without bias).
@pytest.mark.parametrize("M,N,K,G", [(17, 200, 4096, 128), (40, 300, 2048, 32),
                                     (63, 130, 14336, 64), (100, 64, 1024, 128)])
def test_auto_row_slices(w4, M, N, K, G):
    run_case(w4, M, N, K, G, bias=(M % 2 == 1), path=gu_path(w4, "AUTO"), seed=17 * M + N + K)


@pytest.mark.parametrize("M", [1, 16, 40, 300])
@pytest.mark.parametrize("G", [32, 128])
def test_auto_dispatch_outliers(w4, M, G):
    run_case(w4, M, 96, 1024, G, bias=True, path=gu_path(w4, "AUTO"), seed=M * 7 + G,
             outliers=True)


def gu_path(w4, name):
    return getattr(w4.W4Path, name)


def test_zero_input_gives_bias_exactly(w4):
    N, K, G = 40, 256, 64
    W = workloads.random_bf16((N, K), 0.02, 1)
    b = workloads.random_bf16((1, N), 1.0, 2)[0]
    cd, sd, zd = w4.quantize_int4_grouped(gu.to_dev_bf16(W), G)
    for M, path in ((3, w4.W4Path.GEMV), (20, w4.W4Path.GEMM)):
        x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
        y = w4.w4a16_linear(x, cd, sd, zd, G, bias=gu.to_dev_bf16(b), path=path)
        torch.cuda.synchronize()
        assert np.array_equal(gu.to_host_bits(y), np.tile(b, (M, 1)))


def test_constant_groups_are_exact(w4):
    # scale 0 everywhere: w_hat == w, and small-integer data makes y exact
    N, K, G = 24, 256, 32
    rng = np.random.default_rng(3)
    vals = rng.integers(-3, 4, (N, K // G, 1)).repeat(G, axis=2).reshape(N, K)
    W = pins.bf16_from_float(vals.astype(np.float64))
    x = pins.bf16_from_float(rng.integers(-2, 3, (5, K)).astype(np.float64))
    cd, sd, zd = w4.quantize_int4_grouped(gu.to_dev_bf16(W), G)
    assert np.all(gu.to_host_bits(sd) == 0)
    for path in (w4.W4Path.GEMV, w4.W4Path.GEMM):
        y = w4.w4a16_linear(gu.to_dev_bf16(x), cd, sd, zd, G, path=path)
        torch.cuda.synchronize()
        exact = pins.f32_from_bf16(x).astype(np.float64) @ vals.T.astype(np.float64)
        # integer sums are exact in float32; the only rounding is the bf16 store
        assert np.array_equal(gu.to_host_bits(y), pins.bf16_from_float(exact))


def test_m_zero_is_a_no_op(w4):
    N, K, G = 16, 128, 32
    cd, sd, zd = w4.quantize_int4_grouped(
        gu.to_dev_bf16(workloads.random_bf16((N, K), 0.02, 4)), G)
    x = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    y = w4.w4a16_linear(x, cd, sd, zd, G)
    assert y.shape == (0, N)


def test_linear_deterministic(w4):
    N, K, G = 300, 1024, 64
    W = workloads.random_bf16((N, K), 0.02, 9)
    cd, sd, zd = w4.quantize_int4_grouped(gu.to_dev_bf16(W), G)
    for M in (4, 200):
        x = gu.to_dev_bf16(workloads.random_bf16((M, K), 1.0, 10))
        a = gu.to_host_bits(w4.w4a16_linear(x, cd, sd, zd, G))
        b = gu.to_host_bits(w4.w4a16_linear(x, cd, sd, zd, G))
        assert np.array_equal(a, b)
