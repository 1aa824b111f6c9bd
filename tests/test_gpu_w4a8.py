"""W4A8 on the GPU: per-token int8 activations bit-exact against the oracle,
and the int8-MFMA linear (on the GPU's own int8 activations, which are
checked first) against the oracle's product of the same integers, over
ragged shapes, every group size, bias, and the Gemma3-12B prefill layers."""
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


def act_checked(w4, x_bits, what):
    M, K = x_bits.shape
    x8o = gu.Guarded((M, K), torch.int8)
    sxo = gu.Guarded((M,), torch.float32)
    x8, sx = w4.quantize_act_int8(gu.to_dev_bf16(x_bits), x8=x8o.tensor, sx=sxo.tensor)
    torch.cuda.synchronize()
    x8o.check_guards()
    sxo.check_guards()
    x8_ref, sx_ref = oracle.act_quant_ref(x_bits)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32)), \
        f"{what}: per-token scales differ"
    assert np.array_equal(x8.cpu().numpy(), x8_ref), f"{what}: int8 activations differ"
    return x8, sx, x8_ref, sx_ref


def w4a8_bound(x8, sx, codes, s, z, G):
    """sum_k |sx x8| |w_hat| (float64): scale of the accumulation error."""
    xa = np.abs(x8.astype(np.float64)) * sx.astype(np.float64)[:, None]
    return xa @ np.abs(oracle.dequant_ref(codes, s, z, G)).T


@pytest.mark.parametrize("M,K", [(1, 32), (7, 96), (64, 1024), (300, 4096 + 32)])
def test_act_quant_bit_exact(w4, M, K):
    x = workloads.random_bf16((M, K), 1.0, M + K)
    x[0, :] = 0                                   # a zero row
    if M > 2:
        x[2, 5] = workloads.random_bf16((1, 1), 50.0, 3)[0, 0]   # an outlier
    act_checked(w4, x, f"M={M} K={K}")


@pytest.mark.parametrize("K", [64, 2048, 3840, 8192, 8192 + 32, 15360, 16384 + 32])
def test_act_quant_rounding_edges(w4, K):
    """Rows whose quotients land on or next to half-integers (scale 1 with
    exact ties; half the row maximum within an ulp of 63.5, where a
    reciprocal multiply and the binary32 quotient round apart; a quarter
    grid), rows spanning eight decades, subnormal and huge scales, and a zero
    row, at row lengths held in registers (K <= 16384) and beyond."""
    rng = np.random.default_rng(K)
    V = rng.uniform(-1.0, 1.0, (10, K))
    V[0, :10] = [1.0, -0.5, 0.25, -0.75, 0.0, -0.0, 127.0, 63.5, 2.5, -3.5]   # scale 1
    V[0, 10:] = np.round(V[0, 10:] * 254.0) / 2.0                               # more ties
    V[1, :2] = [43.75, 21.875]
    V[2, :2] = [-89.5, 44.75]
    V[3] = np.round(rng.uniform(-50.0, 50.0, K) * 4.0) / 4.0
    V[4] = rng.standard_normal(K) * 10.0 ** rng.integers(-4, 4, K)
    V[5] = rng.uniform(-1.0, 1.0, K) * 1e-38        # scale far below 2^-100
    V[6] = rng.uniform(-1.0, 1.0, K) * 1e38         # scale above 2^100
    V[7] = 0.0
    # a row maximum of 127 * 2^j: scale 2^j, every x / s exact
    V[8] = np.round(rng.uniform(-127.0, 127.0, K) * 2.0) / 2.0 * 2.0 ** -20
    V[8, 0] = 127.0 * 2.0 ** -20
    V[9] = -V[1]
    act_checked(w4, pins.bf16_from_float(V), f"rounding edges K={K}")


def run_case(w4, M, N, K, G, bias, seed, outliers=False):
    W = workloads.random_bf16((N, K), 0.02, seed)
    if outliers:
        W = workloads.normal_bf16_rows(N, K, 0.02, seed,
                                       outlier_cols=workloads.outlier_columns(K, seed))
    x = workloads.random_bf16((M, K), 1.0, seed + 1)
    b = workloads.random_bf16((1, N), 1.0, seed + 2)[0] if bias else None
    codes, s, z = oracle.quantize_ref(W, G)
    gu.log(f"w4a8 M={M} N={N} K={K} G={G} bias={bias} seed={seed}")
    cd, sd, zd = w4.quantize_int4_grouped(gu.to_dev_bf16(W), G)
    x8, sx, x8r, sxr = act_checked(w4, x, f"M={M} K={K}")
    y = gu.Guarded((M, N), torch.bfloat16)
    w4.w4a8_linear(x8, sx, cd, sd, zd, G, bias=gu.to_dev_bf16(b) if bias else None,
                   out=y.tensor)
    torch.cuda.synchronize()
    y.check_guards()
    y_ref = oracle.w4a8_linear_ref(x8r, sxr, codes, s, z, G, b)
    gu.check_linear(gu.to_host_bits(y.tensor), y_ref, w4a8_bound(x8r, sxr, codes, s, z, G),
                    what=f"w4a8 M={M} N={N} K={K} G={G}")


@pytest.mark.parametrize("G,M,N,K", [
    (G, M, N, K)
    for M, N, K in [(1, 64, 128), (17, 300, 256), (129, 130, 512), (257, 257, 1024),
                    (40, 96, 3840),
                    # fewer output rows than one 16-row tile, smallest K
                    (1, 1, 64), (3, 7, 64), (20, 15, 64),
                    # M <= 8 on the vector-ALU kernel: 2048-wide segments, a
                    # partial last one, more than 8 per row (a wave takes
                    # several)
                    (2, 33, 3840), (4, 19, 2048 + 64), (1, 40, 16384 + 2048), (3, 9, 20480),
                    (4, 130, 4096), (6, 33, 3840), (8, 19, 2048 + 64), (5, 40, 18432),
                    (7, 130, 4096), (8, 9, 20480)]
    for G in (32, 64, 128) if K % G == 0])
def test_w4a8_linear(w4, G, M, N, K):
    run_case(w4, M, N, K, G, bias=(M % 2 == 1), seed=7 * N + K + M + G)


# M > 8 on a layer with few output tiles: 8-row slices of the decode kernel
@pytest.mark.parametrize("M,N,K,G", [(9, 200, 4096, 128), (16, 300, 2048, 32), (27, 130, 14336, 64)])
def test_w4a8_row_slices(w4, M, N, K, G):
    run_case(w4, M, N, K, G, bias=(M % 2 == 1), seed=19 * M + N + K)


@pytest.mark.parametrize("M", [2, 4, 6, 8])
@pytest.mark.parametrize("G,N,K", [(32, 37, 2048), (128, 64, 4096), (64, 21, 14336)])
def test_w4a8_even_rows_with_bias(w4, M, G, N, K):
    run_case(w4, M, N, K, G, bias=True, seed=9 * N + K + M)


def test_w4a8_outliers(w4):
    run_case(w4, 300, 96, 1024, 32, bias=True, seed=41, outliers=True)


def test_w4a8_rejects_k_not_multiple_of_64(w4):
    x = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    x8, sx = w4.quantize_act_int8(x)
    W = torch.zeros((16, 96), dtype=torch.bfloat16, device="cuda")
    c, s, z = w4.quantize_int4_grouped(W, 32)
    with pytest.raises(w4.W4Error):
        w4.w4a8_linear(x8, sx, c, s, z, 32)


@pytest.mark.parametrize("layer,G", [("gate", 128), ("q", 32), ("k", 128)])
def test_gemma3_12b_prefill_w4a8(w4, layer, G):
    N, K = workloads.GEMMA3_12B[layer]
    W = workloads.weight_bits(4, layer)
    gu.log(f"w4a8 full {layer} G={G}")
    cd, sd, zd = w4.quantize_int4_grouped(gu.to_dev_bf16(W), G)
    torch.cuda.synchronize()
    c, s, z = oracle.quantize_ref(W, G)
    gu.assert_quant_equal((cd.cpu().numpy(), gu.to_host_bits(sd), gu.to_host_bits(zd)),
                          (c, s, z), f"gemma {layer}")
    x = workloads.activation_bits(4, 2048, K)
    x8, sx, x8r, sxr = act_checked(w4, x, "gemma x")
    y = w4.w4a8_linear(x8, sx, cd, sd, zd, G)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, 127, 128, 2047, np.random.default_rng(N + G).integers(0, 2048, 6)])
    y_ref = oracle.w4a8_linear_ref(x8r[rows], sxr[rows], c, s, z, G)
    gu.check_linear(gu.to_host_bits(y)[rows], y_ref, w4a8_bound(x8r[rows], sxr[rows], c, s, z, G),
                    what=f"gemma {layer} w4a8 G={G} rows {len(rows)}", strict=True)
