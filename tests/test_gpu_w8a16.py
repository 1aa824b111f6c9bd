"""Int8 weight-only on the GPU: the group-wise symmetric int8 quantizer
bit-exact against the oracle (ties, zero groups, outliers, every group size,
full Llama-3-8B layers), and the bf16-activation linear against the oracle's
product of the same codes and scales, on the split-K path (M <= 16) and the
tiled path (M > 16), ragged shapes, bias, and full-size layers."""
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


def quant8_checked(w4, W_bits, G, what):
    N, K = W_bits.shape
    qo = gu.Guarded((N, K), torch.int8)
    so = gu.Guarded((N, K // G), torch.bfloat16)
    q, s = w4.quantize_int8_grouped(gu.to_dev_bf16(W_bits), G, codes8=qo.tensor,
                                    scales=so.tensor)
    torch.cuda.synchronize()
    qo.check_guards()
    so.check_guards()
    q_ref, s_ref = oracle.quantize_int8_ref(W_bits, G)
    got_s = gu.to_host_bits(s)
    if not np.array_equal(got_s, s_ref):
        bad = np.argwhere(got_s != s_ref)[0]
        raise AssertionError(f"{what}: scale {bad.tolist()} gpu {got_s[tuple(bad)]:#x} "
                             f"oracle {s_ref[tuple(bad)]:#x}")
    got_q = q.cpu().numpy()
    if not np.array_equal(got_q, q_ref):
        bad = np.argwhere(got_q != q_ref)
        raise AssertionError(f"{what}: {len(bad)} codes differ, first {bad[0].tolist()}: "
                             f"gpu {got_q[tuple(bad[0])]} oracle {q_ref[tuple(bad[0])]}")
    return q, s, q_ref, s_ref


def bound8(x_bits, q_ref, s_ref, G):
    """sum_k |x| |w_hat| (float64): scale of the accumulation error."""
    x = np.abs(oracle.bf16_bits_to_f32(x_bits).astype(np.float64))
    w = np.abs(q_ref.astype(np.float64)) * np.repeat(
        oracle.bf16_bits_to_f32(s_ref).astype(np.float64), G, axis=1)
    return x @ w.T


def tie_row(K, seed):
    """Half-integers in [-127, 127] with 127 present: s = 1 and every odd
    multiple of 0.5 is a rounding tie."""
    v = np.random.default_rng(seed).integers(-254, 255, K).astype(np.float32) * 0.5
    v[::32] = 127.0
    return oracle.f32_to_bf16_bits(v)


@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("N,K", [(1, 128), (7, 384), (300, 4096 + 128), (33, 1024)])
def test_quantize_int8_bit_exact(w4, G, N, K):
    W = workloads.random_bf16((N, K), 0.02, N * K + G)
    W[0, :G] = 0                                  # a zero group
    W[0, G:] = tie_row(K - G, G)
    if N > 2:
        W[2, 5] = workloads.random_bf16((1, 1), 5.0, 3)[0, 0]   # an outlier
    gu.log(f"quantize8 N={N} K={K} G={G}")
    quant8_checked(w4, W, G, f"N={N} K={K} G={G}")


def test_quantize_int8_outlier_rows(w4):
    N, K = 96, 2048
    W = workloads.normal_bf16_rows(N, K, 0.02, 5, outlier_cols=workloads.outlier_columns(K, 5))
    for G in (32, 64, 128):
        quant8_checked(w4, W, G, f"outlier rows G={G}")


def run_linear(w4, M, N, K, G, bias, seed):
    W = workloads.random_bf16((N, K), 0.02, seed)
    x = workloads.random_bf16((M, K), 1.0, seed + 1)
    b = workloads.random_bf16((1, N), 1.0, seed + 2)[0] if bias else None
    gu.log(f"w8a16 M={M} N={N} K={K} G={G} bias={bias} seed={seed}")
    q, s, q_ref, s_ref = quant8_checked(w4, W, G, f"N={N} K={K} G={G}")
    y = gu.Guarded((M, N), torch.bfloat16)
    w4.w8a16_linear(gu.to_dev_bf16(x), q, s, G, bias=gu.to_dev_bf16(b) if bias else None,
                    out=y.tensor)
    torch.cuda.synchronize()
    y.check_guards()
    y_ref = oracle.linear_int8_ref(x, q_ref, s_ref, G, b)
    gu.check_linear(gu.to_host_bits(y.tensor), y_ref, bound8(x, q_ref, s_ref, G),
                    what=f"w8a16 M={M} N={N} K={K} G={G}")


@pytest.mark.parametrize("G,M,N,K", [
    (G, M, N, K)
    for M, N, K in [(1, 64, 128), (1, 300, 1024), (5, 17, 384), (16, 130, 3840),
                    (17, 300, 256), (129, 130, 512), (257, 257, 1024), (40, 96, 3840),
                    # fewer output rows than one 16-row tile, smallest K
                    (1, 1, 64), (3, 7, 64), (16, 15, 64), (20, 7, 64),
                    # M <= 4 on the vector-ALU kernel: 1024-wide segments,
                    # a partial last segment, and more than 8 segments per
                    # row (a wave takes several)
                    (2, 7, 64), (2, 33, 3840), (1, 19, 1024 + 64), (2, 13, 5120 + 192),
                    (1, 40, 16384 + 1024), (2, 9, 18432), (4, 33, 3840), (3, 19, 1024 + 64),
                    (4, 9, 18432), (3, 5, 9216)]
    for G in (32, 64, 128) if K % G == 0])
def test_w8a16_linear(w4, G, M, N, K):
    run_linear(w4, M, N, K, G, bias=(M % 2 == 1), seed=7 * N + K + M + G)


# Even M with a bias on the vector-ALU kernel (the shared parametrisation
# gives only odd M a bias).
@pytest.mark.parametrize("M", [2, 4])
@pytest.mark.parametrize("G,N,K", [(32, 37, 2048), (128, 64, 4096), (64, 21, 14336)])
def test_w8a16_even_rows_with_bias(w4, M, G, N, K):
    run_linear(w4, M, N, K, G, bias=True, seed=5 * N + K + M)


def _random_cases(n=24, seed=808):
    """Seeded shapes: ragged N, M across the three kernels (M <= 4 vector-ALU
    rows, M <= 16 split-K matrix cores, tiled GEMM above), K any multiple of
    64 and of G up to about 20000 (so up to 20 segments of 1024 on the row
    kernel), with and without bias."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([32, 64, 128]))
        step = max(64, G)
        K = step * int(rng.integers(1, 20480 // step + 1))
        N = int(rng.integers(1, 700))
        M = int(rng.choice([1, 2, 3, 4, int(rng.integers(5, 17)), int(rng.integers(17, 200))]))
        out.append((i, M, N, K, G, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("i,M,N,K,G,bias", _random_cases())
def test_w8a16_random_shapes(w4, i, M, N, K, G, bias):
    run_linear(w4, M, N, K, G, bias=bias, seed=4000 + i)


# M > 16 on a layer with few output tiles: 16-row slices of the decode
# kernels (a last slice of <= 4 rows on the vector-ALU kernel)
@pytest.mark.parametrize("M,N,K,G", [(17, 200, 4096, 128), (35, 300, 2048, 32), (50, 130, 14336, 64)])
def test_w8a16_row_slices(w4, M, N, K, G):
    run_linear(w4, M, N, K, G, bias=(M % 2 == 1), seed=23 * M + N + K)


def test_w8a16_empty_batch(w4):
    q = torch.zeros((16, 128), dtype=torch.int8, device="cuda")
    s = torch.zeros((16, 4), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    y = w4.w8a16_linear(x, q, s, 32)
    assert y.shape == (0, 16)


def test_w8a16_rejects_k_not_multiple_of_64(w4):
    W = torch.zeros((16, 96), dtype=torch.bfloat16, device="cuda")
    q, s = w4.quantize_int8_grouped(W, 32)
    x = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(w4.W4Error):
        w4.w8a16_linear(x, q, s, 32)


@pytest.mark.parametrize("layer", ["qkv", "down"])
def test_llama3_8b_decode_w8a16(w4, layer):
    """Full decode layer, M = 1, G = 128: codes bit-exact, every output checked."""
    N, K = workloads.LLAMA3_8B[layer]
    W = workloads.weight_bits(2, layer)
    gu.log(f"w8a16 full llama {layer}")
    q, s, q_ref, s_ref = quant8_checked(w4, W, 128, f"llama {layer}")
    x = workloads.activation_bits(2, 1, K)
    y = w4.w8a16_linear(gu.to_dev_bf16(x), q, s, 128)
    torch.cuda.synchronize()
    y_ref = oracle.linear_int8_ref(x, q_ref, s_ref, 128)
    gu.check_linear(gu.to_host_bits(y), y_ref, bound8(x, q_ref, s_ref, 128),
                    what=f"llama {layer} w8a16", strict=True)


@pytest.mark.parametrize("layer", ["gate", "o", "k"])
def test_gemma3_12b_prefill_w8a16(w4, layer):
    """Full prefill layer, M = 2048, G = 128, sampled rows."""
    N, K = workloads.GEMMA3_12B[layer]
    W = workloads.weight_bits(4, layer)
    gu.log(f"w8a16 full gemma {layer}")
    q, s, q_ref, s_ref = quant8_checked(w4, W, 128, f"gemma {layer}")
    x = workloads.activation_bits(4, 2048, K)
    y = w4.w8a16_linear(gu.to_dev_bf16(x), q, s, 128)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, 127, 128, 2047, np.random.default_rng(N).integers(0, 2048, 6)])
    y_ref = oracle.linear_int8_ref(x[rows], q_ref, s_ref, 128)
    gu.check_linear(gu.to_host_bits(y)[rows], y_ref, bound8(x[rows], q_ref, s_ref, 128),
                    what=f"gemma {layer} w8a16 rows {len(rows)}", strict=True)
