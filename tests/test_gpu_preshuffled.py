"""The pre-shuffled weight layout on the GPU: the repack is bit-exact
against the oracle's rearrangement, and the linear on the repacked weights
meets the oracle's linear of the plain weights (every kernel path, ragged
tails, bias, the full-size workloads)."""
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


def repack_checked(w4, cd, sd, zd, ref_plain, G, what):
    """GPU repack of the GPU's plain tensors, compared bit for bit with the
    oracle's repack of the oracle's plain tensors."""
    codes, s, z = ref_plain
    N, K = codes.shape[0], codes.shape[1] * 2
    out = gu.Guarded((N, K // 2), torch.uint8)
    szo = gu.Guarded((N, K // G), torch.int32)
    cp, sz = w4.repack_int4_preshuffled(cd, sd, zd, G, codes_ps=out.tensor, sz=szo.tensor)
    torch.cuda.synchronize()
    out.check_guards()
    szo.check_guards()
    cp_ref, sz_ref = oracle.repack_preshuffled_ref(codes, s, z, G)
    assert np.array_equal(cp.cpu().numpy(), cp_ref), f"{what}: codes_ps differ"
    assert np.array_equal(sz.cpu().numpy().view(np.uint32), sz_ref), f"{what}: sz differ"
    return cp, sz


def run_case(w4, M, N, K, G, bias, path, seed, outliers=False):
    W = workloads.random_bf16((N, K), 0.02, seed)
    if outliers:
        W = workloads.normal_bf16_rows(N, K, 0.02, seed,
                                       outlier_cols=workloads.outlier_columns(K, seed))
    x = workloads.random_bf16((M, K), 1.0, seed + 1)
    b = workloads.random_bf16((1, N), 1.0, seed + 2)[0] if bias else None
    ref_plain = oracle.quantize_ref(W, G)
    gu.log(f"preshuffled M={M} N={N} K={K} G={G} bias={bias} path={path.name} seed={seed}")
    cd, sd, zd = w4.quantize_int4_grouped(gu.to_dev_bf16(W), G)
    cp, sz = repack_checked(w4, cd, sd, zd, ref_plain, G, f"N={N} K={K} G={G}")
    y = gu.Guarded((M, N), torch.bfloat16)
    w4.w4a16_linear_preshuffled(gu.to_dev_bf16(x), cp, sz, G,
                                bias=gu.to_dev_bf16(b) if bias else None, out=y.tensor, path=path)
    torch.cuda.synchronize()
    y.check_guards()
    codes, s, z = ref_plain
    y_ref = oracle.linear_ref(x, codes, s, z, G, b)
    gu.check_linear(gu.to_host_bits(y.tensor), y_ref, gu.abs_bound(x, codes, s, z, G),
                    what=f"preshuffled M={M} N={N} K={K} G={G}")


@pytest.mark.parametrize("N,K,G", [(1, 32, 32), (7, 64, 32), (33, 256, 64), (130, 1024, 128),
                                   (300, 4096 + 128, 32)])
def test_repack_bit_exact(w4, N, K, G):
    W = workloads.random_bf16((N, K), 0.02, N + K)
    cd, sd, zd = w4.quantize_int4_grouped(gu.to_dev_bf16(W), G)
    repack_checked(w4, cd, sd, zd, oracle.quantize_ref(W, G), G, f"N={N} K={K} G={G}")


# decode kernels: register-staged x (M < 5), LDS-copied x (M >= 5), x read
# from L2 (x too long for LDS, K % 128 == 0), phased staging (otherwise)
GEMV_CASES = [(1, 33, 256), (3, 100, 96 * 2), (5, 48, 320), (16, 200, 1024),
              (16, 40, 10240), (16, 40, 10016), (8, 17, 4096 + 128),
              (2, 40, 10240), (4, 17, 4096 + 128), (4, 24, 14336)]


def _with_groups(cases, groups=(32, 64, 128)):
    """(G, M, N, K) for every group size that divides K."""
    return [(G, M, N, K) for M, N, K in cases for G in groups if K % G == 0]


@pytest.mark.parametrize("G,M,N,K", _with_groups(GEMV_CASES))
def test_gemv_preshuffled(w4, G, M, N, K):
    run_case(w4, M, N, K, G, bias=(M % 2 == 1), path=w4.W4Path.GEMV, seed=N + K + M + G)


@pytest.mark.parametrize("G,M,N,K", _with_groups(
    [(17, 64, 128), (129, 320, 256), (257, 130, 512), (40, 96, 1024 + 32)]))
def test_gemm_preshuffled(w4, G, M, N, K):
    run_case(w4, M, N, K, G, bias=(M % 2 == 0), path=w4.W4Path.GEMM, seed=3 * N + K + M)


# enough 128 x 256 tiles to fill a 256-unit chip: the eight-wave GEMM block
# (G >= 64), ragged M and N, a one-column tail, bias on half
@pytest.mark.parametrize("M,N,K", [(2000, 4000, 256), (2047, 4097, 128), (4000, 2048, 256)])
@pytest.mark.parametrize("G", [64, 128])
def test_gemm_preshuffled_wide_blocks(w4, G, M, N, K):
    run_case(w4, M, N, K, G, bias=(N % 2 == 0), path=w4.W4Path.GEMM, seed=N + K + G)


# smallest legal K and fewer output rows than one tile, on both paths
@pytest.mark.parametrize("path", ["GEMV", "GEMM"])
@pytest.mark.parametrize("G,M,N,K", _with_groups(
    [(M, N, K) for M in (1, 3, 16) for N, K in ((1, 32), (7, 32), (15, 64), (7, 4096))]))
def test_edge_shapes_preshuffled(w4, path, G, M, N, K):
    run_case(w4, M, N, K, G, bias=(N % 2 == 1), path=getattr(w4.W4Path, path),
             seed=13 * N + K + M)


@pytest.mark.parametrize("M", [1, 16, 300])
def test_auto_preshuffled_outliers(w4, M):
    run_case(w4, M, 96, 1024, 32, bias=True, path=w4.W4Path.AUTO, seed=M + 5, outliers=True)


def quant_full(w4, cfg, layer, G):
    W = workloads.weight_bits(cfg, layer)
    gu.log(f"full quantize + repack config={cfg} layer={layer} shape={W.shape} G={G}")
    cd, sd, zd = w4.quantize_int4_grouped(gu.to_dev_bf16(W), G)
    torch.cuda.synchronize()
    ref = oracle.quantize_ref(W, G)
    gu.assert_quant_equal((cd.cpu().numpy(), gu.to_host_bits(sd), gu.to_host_bits(zd)), ref,
                          f"config {cfg} {layer}")
    cp, sz = repack_checked(w4, cd, sd, zd, ref, G, f"config {cfg} {layer}")
    return (cd, sd, zd), (cp, sz), ref


@pytest.mark.parametrize("layer", ["o", "gate_up"])
def test_llama3_8b_decode_m1_preshuffled(w4, layer):
    N, K = workloads.LLAMA3_8B[layer]
    _, (cp, sz), (c, s, z) = quant_full(w4, 2, layer, 128)
    x = workloads.activation_bits(2, 1, K)
    y = w4.w4a16_linear_preshuffled(gu.to_dev_bf16(x), cp, sz, 128)
    torch.cuda.synchronize()
    y_ref = oracle.linear_ref(x, c, s, z, 128)
    gu.check_linear(gu.to_host_bits(y), y_ref, gu.abs_bound(x, c, s, z, 128),
                    what=f"llama {layer} M=1 preshuffled", strict=True)


@pytest.mark.parametrize("layer", ["qkv", "down"])
def test_llama3_8b_m16_preshuffled(w4, layer):
    N, K = workloads.LLAMA3_8B[layer]
    _, (cp, sz), (c, s, z) = quant_full(w4, 3, layer, 32)
    x = workloads.activation_bits(3, 16, K)
    y = w4.w4a16_linear_preshuffled(gu.to_dev_bf16(x), cp, sz, 32)
    torch.cuda.synchronize()
    y_ref = oracle.linear_ref(x, c, s, z, 32)
    gu.check_linear(gu.to_host_bits(y), y_ref, gu.abs_bound(x, c, s, z, 32),
                    what=f"llama {layer} M=16 preshuffled", strict=True)


def test_gemma3_12b_gate_m2048_preshuffled(w4):
    N, K = workloads.GEMMA3_12B["gate"]
    _, (cp, sz), (c, s, z) = quant_full(w4, 4, "gate", 128)
    x = workloads.activation_bits(4, 2048, K)
    y = w4.w4a16_linear_preshuffled(gu.to_dev_bf16(x), cp, sz, 128)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, 127, 128, 2047, np.random.default_rng(N).integers(0, 2048, 6)])
    y_ref = oracle.linear_rows_ref(x, rows, c, s, z, 128)
    gu.check_linear(gu.to_host_bits(y)[rows], y_ref, gu.abs_bound(x, c, s, z, 128, rows=rows),
                    what=f"gemma gate M=2048 preshuffled rows {len(rows)}", strict=True)
