"""Pins of the CPU oracle against facts outside itself (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import ref
from tests import pins


# --- bf16 helpers against torch's own conversion --------------------------

def test_bf16_decode_all_patterns_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_bits_to_f32(bits)
    theirs = pins.f32_from_bf16(bits)
    fin = np.isfinite(theirs)
    assert np.array_equal(ours[fin].view(np.uint32), theirs[fin].view(np.uint32))


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    parts = [
        rng.standard_normal(200000).astype(np.float32) * np.float32(0.02),
        (rng.standard_normal(200000) * 10.0 ** rng.integers(-40, 38, 200000)).astype(np.float32),
        # exact ties: bf16 value plus half an ulp (low 16 bits = 0x8000)
        ((rng.integers(0, 0x7F7F, 50000, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
        # subnormals and the top of the range
        (rng.integers(1, 0x007FFFFF, 50000, dtype=np.uint32)).view(np.float32),
        np.array([3.3895314e38, -3.3895314e38, 3.4e38, 0.0, -0.0], dtype=np.float32),
    ]
    x = np.concatenate(parts).astype(np.float32)
    ours = oracle.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_bf16_rne_rejects_nonfinite():
    with pytest.raises(ValueError):
        oracle.f32_to_bf16_bits(np.array([np.inf], dtype=np.float32))


# --- hand-derived fixtures --------------------------------------------------

def test_golden_halfsteps_ties_to_even():
    pins.check_golden_halfsteps(oracle.quantize_ref)


def test_golden_special_groups():
    pins.check_golden_special(oracle.quantize_ref)


# --- brute force on tiny inputs ----------------------------------------------

@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("dist", ["normal", "uniform_pos", "outlier", "tiny", "wide"])
def test_brute_force_nearest_code(G, dist):
    rng = np.random.default_rng(G * 7 + len(dist))
    N, K = 3, 2 * G
    if dist == "normal":
        v = rng.standard_normal((N, K)) * 0.02
    elif dist == "uniform_pos":
        v = rng.uniform(3.0, 5.0, (N, K))
    elif dist == "outlier":
        v = rng.standard_normal((N, K))
        v[:, rng.integers(0, K, 2)] *= 20.0
    elif dist == "tiny":
        v = rng.standard_normal((N, K)) * 1e-30
    else:
        v = rng.standard_normal((N, K)) * 10.0 ** rng.integers(-6, 6, (N, K))
    W = pins.bf16_from_float(v)
    near = pins.check_brute_force(oracle.quantize_ref, W, G)
    assert near <= 2  # boundary cases are rare


def test_brute_force_constructed_ties():
    # every element an exact tie j + 1/2 (or an endpoint) for several scales
    rows = []
    for s_exp in (-12, -3, 0, 4):
        s = 2.0 ** s_exp
        lo = -7 * s
        vals = [lo + (j + 0.5) * s for j in range(15)] + [lo, lo + 15 * s]
        vals = (vals * 2)[:32]
        rows.append(vals)
    W = pins.bf16_from_float(np.array(rows))
    codes, s_bits, _ = oracle.quantize_ref(W, 32)
    q = pins.unpack_test(codes)
    for r in range(len(rows)):
        for k in range(32):
            j = (k % 17)
            if j < 15:
                assert q[r, k] == (j if j % 2 == 0 else j + 1), (r, k, q[r, k])
    assert pins.check_brute_force(oracle.quantize_ref, W, 32) == 0


# --- invariants ----------------------------------------------------------------

@pytest.mark.parametrize("G", [32, 64, 128])
def test_invariants_many_magnitudes(G):
    rng = np.random.default_rng(100 + G)
    blocks = []
    for mag in (1e-30, 1e-8, 1e-2, 0.02, 1.0, 1e3, 1e30):
        blocks.append(rng.standard_normal((8, 4 * G)) * mag)
    v = np.concatenate(blocks)
    v[3, :G] = 0.7                                  # constant group
    v[5, G:2 * G] = -2.5                            # constant negative group
    v[7, :G] = np.abs(v[7, :G]) + 1.0               # all positive
    v[9, :G] = -np.abs(v[9, :G]) - 1.0              # all negative
    v[11, 5] *= 500.0                               # single outlier
    W = pins.bf16_from_float(v)
    pins.check_invariants(oracle.quantize_ref, oracle.dequant_ref, W, G)


def test_invariants_outlier_columns():
    import workloads
    K, G = 512, 32
    cols = workloads.outlier_columns(K, 3)
    W = workloads.normal_bf16_rows(64, K, 0.02, 3, outlier_cols=cols)
    pins.check_invariants(oracle.quantize_ref, oracle.dequant_ref, W, G)


# --- fake quantization (quantize -> dequantize round trip) ----------------------

@pytest.mark.parametrize("G", [32, 64, 128])
def test_fake_quant_many_magnitudes(G):
    rng = np.random.default_rng(200 + G)
    blocks = [rng.standard_normal((6, 4 * G)) * mag
              for mag in (1e-30, 1e-8, 0.02, 1.0, 1e3, 1e30)]
    v = np.concatenate(blocks)
    v[1, :G] = 0.7                                  # constant group
    v[4, G:2 * G] = -2.5                            # constant negative group
    v[7, 3] *= 400.0                                # single outlier
    pins.check_fake_quant(oracle.fake_quant_ref, oracle.quantize_ref,
                          pins.bf16_from_float(v), G)


def test_fake_quant_outlier_columns():
    import workloads
    K, G = 512, 32
    cols = workloads.outlier_columns(K, 4)
    W = workloads.normal_bf16_rows(48, K, 0.02, 4, outlier_cols=cols)
    pins.check_fake_quant(oracle.fake_quant_ref, oracle.quantize_ref, W, G)


@pytest.mark.parametrize("G", [32, 128])
def test_fake_quant_grid_weights_come_back_unchanged(G):
    W, _, _, _ = pins.grid_weights(12, 4 * G, G, seed=G)
    assert np.array_equal(oracle.fake_quant_ref(W, G), W)


# --- exact reconstruction and the linear -------------------------------------

@pytest.mark.parametrize("G,M,N,K,bias", [
    (32, 1, 48, 96, False), (64, 3, 40, 192, True), (128, 5, 17, 256, True),
    (128, 2, 8, 128, False),               # G = K: per-row min/max
])
def test_grid_exact_reconstruction_and_linear(G, M, N, K, bias):
    pins.check_grid_exact(oracle.quantize_ref, oracle.dequant_ref,
                          oracle.linear_ref, M, N, K, G, seed=G + M, with_bias=bias)


def test_linear_m1_is_dot_product():
    rng = np.random.default_rng(5)
    W = pins.bf16_from_float(rng.standard_normal((20, 64)) * 0.02)
    x = pins.bf16_from_float(rng.standard_normal((1, 64)))
    codes, s, z = oracle.quantize_ref(W, 32)
    y = oracle.linear_ref(x, codes, s, z, 32)
    w_hat = oracle.dequant_ref(codes, s, z, 32)
    xv = pins.f32_from_bf16(x)[0].astype(np.float64)
    for n in range(20):
        assert abs(y[0, n] - float(np.dot(xv, w_hat[n]))) <= 1e-12


def test_linear_rows_subset_matches_full():
    rng = np.random.default_rng(6)
    W = pins.bf16_from_float(rng.standard_normal((30, 128)) * 0.02)
    x = pins.bf16_from_float(rng.standard_normal((9, 128)))
    b = pins.bf16_from_float(rng.standard_normal(30))
    c, s, z = oracle.quantize_ref(W, 64)
    full = oracle.linear_ref(x, c, s, z, 64, b)
    sub = oracle.linear_rows_ref(x, [2, 7], c, s, z, 64, b, cols=[0, 5, 29])
    assert np.array_equal(sub, full[np.ix_([2, 7], [0, 5, 29])])


# --- closed forms and sizes -----------------------------------------------------

@pytest.mark.parametrize("G,expect", [(32, 0.078), (64, 0.090), (128, 0.100)])
def test_gaussian_quantization_noise_closed_form(G, expect):
    # uniform quantiser noise: rms error = s / sqrt(12) with s = E[range]/15
    rng = np.random.default_rng(G)
    W = pins.bf16_from_float(rng.standard_normal((64, 4096)) * 0.02)
    c, s, z = oracle.quantize_ref(W, G)
    w = pins.f32_from_bf16(W).astype(np.float64)
    rel = np.linalg.norm(oracle.dequant_ref(c, s, z, G) - w) / np.linalg.norm(w)
    assert abs(rel - expect) < 0.012, rel


@pytest.mark.parametrize("G", [32, 64, 128])
def test_packed_byte_count(G):
    N, K = 24, 512
    W = pins.bf16_from_float(np.random.default_rng(1).standard_normal((N, K)))
    c, s, z = oracle.quantize_ref(W, G)
    assert c.nbytes + s.nbytes + z.nbytes == N * K // 2 + 4 * N * K // G


def test_rejects_bad_arguments():
    W = np.zeros((2, 96), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.quantize_ref(W, 48)
    with pytest.raises(ValueError):
        oracle.quantize_ref(W, 64)          # K % G != 0
    bad = W.copy()
    bad[0, 0] = 0x7F80                      # +inf
    with pytest.raises(ValueError):
        oracle.quantize_ref(bad, 32)
    huge = W.copy()
    huge[0, 0] = 0x7F7F                     # +max
    huge[0, 1] = 0xFF7F                     # -max: range overflows float32
    with pytest.raises(ValueError):
        oracle.quantize_ref(huge, 32)


def test_oracle_does_not_import_product():
    src = open(ref.__file__).read() + open(oracle.__file__).read()
    assert "bit_gemm_quantize_amd" not in src
