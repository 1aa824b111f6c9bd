"""Quantizer on the GPU against the oracle: bit-exact codes, scales and
zero-points (small seeded shapes, edge cases, guard bytes)."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads
from tests import gpu_util as gu
from tests import pins

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    return gu.lib_or_skip()


def _dist(name, N, K, seed):
    rng = np.random.default_rng(seed)
    if name == "normal":
        v = rng.standard_normal((N, K)) * 0.02
    elif name == "outliers":
        v = rng.standard_normal((N, K)) * 0.02
        cols = rng.choice(K, max(1, K // 100), replace=False)
        v[:, cols] *= 20.0
    elif name == "constant_groups":
        v = rng.standard_normal((N, K))
        v[:, : K // 2] = np.round(rng.standard_normal((N, 1)) * 4) / 4
    elif name == "signed_zeros":
        v = np.where(rng.random((N, K)) < 0.5, 0.0, -0.0) * np.ones((N, K))
        v[::3] = rng.standard_normal((len(v[::3]), K))
        v[1::3, ::7] = -0.0
    elif name == "subnormal_range":
        v = 1.0 + rng.integers(0, 3, (N, K)) * 2.0 ** -7       # tiny ranges
        v[::2] = rng.standard_normal((len(v[::2]), K)) * 1e-38   # subnormal scales
    elif name == "huge":
        v = rng.standard_normal((N, K)) * 1e37
    elif name == "positive":
        v = np.abs(rng.standard_normal((N, K))) + 3.0
    elif name == "negative":
        v = -np.abs(rng.standard_normal((N, K))) - 100.0
    elif name == "wide":
        v = rng.standard_normal((N, K)) * 10.0 ** rng.integers(-20, 20, (N, K))
    elif name == "ties":
        s = 2.0 ** rng.integers(-8, 4, (N, K // 32, 1))
        j = rng.integers(0, 15, (N, K // 32, 32)) + 0.5
        j[:, :, 0] = 0.0
        j[:, :, 1] = 15.0
        v = (j * s).reshape(N, K) - 3.0 * s.repeat(32, axis=2).reshape(N, K)
    else:
        raise ValueError(name)
    return pins.bf16_from_float(v)


DISTS = ["normal", "outliers", "constant_groups", "signed_zeros", "subnormal_range",
         "huge", "positive", "negative", "wide", "ties"]


@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("dist", DISTS)
def test_quantize_bit_exact_distributions(w4, G, dist):
    N, K = 37, 4 * 128 + (G if G < 128 else 0)
    W = _dist(dist, N, K, seed=G + DISTS.index(dist))
    gu.log(f"quantize dist={dist} G={G} N={N} K={K}")
    gu.assert_quant_equal(gu.gpu_quantize(w4, W, G), oracle.quantize_ref(W, G), dist)


@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("dist", DISTS)
def test_fake_quant_bit_exact_distributions(w4, G, dist):
    import torch
    N, K = 29, 4 * 128 + (G if G < 128 else 0)
    W = _dist(dist, N, K, seed=500 + G + DISTS.index(dist))
    gu.log(f"fake quant dist={dist} G={G} N={N} K={K}")
    out = gu.Guarded((N, K), torch.bfloat16)
    w4.fake_quant_int4_grouped(gu.to_dev_bf16(W), G, out=out.tensor)
    torch.cuda.synchronize()
    out.check_guards()
    got = gu.to_host_bits(out.tensor)
    ref = oracle.fake_quant_ref(W, G)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{dist} G={G}: {len(bad)} elements differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("N,Kmul", [(1, 1), (3, 7), (130, 2)])
def test_fake_quant_shapes(w4, G, N, Kmul):
    import torch
    K = G * Kmul
    W = workloads.random_bf16((N, K), 0.02, seed=N * 17 + K)
    gu.log(f"fake quant shape N={N} K={K} G={G}")
    got = gu.to_host_bits(w4.fake_quant_int4_grouped(gu.to_dev_bf16(W), G))
    torch.cuda.synchronize()
    assert np.array_equal(got, oracle.fake_quant_ref(W, G))


@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("N,Kmul", [(1, 1), (1, 3), (2, 1), (7, 5), (16, 8), (129, 3),
                                    (1000, 2), (3, 64)])
def test_quantize_bit_exact_shapes(w4, G, N, Kmul):
    K = G * Kmul
    W = workloads.random_bf16((N, K), 0.02, seed=N * 31 + K)
    gu.log(f"quantize shape N={N} K={K} G={G}")
    gu.assert_quant_equal(gu.gpu_quantize(w4, W, G), oracle.quantize_ref(W, G),
                          f"N={N} K={K}")


def test_quantize_golden_fixtures(w4):
    g = json.load(open(os.path.join(pins.GOLDEN, "g32_halfsteps.json")))
    W = pins.bf16_from_float(g["values"]).reshape(1, -1)
    codes, s, z = gu.gpu_quantize(w4, W, 32)
    assert [f"{b:02x}" for b in codes[0]] == g["codes_packed_hex"]
    assert f"{int(s[0, 0]):04x}" == g["scale_bits_hex"]
    assert f"{int(z[0, 0]):04x}" == g["zero_bits_hex"]
    # the degenerate groups of the special fixture, all in one matrix
    rows = []
    for case in json.load(open(os.path.join(pins.GOLDEN, "special_groups.json")))["cases"]:
        if "values_head" in case:
            vals = np.full(32, case["rest"], dtype=np.float32)
            vals[:len(case["values_head"])] = case["values_head"]
        elif "fill" in case:
            vals = np.full(32, case["fill"], dtype=np.float32)
        elif case["pattern"].startswith("alternate"):
            vals = np.array([0.0, -0.0] * 16, dtype=np.float32)
        else:
            vals = np.zeros(32, dtype=np.float32)
            vals[0] = -0.0
            vals[1] = 15.0
        rows.append(vals)
    W = pins.bf16_from_float(np.array(rows))
    gu.assert_quant_equal(gu.gpu_quantize(w4, W, 32), oracle.quantize_ref(W, 32), "special")


def test_quantize_tiny_config(w4):
    W = workloads.weight_bits(1, "linear")
    gu.assert_quant_equal(gu.gpu_quantize(w4, W, 32), oracle.quantize_ref(W, 32), "tiny")


def test_quantize_deterministic(w4):
    W = _dist("wide", 64, 1024, seed=5)
    a = gu.gpu_quantize(w4, W, 64, guarded=False)
    b = gu.gpu_quantize(w4, W, 64, guarded=False)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("G", [32, 64, 128])
def test_quantize_batch_matches_oracle(w4, G):
    """Several weights in one launch: each job's codes, scales and zeros
    bit-exact against the oracle (ragged rows, different K, a job smaller
    than one wave chunk)."""
    import torch
    shapes = [(300, 1024), (7, 4 * G), (1, G), (129, 3 * 512), (64, 2048 + G)]
    Ws = [workloads.random_bf16(s, 0.02, 97 * G + i) for i, s in enumerate(shapes)]
    Ws[1][0, :G] = 0                                  # a constant group
    outs = [(gu.Guarded((N, K // 2), torch.uint8), gu.Guarded((N, K // G), torch.bfloat16),
             gu.Guarded((N, K // G), torch.bfloat16)) for N, K in shapes]
    gu.log(f"quantize batch G={G} shapes={shapes}")
    w4.quantize_int4_grouped_batch([gu.to_dev_bf16(W) for W in Ws], G,
                                   outs=[tuple(b.tensor for b in o) for o in outs])
    torch.cuda.synchronize()
    for (N, K), W, o in zip(shapes, Ws, outs):
        for b in o:
            b.check_guards()
        got = (o[0].tensor.cpu().numpy(), gu.to_host_bits(o[1].tensor), gu.to_host_bits(o[2].tensor))
        gu.assert_quant_equal(got, oracle.quantize_ref(W, G), f"batch job {N}x{K} G={G}")


def test_quantize_batch_llama3_8b_set(w4):
    """The four Llama-3-8B decode layers in one launch equal four single calls."""
    import torch
    Ws = [gu.to_dev_bf16(workloads.weight_bits(2, layer)) for layer in workloads.LLAMA3_8B]
    gu.log("quantize batch llama3-8b set")
    batch = w4.quantize_int4_grouped_batch(Ws, 128)
    single = [w4.quantize_int4_grouped(W, 128) for W in Ws]
    torch.cuda.synchronize()
    for (cb, sb, zb), (cs, ss, zs) in zip(batch, single):
        assert torch.equal(cb, cs) and torch.equal(sb, ss) and torch.equal(zb, zs)
