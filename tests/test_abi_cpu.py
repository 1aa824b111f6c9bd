"""The C interface on the CPU: the library loads, exports every function the
header declares, and rejects invalid arguments before any HIP call (so no
kernel is launched and no GPU is needed)."""
import ctypes
import os
import re

import pytest

import bit_gemm_quantize_amd as w4
from bit_gemm_quantize_amd.build import LIB_PATH, ROOT

HEADER = os.path.join(ROOT, "include", "w4a16.h")
MEASURE_HEADER = os.path.join(ROOT, "include", "w4_measure.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB_PATH):
        from bit_gemm_quantize_amd.build import build
        build()
    return w4.lib()


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \t\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted([
        "quantize_int4_grouped", "fake_quant_int4_grouped", "w4a16_linear",
        "w4a16_linear_select", "repack_int4_preshuffled", "w4a16_linear_preshuffled",
        "w4a16_linear_preshuffled_select", "quantize_act_int8", "w4a8_linear",
        "quantize_int8_grouped", "w8a16_linear", "quantize_int4_grouped_batch",
        "w4_status_string"])


def test_measure_header_declares_the_stream_reference():
    assert declared_functions(MEASURE_HEADER) == ["w4_read_stream"]


def test_library_exports_every_declared_function(L):
    for name in declared_functions() + declared_functions(MEASURE_HEADER):
        assert hasattr(L, name), f"{name} not exported by {LIB_PATH}"


@pytest.mark.parametrize("args,expect", [
    ((None, 1024, 0x7F0000001000), w4.W4Status.ERR_NULL),
    ((0x7F0000000000, 1024, None), w4.W4Status.ERR_NULL),
    ((0x7F0000000000, 0, 0x7F0000001000), w4.W4Status.ERR_SHAPE),
    ((0x7F0000000000, 1000, 0x7F0000001000), w4.W4Status.ERR_SHAPE),
    ((0x7F0000000000, (1 << 40) + 16, 0x7F0000001000), w4.W4Status.ERR_SHAPE),
    ((0x7F0000000008, 1024, 0x7F0000001000), w4.W4Status.ERR_ALIGN),
    ((0x7F0000000000, 1024, 0x7F0000001004), w4.W4Status.ERR_ALIGN),
])
def test_read_stream_validation(L, args, expect):
    assert L.w4_read_stream(*args, None) == expect


def test_status_strings(L):
    for st in w4.W4Status:
        s = w4.status_string(st)
        assert s.startswith("W4_" + st.name), s
    assert "unknown" in w4.status_string(99)


# Fake device addresses: never dereferenced, because every call below fails
# validation before the library touches HIP.
A = 0x7F0000000000
B = A + (1 << 32)
C = B + (1 << 32)
D = C + (1 << 32)
E = D + (1 << 32)


def q(L, W=A, N=64, K=128, G=32, codes=B, s=C, z=D):
    return L.quantize_int4_grouped(W, N, K, G, codes, s, z, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(W=None), w4.W4Status.ERR_NULL),
    (dict(codes=None), w4.W4Status.ERR_NULL),
    (dict(s=None), w4.W4Status.ERR_NULL),
    (dict(z=None), w4.W4Status.ERR_NULL),
    (dict(N=0), w4.W4Status.ERR_SHAPE),
    (dict(K=0), w4.W4Status.ERR_SHAPE),
    (dict(N=-3), w4.W4Status.ERR_SHAPE),
    (dict(G=48), w4.W4Status.ERR_GROUP),
    (dict(G=16), w4.W4Status.ERR_GROUP),
    (dict(G=256), w4.W4Status.ERR_GROUP),
    (dict(K=96, G=64), w4.W4Status.ERR_SHAPE),
    (dict(N=1 << 31), w4.W4Status.ERR_SHAPE),
    (dict(W=A + 2), w4.W4Status.ERR_ALIGN),
    (dict(codes=B + 8), w4.W4Status.ERR_ALIGN),
    (dict(s=C + 4), w4.W4Status.ERR_ALIGN),
    (dict(z=D + 1), w4.W4Status.ERR_ALIGN),
    (dict(codes=A + 64), w4.W4Status.ERR_ALIAS),            # codes inside W
    (dict(s=B + 16), w4.W4Status.ERR_ALIAS),                # scales inside codes
    (dict(z=C), w4.W4Status.ERR_ALIAS),                     # zeros == scales
])
def test_quantize_validation(L, kw, expect):
    assert q(L, **kw) == expect


def fq(L, W=A, N=64, K=128, G=32, out=B):
    return L.fake_quant_int4_grouped(W, N, K, G, out, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(W=None), w4.W4Status.ERR_NULL),
    (dict(out=None), w4.W4Status.ERR_NULL),
    (dict(N=0), w4.W4Status.ERR_SHAPE),
    (dict(K=-128), w4.W4Status.ERR_SHAPE),
    (dict(G=96), w4.W4Status.ERR_GROUP),
    (dict(K=160, G=64), w4.W4Status.ERR_SHAPE),
    (dict(W=A + 2), w4.W4Status.ERR_ALIGN),
    (dict(out=B + 8), w4.W4Status.ERR_ALIGN),
    (dict(out=A), w4.W4Status.ERR_ALIAS),                     # in place
    (dict(out=A + 64 * 128 * 2 - 16), w4.W4Status.ERR_ALIAS),  # tail overlap
])
def test_fake_quant_validation(L, kw, expect):
    assert fq(L, **kw) == expect


def lin(L, x=A, M=4, codes=B, s=C, z=D, bias=None, N=64, K=128, G=32, y=E, path=0):
    return L.w4a16_linear_select(x, M, codes, s, z, bias, N, K, G, y, path, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(codes=None), w4.W4Status.ERR_NULL),
    (dict(s=None), w4.W4Status.ERR_NULL),
    (dict(z=None), w4.W4Status.ERR_NULL),
    (dict(x=None), w4.W4Status.ERR_NULL),
    (dict(y=None), w4.W4Status.ERR_NULL),
    (dict(M=-1), w4.W4Status.ERR_SHAPE),
    (dict(M=1 << 24), w4.W4Status.ERR_SHAPE),
    (dict(N=0), w4.W4Status.ERR_SHAPE),
    (dict(K=48, G=32), w4.W4Status.ERR_SHAPE),
    (dict(G=100), w4.W4Status.ERR_GROUP),
    (dict(path=3), w4.W4Status.ERR_PATH),
    (dict(path=-1), w4.W4Status.ERR_PATH),
    (dict(path=1, M=17), w4.W4Status.ERR_PATH),
    (dict(x=A + 8), w4.W4Status.ERR_ALIGN),
    (dict(y=E + 2), w4.W4Status.ERR_ALIGN),
    (dict(bias=E + (1 << 30) + 6), w4.W4Status.ERR_ALIGN),
    (dict(y=A + 256), w4.W4Status.ERR_ALIAS),                # y inside x
    (dict(y=B), w4.W4Status.ERR_ALIAS),                      # y == codes
    (dict(bias=E + 16), w4.W4Status.ERR_ALIAS),              # bias inside y
    # M == 0: nothing to do, x and y may be NULL; nothing is launched
    (dict(M=0, x=None, y=None), w4.W4Status.OK),
    (dict(M=0), w4.W4Status.OK),
    (dict(M=0, x=None, y=None, codes=None), w4.W4Status.ERR_NULL),
    (dict(M=0, G=33), w4.W4Status.ERR_GROUP),
])
def test_linear_validation(L, kw, expect):
    assert lin(L, **kw) == expect


def test_gemv_refuses_k_beyond_its_limit(L):
    # the decode kernels address a row block with 32-bit offsets; a forced
    # GEMV past W4_GEMV_MAX_K is refused before anything is launched
    K = w4.GEMV_MAX_K + 128
    for M in (1, 16):
        assert lin(L, M=M, N=64, K=K, path=w4.W4Path.GEMV) == w4.W4Status.ERR_PATH
        assert L.w4a16_linear_preshuffled_select(A, M, B, C, None, 64, K, 32, E,
                                                 int(w4.W4Path.GEMV), None) == w4.W4Status.ERR_PATH


def test_gemv_k_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define\s+W4_GEMV_MAX_K\s+\(1 << (\d+)\)", text)
    assert m and w4.GEMV_MAX_K == 1 << int(m.group(1))


def test_linear_plain_entry_point_validates(L):
    assert L.w4a16_linear(A, 1, None, C, D, None, 64, 128, 32, E, None) == w4.W4Status.ERR_NULL
    assert L.w4a16_linear(A, 0, B, C, D, None, 64, 128, 32, E, None) == w4.W4Status.OK


def rp(L, codes=A, s=B, z=C, N=64, K=128, G=32, out=D, sz=E):
    return L.repack_int4_preshuffled(codes, s, z, N, K, G, out, sz, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(codes=None), w4.W4Status.ERR_NULL),
    (dict(sz=None), w4.W4Status.ERR_NULL),
    (dict(z=None), w4.W4Status.ERR_NULL),
    (dict(N=0), w4.W4Status.ERR_SHAPE),
    (dict(K=96, G=64), w4.W4Status.ERR_SHAPE),
    (dict(G=8), w4.W4Status.ERR_GROUP),
    (dict(out=D + 4), w4.W4Status.ERR_ALIGN),
    (dict(sz=E + 8), w4.W4Status.ERR_ALIGN),
    (dict(out=A), w4.W4Status.ERR_ALIAS),                    # in place
    (dict(sz=B + 16), w4.W4Status.ERR_ALIAS),                # sz over the scales
    (dict(sz=D + 16), w4.W4Status.ERR_ALIAS),                # sz inside codes_ps
])
def test_repack_validation(L, kw, expect):
    assert rp(L, **kw) == expect


def lin_ps(L, x=A, M=4, codes=B, sz=C, bias=None, N=64, K=128, G=32, y=E, path=0):
    return L.w4a16_linear_preshuffled_select(x, M, codes, sz, bias, N, K, G, y, path, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(codes=None), w4.W4Status.ERR_NULL),
    (dict(sz=None), w4.W4Status.ERR_NULL),
    (dict(x=None), w4.W4Status.ERR_NULL),
    (dict(M=-1), w4.W4Status.ERR_SHAPE),
    (dict(K=48, G=32), w4.W4Status.ERR_SHAPE),
    (dict(G=100), w4.W4Status.ERR_GROUP),
    (dict(path=3), w4.W4Status.ERR_PATH),
    (dict(path=1, M=17), w4.W4Status.ERR_PATH),
    (dict(sz=C + 4), w4.W4Status.ERR_ALIGN),
    (dict(y=C), w4.W4Status.ERR_ALIAS),                      # y over sz
    (dict(M=0, x=None, y=None), w4.W4Status.OK),
])
def test_linear_preshuffled_validation(L, kw, expect):
    assert lin_ps(L, **kw) == expect


def test_linear_preshuffled_auto_entry_point_validates(L):
    assert L.w4a16_linear_preshuffled(A, 1, B, None, None, 64, 128, 32, E, None) == \
        w4.W4Status.ERR_NULL
    assert L.w4a16_linear_preshuffled(A, 0, B, C, None, 64, 128, 32, E, None) == w4.W4Status.OK


def aq(L, x=A, M=4, K=64, x8=B, sx=C):
    return L.quantize_act_int8(x, M, K, x8, sx, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(x=None), w4.W4Status.ERR_NULL),
    (dict(sx=None), w4.W4Status.ERR_NULL),
    (dict(K=48), w4.W4Status.ERR_SHAPE),
    (dict(K=16), w4.W4Status.ERR_SHAPE),
    (dict(M=-1), w4.W4Status.ERR_SHAPE),
    (dict(x8=B + 8), w4.W4Status.ERR_ALIGN),
    (dict(sx=C + 4), w4.W4Status.ERR_ALIGN),
    (dict(x8=A + 64), w4.W4Status.ERR_ALIAS),                # x8 inside x
    (dict(sx=B), w4.W4Status.ERR_ALIAS),                     # sx over x8
    (dict(M=0, x=None, x8=None, sx=None), w4.W4Status.OK),
])
def test_act_quant_validation(L, kw, expect):
    assert aq(L, **kw) == expect


def w8(L, x8=A, sx=B, M=4, codes=C, s=D, z=E, bias=None, N=64, K=128, G=32, y=E + (1 << 31)):
    return L.w4a8_linear(x8, sx, M, codes, s, z, bias, N, K, G, y, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(codes=None), w4.W4Status.ERR_NULL),
    (dict(sx=None), w4.W4Status.ERR_NULL),
    (dict(K=96), w4.W4Status.ERR_SHAPE),                     # K % 64 != 0
    (dict(G=100), w4.W4Status.ERR_GROUP),
    (dict(M=-1), w4.W4Status.ERR_SHAPE),
    (dict(sx=B + 4), w4.W4Status.ERR_ALIGN),
    (dict(y=C), w4.W4Status.ERR_ALIAS),                      # y over codes
    (dict(M=0, x8=None, sx=None, y=None), w4.W4Status.OK),
])
def test_w4a8_validation(L, kw, expect):
    assert w8(L, **kw) == expect


def q8(L, W=A, N=16, K=128, G=32, codes=B, s=C):
    return L.quantize_int8_grouped(W, N, K, G, codes, s, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(W=None), w4.W4Status.ERR_NULL),
    (dict(codes=None), w4.W4Status.ERR_NULL),
    (dict(s=None), w4.W4Status.ERR_NULL),
    (dict(G=48), w4.W4Status.ERR_GROUP),
    (dict(K=96, G=64), w4.W4Status.ERR_SHAPE),               # K % G != 0
    (dict(N=0), w4.W4Status.ERR_SHAPE),
    (dict(codes=B + 8), w4.W4Status.ERR_ALIGN),
    (dict(codes=A + 1024), w4.W4Status.ERR_ALIAS),           # codes inside W
    (dict(s=B + 1024), w4.W4Status.ERR_ALIAS),               # scales inside codes
])
def test_quantize_int8_validation(L, kw, expect):
    assert q8(L, **kw) == expect


def l8(L, x=A, M=4, codes=B, s=C, bias=None, N=64, K=128, G=32, y=E):
    return L.w8a16_linear(x, M, codes, s, bias, N, K, G, y, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(codes=None), w4.W4Status.ERR_NULL),
    (dict(s=None), w4.W4Status.ERR_NULL),
    (dict(x=None), w4.W4Status.ERR_NULL),
    (dict(K=96), w4.W4Status.ERR_SHAPE),                     # K % 64 != 0
    (dict(G=100), w4.W4Status.ERR_GROUP),
    (dict(M=-1), w4.W4Status.ERR_SHAPE),
    (dict(bias=D + 2), w4.W4Status.ERR_ALIGN),
    (dict(y=E + 8), w4.W4Status.ERR_ALIGN),
    (dict(y=B), w4.W4Status.ERR_ALIAS),                      # y over codes
    (dict(y=A + 64), w4.W4Status.ERR_ALIAS),                 # y inside x
    (dict(M=0, x=None, y=None), w4.W4Status.OK),
])
def test_w8a16_validation(L, kw, expect):
    assert l8(L, **kw) == expect


def qb(L, jobs, n=None, G=32):
    arr = (w4.QuantJob * max(1, len(jobs)))(*jobs)
    return L.quantize_int4_grouped_batch(arr, len(jobs) if n is None else n, G, None)


def _job(base, N=16, K=128):
    # W, then codes, scales, zeros laid out apart from each other
    return w4.QuantJob(base, N, K, base + (1 << 28), base + (1 << 29), base + (3 << 28))


@pytest.mark.parametrize("case,expect", [
    ("null_array", w4.W4Status.ERR_NULL),
    ("zero_jobs", w4.W4Status.ERR_SHAPE),
    ("too_many", w4.W4Status.ERR_SHAPE),
    ("bad_group", w4.W4Status.ERR_GROUP),
    ("null_member", w4.W4Status.ERR_NULL),
    ("bad_shape", w4.W4Status.ERR_SHAPE),
    ("misaligned", w4.W4Status.ERR_ALIGN),
    ("codes_over_other_W", w4.W4Status.ERR_ALIAS),
    ("codes_over_other_codes", w4.W4Status.ERR_ALIAS),
])
def test_quantize_batch_validation(L, case, expect):
    a, b = _job(A), _job(B)
    if case == "null_array":
        assert L.quantize_int4_grouped_batch(None, 1, 32, None) == expect
        return
    if case == "zero_jobs":
        assert qb(L, [a], n=0) == expect
        return
    if case == "too_many":
        assert qb(L, [_job(A + (i << 32)) for i in range(9)]) == expect
        return
    if case == "bad_group":
        assert qb(L, [a, b], G=48) == expect
        return
    if case == "null_member":
        b.zeros = None
    elif case == "bad_shape":
        b.K = 100                                # K % G != 0
    elif case == "misaligned":
        b.scales = b.scales + 8
    elif case == "codes_over_other_W":
        b.codes = A + 64
    elif case == "codes_over_other_codes":
        b.codes = a.codes
    assert qb(L, [a, b]) == expect


def test_binding_rejects_host_tensors():
    import torch
    W = torch.zeros(16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        w4.quantize_int4_grouped(W, 32)
    with pytest.raises(TypeError):
        w4.quantize_int4_grouped(W.float(), 32)
