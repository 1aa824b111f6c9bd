"""Helpers for the GPU parity tests: move raw bf16 bits between numpy and
the device, call the library through its binding, and compare with the
oracle."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

import oracle

GUARD = 4096          # guard bytes on each side of an output buffer
FILL = 0xA5


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def lib_or_skip():
    from bit_gemm_quantize_amd.build import LIB_PATH
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libw4a16.so is not built")
    import bit_gemm_quantize_amd as w4
    w4.lib()
    return w4


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class Guarded:
    """An output tensor with guard bytes on both sides, filled with FILL,
    so writes outside the tensor are detected."""

    def __init__(self, shape, dtype):
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape))
        # one byte buffer; the tensor starts GUARD bytes in (a multiple of
        # every element size, so the view stays aligned)
        self.buf = torch.full((n * esz + 2 * GUARD,), FILL, dtype=torch.uint8, device="cuda")
        self.nbytes = n * esz
        self.tensor = self.buf[GUARD:GUARD + n * esz].view(dtype).view(*shape)

    def check_guards(self):
        raw = self.buf.cpu().numpy()
        lo = raw[:GUARD]
        hi = raw[GUARD + self.nbytes:]
        assert np.all(lo == FILL) and np.all(hi == FILL), "write outside the output"


def gpu_quantize(w4, W_bits, G, guarded=True):
    N, K = W_bits.shape
    W = to_dev_bf16(W_bits)
    if guarded:
        c = Guarded((N, K // 2), torch.uint8)
        s = Guarded((N, K // G), torch.bfloat16)
        z = Guarded((N, K // G), torch.bfloat16)
        w4.quantize_int4_grouped(W, G, c.tensor, s.tensor, z.tensor)
        torch.cuda.synchronize()
        for b in (c, s, z):
            b.check_guards()
        return (c.tensor.cpu().numpy(), to_host_bits(s.tensor), to_host_bits(z.tensor))
    c, s, z = w4.quantize_int4_grouped(W, G)
    torch.cuda.synchronize()
    return c.cpu().numpy(), to_host_bits(s), to_host_bits(z)


def assert_quant_equal(got, ref, what=""):
    names = ("codes", "scales", "zeros")
    for name, a, b in zip(names, got, ref):
        assert a.shape == b.shape, f"{what} {name} shape {a.shape} != {b.shape}"
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            raise AssertionError(
                f"{what} {name}: {len(bad)} mismatches, first at {bad[0].tolist()}: "
                f"gpu {a[tuple(bad[0])]:#x} oracle {b[tuple(bad[0])]:#x}")


def abs_bound(x_bits, codes, s_bits, z_bits, G, rows=None, cols=None):
    """sum_k |x[m,k]| |w_hat[n,k]| (float64): scale of the accumulation error."""
    x = np.abs(oracle.bf16_bits_to_f32(x_bits).astype(np.float64))
    if rows is not None:
        x = x[np.asarray(rows)]
    if cols is not None:
        codes, s_bits, z_bits = codes[cols], s_bits[cols], z_bits[cols]
    w = np.abs(oracle.dequant_ref(codes, s_bits, z_bits, G))
    return x @ w.T


def output_floor(y_ref):
    """Relative Frobenius error of the exact result rounded to bf16: what the
    output format alone costs (per element up to half a bf16 ulp, 2^-9 to
    2^-8 relative)."""
    yr = np.asarray(y_ref, dtype=np.float64)
    yb = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(yr.astype(np.float32)))
    return oracle.rel_frobenius(yb.astype(np.float64), yr)


def check_linear(y_bits, y_ref, bound, rel_tol=2e-3, what="", strict=False):
    """Relative Frobenius error <= rel_tol, and elementwise within one bf16
    rounding of the exact value plus float32 accumulation error.

    strict=True (the five workload configurations) applies rel_tol as is.
    Otherwise (small ad-hoc shapes with few outputs, where the bf16 output
    rounding alone can exceed 2e-3) the bar is max(rel_tol, floor + 1e-4),
    floor being the error of the exact result rounded to bf16."""
    y = oracle.bf16_bits_to_f32(y_bits).astype(np.float64)
    assert y.shape == y_ref.shape, f"{what} shape {y.shape} != {y_ref.shape}"
    assert np.all(np.isfinite(y)), f"{what} non-finite output"
    rel = oracle.rel_frobenius(y, y_ref)
    tol = rel_tol if strict else max(rel_tol, output_floor(y_ref) + 1e-4)
    assert rel <= tol, f"{what} relative Frobenius error {rel:.3e} > {tol:.3e}"
    err = np.abs(y - y_ref)
    lim = np.abs(y_ref) * 2.0 ** -8 + 2e-5 * bound + 1e-30
    if not np.all(err <= lim):
        i = np.unravel_index(np.argmax(err / lim), err.shape)
        raise AssertionError(
            f"{what} element {tuple(int(v) for v in i)}: gpu {y[i]!r} oracle {y_ref[i]!r} "
            f"bound {lim[i]:.3e}")
    return rel
