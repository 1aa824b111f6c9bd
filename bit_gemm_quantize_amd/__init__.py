"""Python binding of libw4a16.so: group-wise asymmetric int4 weight-only
quantization and the W4A16 linear on MI355X (gfx950).

Argument marshalling only: every step runs in the library's HIP kernels.
torch supplies device memory and the current stream. The library must be
built (``python -m bit_gemm_quantize_amd.build``); nothing here falls back
to another implementation.
"""
from __future__ import annotations

import ctypes
import enum
import os

from .build import LIB_PATH

__all__ = [
    "W4Status", "W4Path", "W4Error", "GROUP_SIZES", "GEMV_MAX_M", "GEMV_MAX_K", "lib",
    "repack_int4_preshuffled", "w4a16_linear_preshuffled", "quantize_act_int8", "w4a8_linear",
    "quantize_int8_grouped", "w8a16_linear", "quantize_int4_grouped_batch",
    "quantize_int4_grouped", "fake_quant_int4_grouped", "w4a16_linear", "status_string",
    "read_stream",
]

GROUP_SIZES = (32, 64, 128)
GEMV_MAX_M = 16
GEMV_MAX_K = 1 << 24  # W4_GEMV_MAX_K: AUTO sends larger K to the GEMM


class W4Status(enum.IntEnum):
    OK = 0
    ERR_NULL = 1
    ERR_SHAPE = 2
    ERR_GROUP = 3
    ERR_ALIGN = 4
    ERR_HIP = 5
    ERR_ALIAS = 6
    ERR_PATH = 7


class W4Path(enum.IntEnum):
    AUTO = 0
    GEMV = 1
    GEMM = 2


class W4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


_LIB = None
_p, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int

QUANT_BATCH_MAX = 8   # W4_QUANT_BATCH_MAX


class QuantJob(ctypes.Structure):
    """w4_quant_job: one weight of quantize_int4_grouped_batch."""
    _fields_ = [("W", _p), ("N", _i64), ("K", _i64), ("codes", _p), ("scales", _p),
                ("zeros", _p)]


def lib() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m bit_gemm_quantize_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        L.quantize_int4_grouped.argtypes = [_p, _i64, _i64, _i64, _p, _p, _p, _p]
        L.quantize_int4_grouped.restype = _int
        L.fake_quant_int4_grouped.argtypes = [_p, _i64, _i64, _i64, _p, _p]
        L.fake_quant_int4_grouped.restype = _int
        L.w4a16_linear.argtypes = [_p, _i64, _p, _p, _p, _p, _i64, _i64, _i64, _p, _p]
        L.w4a16_linear.restype = _int
        L.w4a16_linear_select.argtypes = [_p, _i64, _p, _p, _p, _p, _i64, _i64, _i64,
                                          _p, _int, _p]
        L.w4a16_linear_select.restype = _int
        L.repack_int4_preshuffled.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _p, _p]
        L.repack_int4_preshuffled.restype = _int
        L.w4a16_linear_preshuffled.argtypes = [_p, _i64, _p, _p, _p, _i64, _i64, _i64, _p, _p]
        L.w4a16_linear_preshuffled.restype = _int
        L.w4a16_linear_preshuffled_select.argtypes = [_p, _i64, _p, _p, _p, _i64, _i64, _i64,
                                                      _p, _int, _p]
        L.w4a16_linear_preshuffled_select.restype = _int
        L.quantize_act_int8.argtypes = [_p, _i64, _i64, _p, _p, _p]
        L.quantize_act_int8.restype = _int
        L.w4a8_linear.argtypes = [_p, _p, _i64, _p, _p, _p, _p, _i64, _i64, _i64, _p, _p]
        L.w4a8_linear.restype = _int
        L.quantize_int8_grouped.argtypes = [_p, _i64, _i64, _i64, _p, _p, _p]
        L.quantize_int8_grouped.restype = _int
        L.w8a16_linear.argtypes = [_p, _i64, _p, _p, _p, _i64, _i64, _i64, _p, _p]
        L.w8a16_linear.restype = _int
        L.quantize_int4_grouped_batch.argtypes = [ctypes.POINTER(QuantJob), _i64, _i64, _p]
        L.quantize_int4_grouped_batch.restype = _int
        L.w4_status_string.argtypes = [_int]
        L.w4_status_string.restype = ctypes.c_char_p
        L.w4_read_stream.argtypes = [_p, _i64, _p, _p]
        L.w4_read_stream.restype = _int
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().w4_status_string(int(status)).decode()


def _torch():
    import torch
    return torch


def _check(t, name, dtype, shape, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_ptr(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def quantize_int4_grouped(W, G: int, codes=None, scales=None, zeros=None):
    """Quantize a bf16 GPU weight W[N, K] (group size G along K).

    Returns (codes uint8 [N, K/2], scales bf16 [N, K/G], zeros bf16 [N, K/G]);
    outputs are allocated when not given. Enqueued on torch's current stream.
    """
    torch = _torch()
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N, K]")
    N, K = W.shape
    _check(W, "W", torch.bfloat16, (N, K))
    ng = K // G if G else 0
    if codes is None:
        codes = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    if scales is None:
        scales = torch.empty((N, ng), dtype=torch.bfloat16, device=W.device)
    if zeros is None:
        zeros = torch.empty((N, ng), dtype=torch.bfloat16, device=W.device)
    _check(codes, "codes", torch.uint8, (N, K // 2), W.device)
    _check(scales, "scales", torch.bfloat16, (N, ng), W.device)
    _check(zeros, "zeros", torch.bfloat16, (N, ng), W.device)
    st = lib().quantize_int4_grouped(W.data_ptr(), N, K, G, codes.data_ptr(),
                                     scales.data_ptr(), zeros.data_ptr(),
                                     _stream_ptr(W.device))
    if st != W4Status.OK:
        raise W4Error(st, "quantize_int4_grouped")
    return codes, scales, zeros


def quantize_int4_grouped_batch(weights, G: int, outs=None):
    """quantize_int4_grouped on several bf16 GPU weights in one launch (same
    G). Returns [(codes, scales, zeros), ...]; ``outs`` (same form) are used
    when given. Bit-identical to one call per weight."""
    torch = _torch()
    weights = list(weights)
    if not 1 <= len(weights) <= QUANT_BATCH_MAX:
        raise ValueError(f"1..{QUANT_BATCH_MAX} weights per batch")
    if outs is None:
        outs = [None] * len(weights)
    jobs = (QuantJob * len(weights))()
    result = []
    for i, (W, o) in enumerate(zip(weights, outs)):
        if W.dim() != 2:
            raise ValueError("each W must be 2-D [N, K]")
        N, K = W.shape
        _check(W, "W", torch.bfloat16, (N, K), weights[0].device)
        ng = K // G if G else 0
        if o is None:
            o = (torch.empty((N, K // 2), dtype=torch.uint8, device=W.device),
                 torch.empty((N, ng), dtype=torch.bfloat16, device=W.device),
                 torch.empty((N, ng), dtype=torch.bfloat16, device=W.device))
        codes, scales, zeros = o
        _check(codes, "codes", torch.uint8, (N, K // 2), W.device)
        _check(scales, "scales", torch.bfloat16, (N, ng), W.device)
        _check(zeros, "zeros", torch.bfloat16, (N, ng), W.device)
        jobs[i] = QuantJob(W.data_ptr(), N, K, codes.data_ptr(), scales.data_ptr(),
                           zeros.data_ptr())
        result.append((codes, scales, zeros))
    st = lib().quantize_int4_grouped_batch(jobs, len(weights), G,
                                           _stream_ptr(weights[0].device))
    if st != W4Status.OK:
        raise W4Error(st, "quantize_int4_grouped_batch")
    return result


def fake_quant_int4_grouped(W, G: int, out=None):
    """Quantize -> dequantize round trip of a bf16 GPU weight W[N, K] (group
    size G along K): returns bf16 [N, K] (allocated when ``out`` is None).
    Enqueued on torch's current stream."""
    torch = _torch()
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N, K]")
    N, K = W.shape
    _check(W, "W", torch.bfloat16, (N, K))
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=W.device)
    _check(out, "out", torch.bfloat16, (N, K), W.device)
    st = lib().fake_quant_int4_grouped(W.data_ptr(), N, K, G, out.data_ptr(),
                                       _stream_ptr(W.device))
    if st != W4Status.OK:
        raise W4Error(st, "fake_quant_int4_grouped")
    return out


def w4a16_linear(x, codes, scales, zeros, G: int, bias=None, out=None,
                 path: W4Path = W4Path.AUTO):
    """y = x . dequant(codes, scales, zeros)^T (+ bias) for bf16 GPU x[M, K].

    Returns y bf16 [M, N] (allocated when ``out`` is None). ``path`` forces
    the GEMV or GEMM kernel (for tests); AUTO picks by M.
    """
    torch = _torch()
    if x.dim() != 2 or codes.dim() != 2:
        raise ValueError("x and codes must be 2-D")
    M, K = x.shape
    N = codes.shape[0]
    ng = K // G if G else 0
    _check(x, "x", torch.bfloat16, (M, K))
    _check(codes, "codes", torch.uint8, (N, K // 2), x.device)
    _check(scales, "scales", torch.bfloat16, (N, ng), x.device)
    _check(zeros, "zeros", torch.bfloat16, (N, ng), x.device)
    if bias is not None:
        _check(bias, "bias", torch.bfloat16, (N,), x.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(out, "out", torch.bfloat16, (M, N), x.device)
    st = lib().w4a16_linear_select(
        x.data_ptr(), M, codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
        bias.data_ptr() if bias is not None else None, N, K, G, out.data_ptr(),
        int(path), _stream_ptr(x.device))
    if st != W4Status.OK:
        raise W4Error(st, "w4a16_linear")
    return out


def repack_int4_preshuffled(codes, scales, zeros, G: int, codes_ps=None, sz=None):
    """Plain (codes, scales, zeros) -> pre-shuffled (codes_ps uint8 [N, K/2],
    sz int32 [N, K/G] holding the bits s | z << 16). Outputs are allocated
    when not given. Enqueued on torch's current stream."""
    torch = _torch()
    if codes.dim() != 2:
        raise ValueError("codes must be 2-D [N, K/2]")
    N, K = codes.shape[0], codes.shape[1] * 2
    ng = K // G if G else 0
    _check(codes, "codes", torch.uint8, (N, K // 2))
    _check(scales, "scales", torch.bfloat16, (N, ng), codes.device)
    _check(zeros, "zeros", torch.bfloat16, (N, ng), codes.device)
    if codes_ps is None:
        codes_ps = torch.empty((N, K // 2), dtype=torch.uint8, device=codes.device)
    if sz is None:
        sz = torch.empty((N, ng), dtype=torch.int32, device=codes.device)
    _check(codes_ps, "codes_ps", torch.uint8, (N, K // 2), codes.device)
    _check(sz, "sz", torch.int32, (N, ng), codes.device)
    st = lib().repack_int4_preshuffled(codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                                       N, K, G, codes_ps.data_ptr(), sz.data_ptr(),
                                       _stream_ptr(codes.device))
    if st != W4Status.OK:
        raise W4Error(st, "repack_int4_preshuffled")
    return codes_ps, sz


def w4a16_linear_preshuffled(x, codes_ps, sz, G: int, bias=None, out=None,
                             path: W4Path = W4Path.AUTO):
    """w4a16_linear on the pre-shuffled layout (codes_ps, sz from
    repack_int4_preshuffled)."""
    torch = _torch()
    if x.dim() != 2 or codes_ps.dim() != 2:
        raise ValueError("x and codes_ps must be 2-D")
    M, K = x.shape
    N = codes_ps.shape[0]
    ng = K // G if G else 0
    _check(x, "x", torch.bfloat16, (M, K))
    _check(codes_ps, "codes_ps", torch.uint8, (N, K // 2), x.device)
    _check(sz, "sz", torch.int32, (N, ng), x.device)
    if bias is not None:
        _check(bias, "bias", torch.bfloat16, (N,), x.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(out, "out", torch.bfloat16, (M, N), x.device)
    st = lib().w4a16_linear_preshuffled_select(
        x.data_ptr(), M, codes_ps.data_ptr(), sz.data_ptr(),
        bias.data_ptr() if bias is not None else None, N, K, G, out.data_ptr(),
        int(path), _stream_ptr(x.device))
    if st != W4Status.OK:
        raise W4Error(st, "w4a16_linear_preshuffled")
    return out


def quantize_act_int8(x, x8=None, sx=None):
    """Per-token symmetric int8 of a bf16 GPU x[M, K] (K a multiple of 32).
    Returns (x8 int8 [M, K], sx float32 [M])."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    _check(x, "x", torch.bfloat16, (M, K))
    if x8 is None:
        x8 = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if sx is None:
        sx = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(x8, "x8", torch.int8, (M, K), x.device)
    _check(sx, "sx", torch.float32, (M,), x.device)
    st = lib().quantize_act_int8(x.data_ptr(), M, K, x8.data_ptr(), sx.data_ptr(),
                                 _stream_ptr(x.device))
    if st != W4Status.OK:
        raise W4Error(st, "quantize_act_int8")
    return x8, sx


def w4a8_linear(x8, sx, codes, scales, zeros, G: int, bias=None, out=None):
    """W4A8 linear: int8 activations (quantize_act_int8) with the int4
    weights of quantize_int4_grouped; y bf16 [M, N]."""
    torch = _torch()
    if x8.dim() != 2 or codes.dim() != 2:
        raise ValueError("x8 and codes must be 2-D")
    M, K = x8.shape
    N = codes.shape[0]
    ng = K // G if G else 0
    _check(x8, "x8", torch.int8, (M, K))
    _check(sx, "sx", torch.float32, (M,), x8.device)
    _check(codes, "codes", torch.uint8, (N, K // 2), x8.device)
    _check(scales, "scales", torch.bfloat16, (N, ng), x8.device)
    _check(zeros, "zeros", torch.bfloat16, (N, ng), x8.device)
    if bias is not None:
        _check(bias, "bias", torch.bfloat16, (N,), x8.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x8.device)
    _check(out, "out", torch.bfloat16, (M, N), x8.device)
    st = lib().w4a8_linear(x8.data_ptr(), sx.data_ptr(), M, codes.data_ptr(),
                           scales.data_ptr(), zeros.data_ptr(),
                           bias.data_ptr() if bias is not None else None, N, K, G,
                           out.data_ptr(), _stream_ptr(x8.device))
    if st != W4Status.OK:
        raise W4Error(st, "w4a8_linear")
    return out


def quantize_int8_grouped(W, G: int, codes8=None, scales=None):
    """Group-wise symmetric int8 of a bf16 GPU W[N, K]; returns (codes8 int8
    [N, K], scales bf16 [N, K/G])."""
    torch = _torch()
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N, K]")
    N, K = W.shape
    ng = K // G if G else 0
    _check(W, "W", torch.bfloat16, (N, K))
    if codes8 is None:
        codes8 = torch.empty((N, K), dtype=torch.int8, device=W.device)
    if scales is None:
        scales = torch.empty((N, ng), dtype=torch.bfloat16, device=W.device)
    _check(codes8, "codes8", torch.int8, (N, K), W.device)
    _check(scales, "scales", torch.bfloat16, (N, ng), W.device)
    st = lib().quantize_int8_grouped(W.data_ptr(), N, K, G, codes8.data_ptr(), scales.data_ptr(),
                                     _stream_ptr(W.device))
    if st != W4Status.OK:
        raise W4Error(st, "quantize_int8_grouped")
    return codes8, scales


def w8a16_linear(x, codes8, scales, G: int, bias=None, out=None):
    """y = x . (q s)^T (+ bias) for bf16 GPU x[M, K] and int8 weights."""
    torch = _torch()
    if x.dim() != 2 or codes8.dim() != 2:
        raise ValueError("x and codes8 must be 2-D")
    M, K = x.shape
    N = codes8.shape[0]
    ng = K // G if G else 0
    _check(x, "x", torch.bfloat16, (M, K))
    _check(codes8, "codes8", torch.int8, (N, K), x.device)
    _check(scales, "scales", torch.bfloat16, (N, ng), x.device)
    if bias is not None:
        _check(bias, "bias", torch.bfloat16, (N,), x.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(out, "out", torch.bfloat16, (M, N), x.device)
    st = lib().w8a16_linear(x.data_ptr(), M, codes8.data_ptr(), scales.data_ptr(),
                            bias.data_ptr() if bias is not None else None, N, K, G,
                            out.data_ptr(), _stream_ptr(x.device))
    if st != W4Status.OK:
        raise W4Error(st, "w8a16_linear")
    return out


def read_stream(buf, nbytes=None, sink=None):
    """Read the first nbytes (default: all) of a GPU uint8 tensor once and
    discard them (w4_read_stream): a measurement aid, the read bandwidth a
    plain streaming kernel reaches. Returns the sink tensor."""
    torch = _torch()
    if not isinstance(buf, torch.Tensor) or buf.dtype != torch.uint8 or buf.device.type != "cuda":
        raise TypeError("buf must be a uint8 GPU tensor")
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    n = buf.numel() if nbytes is None else int(nbytes)
    if n > buf.numel():
        raise ValueError("nbytes exceeds the buffer")
    if sink is None:
        sink = torch.empty(64, dtype=torch.int32, device=buf.device)
    st = lib().w4_read_stream(buf.data_ptr(), n, sink.data_ptr(), _stream_ptr(buf.device))
    if st != W4Status.OK:
        raise W4Error(st, "w4_read_stream")
    return sink
