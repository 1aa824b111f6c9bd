"""Plain numpy oracle: the quantizer and the W4A16 linear, step by step.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path. It shares no code, table or constant generator with the HIP
library.

Sources (web pages; cited by title and section):
  * "Optimum Quanto" page, "Design overview / Tensors" (设计概览 / 张量):
    for bit-widths below 8 the projection is a group-wise *affine* one with an
    offset ("zero-point"); the integer mapping is a plain rounding
    (``torch.round``, i.e. round half to even); the projection is chosen to
    limit saturated and flushed values.
  * same page, "Modules" (模块): weights are quantized per output channel
    along their first dimension (``nn.Linear`` layout [out, in] = [N, K]);
    the bias is not quantized.
  * same page, "Pitfalls when quantizing activations"
    (量化激活值时需避免的陷阱): matmul results are accumulated at a width well
    above the inputs (int32 / float32) and dequantized afterwards; weights
    are quantized along their first axis because output features are
    computed independently.
  * "torchao模型量化完全指南" page, section 3.1 (一行代码实现INT4量化):
    ``Int4WeightOnlyConfig(group_size=32)`` on ``nn.Linear(512, 512)`` with a
    [1, 512] input; group sizes 32 or 64 recommended, smaller is more accurate.
  * torchao README page ("PyTorch原生训练至推理模型优化"), quick start:
    group-wise int4 weight-only config with ``group_size``; "plain" packing
    format for int4. Same page, "Training / quantization-aware training":
    a group-wise int4 weight config applied in a "prepare" and a "convert"
    step; "torchao模型量化完全指南" section 4.1: QAT simulates the
    quantization error during training; the torchao release notes page,
    "BC Breaking": the int4 weight fake-quantize config.
  * torchao README, int4 weight quantization example: the weight-only config
    takes a packing format (a tile-packed one for one accelerator, a plain
    one for another); torchao release notes, "New Features": a pre-shuffled
    int4 tensor. No format is given (R17).
  * torchao README: int8 dynamic activations with group-wise int4 weights
    (the edge and QAT configuration; group size 32 in its example); "Optimum
    Quanto", "Design overview / Tensors": int8 takes a symmetric projection
    per tensor or per channel (R18).
  * torchao README and its diffusers example: an int8 weight-only config
    with per-group granularity, group size 128; the release notes page
    (0.9.0 API change): the same config as ``group_size=128`` (R19).

Readings taken where the pages leave the step open (each is listed in the
design notes of the repository):
  R1  codes are unsigned 4-bit integers 0..15; the offset is the group
      minimum (a real-valued zero-point stored as bf16), so
      w_hat = q * s + z.
  R2  the range is the group's own [min, max] (no forced inclusion of 0).
  R3  s = bf16_rne( fl32( fl32(hi - lo) / 15 ) ); encoding divides by the
      *stored* bf16 scale so that encode and decode agree.
  R4  division is IEEE binary32 division (correctly rounded), not a
      reciprocal multiply; no fused multiply-add anywhere.
  R5  rounding is half-to-even; results are clamped to [0, 15].
  R6  s == 0 (constant group, or a range whose s underflows bf16) gives all
      codes 0, hence w_hat = lo.
  R7  signed zeros: lo and hi are canonicalised with ``+ 0.0`` (-0 -> +0), so
      the zero-point bits do not depend on which of +0/-0 a min returns.
  R8  packing: codes[n, j] = q[n, 2j] | (q[n, 2j+1] << 4) (low nibble = even
      k); scales and zeros are [N, K/G] row-major.
  R9  the linear uses w_hat exactly (never rounded to bf16), accumulates in
      float64, adds the bias (bf16, if given) in float64, and is returned
      unrounded; the product rounds its fp32 result to bf16.
  R10 inputs must be finite and every group range hi - lo must be finite in
      float32 (the pages say nothing about non-finite weights).
  R16 fake quantization (the quantize -> dequantize round trip a QAT forward
      uses) returns bf16_rne( fl32( q * s + z ) ) per element, with q, s, z
      exactly as the quantizer computes them: the dequantization in binary32
      like every other step, then rounded to the bf16 weight dtype.
  R17 pre-shuffled layout: the pages name kernel-specific int4 packings but
      give none; the library's own is a rearrangement of the plain format:
      each 4-byte word (little endian) of a row holds the codes of 8
      consecutive k = 8j .. 8j+7 with nibble i = q[8j + 2i] and nibble
      4 + i = q[8j + 2i + 1] (i = 0..3), and sz[n, g] = s | z << 16.
  R18 W4A8 activations: symmetric int8 per token (per row of x): a = max|x|,
      sx = fl32(a / 127), x8 = clamp(rne(fl32(x / sx)), -127, 127), 0 when
      a == 0 (binary32 division like R4, ties to even like R5). The linear
      is y = sx * sum_g (s * sum x8 q + z * sum x8) (+ bias): the integer
      sums are exact, the rest float64 here.
  R19 int8 weight-only: symmetric (the Quanto projection for int8) per group
      of G along K: a = max |v| over the group, s = bf16_rne(fl32(a / 127)),
      q = clamp(rne(fl32(v / s)), -127, 127) with the stored scale (as R3,
      R4, R5), 0 when s == 0; w_hat = q * s; codes int8 [N, K], scales bf16
      [N, K/G].
"""
from __future__ import annotations

import numpy as np

GROUP_SIZES = (32, 64, 128)


# ---------------------------------------------------------------------------
# bf16 <-> float32 bit helpers (bf16 is carried as raw uint16 bits)
# ---------------------------------------------------------------------------

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> float32 values. Exact: bf16 is the top half of binary32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest, ties to even (finite inputs).

    Adds 0x7FFF plus the lowest kept bit, then truncates: the standard
    carry-based RNE on the binary32 bit pattern (a carry into the exponent is
    the correct rounding up, including to +-inf at the top of the range).
    """
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("f32_to_bf16_bits: non-finite input")
    u = x.view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# Quantizer
# ---------------------------------------------------------------------------

def _check_group(K: int, G: int) -> None:
    if G not in GROUP_SIZES:
        raise ValueError(f"group size {G} not in {GROUP_SIZES}")
    if K % G != 0:
        raise ValueError(f"K={K} is not a multiple of G={G}")


def quantize_ref(W_bits: np.ndarray, G: int):
    """Group-wise asymmetric int4 quantization of a bf16 weight W[N, K].

    Follows "Optimum Quanto", "Design overview / Tensors": project each group
    of G consecutive weights along K (the per-output-channel axis of
    "Modules") onto the 4-bit range with an offset, then map by rounding.

    Returns (codes uint8 [N, K/2], scales uint16 bf16 bits [N, K/G],
    zeros uint16 bf16 bits [N, K/G]).
    """
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    if W_bits.ndim != 2:
        raise ValueError("W must be 2-D [N, K]")
    N, K = W_bits.shape
    _check_group(K, G)
    v = bf16_bits_to_f32(W_bits).reshape(N, K // G, G)          # step 1
    if not np.all(np.isfinite(v)):
        raise ValueError("R10: non-finite weight")

    # Step 2: the group's range (R2), signed zeros canonicalised (R7).
    lo = v.min(axis=2) + np.float32(0.0)
    hi = v.max(axis=2) + np.float32(0.0)

    # Step 3: scale = range / 15 in binary32, then rounded to bf16 (R3, R4).
    with np.errstate(over="ignore"):
        d = (hi - lo).astype(np.float32)
    if not np.all(np.isfinite(d)):
        raise ValueError("R10: group range overflows float32")
    s32 = (d / np.float32(15.0)).astype(np.float32)
    s_bits = f32_to_bf16_bits(s32)
    s = bf16_bits_to_f32(s_bits)

    # Step 4: the offset is the group minimum; exact in bf16 since lo is one
    # of the inputs (R1).
    z_bits = (lo.view(np.uint32) >> np.uint32(16)).astype(np.uint16)

    # Step 5: encode with the stored scale; IEEE divide, ties to even,
    # clamp to [0, 15]; s == 0 gives code 0 (R3-R6).
    num = (v - lo[:, :, None]).astype(np.float32)
    s_b = np.broadcast_to(s[:, :, None], num.shape)
    zero_scale = s_b == np.float32(0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = np.divide(num, np.where(zero_scale, np.float32(1.0), s_b),
                         dtype=np.float32)
    q = np.clip(np.rint(quot), 0.0, 15.0)
    q = np.where(zero_scale, 0.0, q).astype(np.uint8).reshape(N, K)

    # Step 6: pack two codes per byte, low nibble = even k (R8).
    codes = (q[:, 0::2] | (q[:, 1::2] << np.uint8(4))).astype(np.uint8)
    return codes, s_bits, z_bits


def unpack_codes_ref(codes: np.ndarray) -> np.ndarray:
    """uint8 [N, K/2] -> uint8 [N, K] codes (low nibble = even k, R8)."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, Kh = codes.shape
    q = np.empty((N, 2 * Kh), dtype=np.uint8)
    q[:, 0::2] = codes & np.uint8(0x0F)
    q[:, 1::2] = codes >> np.uint8(4)
    return q


def repack_preshuffled_ref(codes, scales_bits, zeros_bits, G: int):
    """Plain layout -> pre-shuffled layout (R17), by code index.

    Returns (codes_ps uint8 [N, K/2], sz uint32 [N, K/G]). Every word's eight
    codes are listed by nibble position: the four even-k codes, then the
    four odd-k codes; nibble positions 2b and 2b + 1 fill byte b (low, high).
    """
    q = unpack_codes_ref(codes)
    N, K = q.shape
    _check_group(K, G)
    words = q.reshape(N, K // 8, 8)
    nib = np.concatenate([words[:, :, 0::2], words[:, :, 1::2]], axis=2)   # positions 0..7
    b = (nib[:, :, 0::2] | (nib[:, :, 1::2] << np.uint8(4))).astype(np.uint8)
    codes_ps = b.reshape(N, K // 2)
    s = np.asarray(scales_bits, dtype=np.uint16).astype(np.uint32)
    z = np.asarray(zeros_bits, dtype=np.uint16).astype(np.uint32)
    if s.shape != (N, K // G) or z.shape != (N, K // G):
        raise ValueError("scales/zeros must be [N, K/G]")
    return codes_ps, (s | (z << np.uint32(16))).astype(np.uint32)


def dequant_ref(codes, scales_bits, zeros_bits, G: int) -> np.ndarray:
    """w_hat[n, k] = q[n, k] * s[n, k // G] + z[n, k // G] in float64 (R1, R9).

    Exact: q (4 bits) times a bf16 scale needs at most 12 significand bits,
    and adding the bf16 offset stays exact in binary64 for any ordinary
    exponent spread.
    """
    q = unpack_codes_ref(codes).astype(np.float64)
    N, K = q.shape
    _check_group(K, G)
    s = bf16_bits_to_f32(scales_bits).astype(np.float64)
    z = bf16_bits_to_f32(zeros_bits).astype(np.float64)
    if s.shape != (N, K // G) or z.shape != (N, K // G):
        raise ValueError("scales/zeros must be [N, K/G]")
    return q * np.repeat(s, G, axis=1) + np.repeat(z, G, axis=1)


def fake_quant_ref(W_bits: np.ndarray, G: int) -> np.ndarray:
    """Quantize -> dequantize round trip of a bf16 weight W[N, K] (R16).

    torchao README, "Training / quantization-aware training", and
    "torchao模型量化完全指南" section 4.1: the training forward sees the
    weight with the quantization error simulated. Steps: quantize_ref's
    q, s, z; then, in binary32, q * s (exact: a 4-bit integer times a bf16
    value) plus z (one rounding); then round to bf16 (nearest, ties to even).
    Returns uint16 bf16 bits [N, K].
    """
    codes, s_bits, z_bits = quantize_ref(W_bits, G)
    q = unpack_codes_ref(codes).astype(np.float32)
    s = np.repeat(bf16_bits_to_f32(s_bits), G, axis=1)
    z = np.repeat(bf16_bits_to_f32(z_bits), G, axis=1)
    prod = (q * s).astype(np.float32)
    w = (prod + z).astype(np.float32)
    return f32_to_bf16_bits(w)


# ---------------------------------------------------------------------------
# Linear
# ---------------------------------------------------------------------------

def linear_ref(x_bits, codes, scales_bits, zeros_bits, G: int,
               bias_bits=None, n_chunk: int = 4096) -> np.ndarray:
    """y = x . w_hat^T (+ bias), float64, unrounded (R9).

    "Optimum Quanto", "Pitfalls when quantizing activations": the product is
    accumulated wide and dequantized; "Modules": the bias is not quantized.
    The matmul runs in float64 over chunks of output features (memory only;
    no reordering of the sum beyond the library matmul).
    """
    x = bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16)).astype(np.float64)
    if x.ndim != 2:
        raise ValueError("x must be 2-D [M, K]")
    N = codes.shape[0]
    K = 2 * codes.shape[1]
    if x.shape[1] != K:
        raise ValueError("x and codes disagree on K")
    y = np.empty((x.shape[0], N), dtype=np.float64)
    nk = K // G
    for n0 in range(0, N, n_chunk):
        n1 = min(N, n0 + n_chunk)
        w = dequant_ref(codes[n0:n1], np.asarray(scales_bits)[n0:n1],
                        np.asarray(zeros_bits)[n0:n1], G)
        assert w.shape == (n1 - n0, K) and nk == scales_bits.shape[1]
        y[:, n0:n1] = x @ w.T
    if bias_bits is not None:
        y += bf16_bits_to_f32(np.asarray(bias_bits, dtype=np.uint16)
                              ).astype(np.float64)[None, :]
    return y


def quantize_int8_ref(W_bits: np.ndarray, G: int):
    """Group-wise symmetric int8 weight-only quantization of a bf16 W[N, K]
    (R19). Returns (codes int8 [N, K], scales uint16 bf16 bits [N, K/G])."""
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    if W_bits.ndim != 2:
        raise ValueError("W must be 2-D [N, K]")
    N, K = W_bits.shape
    _check_group(K, G)
    v = bf16_bits_to_f32(W_bits).reshape(N, K // G, G)
    if not np.all(np.isfinite(v)):
        raise ValueError("R10: non-finite weight")
    amax = np.abs(v).max(axis=2).astype(np.float32)
    scale_bits = f32_to_bf16_bits((amax / np.float32(127.0)).astype(np.float32))
    sc = np.broadcast_to(bf16_bits_to_f32(scale_bits)[:, :, None], v.shape)
    dead = sc == np.float32(0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.divide(v, np.where(dead, np.float32(1.0), sc), dtype=np.float32)
    q8 = np.where(dead, 0.0, np.clip(np.rint(t), -127.0, 127.0))
    return q8.astype(np.int8).reshape(N, K), scale_bits


def linear_int8_ref(x_bits, codes8, scales_bits, G: int, bias_bits=None) -> np.ndarray:
    """y = x . w_hat^T (+ bias), w_hat = q * s (exact), float64, unrounded."""
    x = bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16)).astype(np.float64)
    q8 = np.asarray(codes8, dtype=np.int8).astype(np.float64)
    N, K = q8.shape
    _check_group(K, G)
    if x.shape[1] != K:
        raise ValueError("x and codes disagree on K")
    sc = bf16_bits_to_f32(scales_bits).astype(np.float64)
    w = q8 * np.repeat(sc, G, axis=1)
    y = x @ w.T
    if bias_bits is not None:
        y = y + bf16_bits_to_f32(np.asarray(bias_bits, dtype=np.uint16)).astype(np.float64)
    return y


def act_quant_ref(x_bits: np.ndarray):
    """Per-token symmetric int8 of a bf16 x[M, K] (R18).

    Returns (x8 int8 [M, K], sx float32 [M]). Division is numpy float32
    (IEEE, correctly rounded); np.rint rounds half to even.
    """
    v = bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16))
    if v.ndim != 2:
        raise ValueError("x must be 2-D [M, K]")
    a = np.abs(v).max(axis=1).astype(np.float32)
    sx = (a / np.float32(127.0)).astype(np.float32)
    zero = sx == np.float32(0.0)
    ratio = np.divide(v, np.where(zero, np.float32(1.0), sx)[:, None],
                      dtype=np.float32)
    code = np.clip(np.rint(ratio), -127.0, 127.0)
    code = np.where(zero[:, None], 0.0, code)
    return code.astype(np.int8), sx


def w4a8_linear_ref(x8, sx, codes, scales_bits, zeros_bits, G: int,
                    bias_bits=None) -> np.ndarray:
    """y = sx * sum_g (s * sum_{k in g} x8 q + z * sum_{k in g} x8) (+ bias),
    float64, unrounded (R18). The per-group integer sums are formed in
    float64, where they are exact (|sum| < 2**53)."""
    x8 = np.asarray(x8, dtype=np.int8).astype(np.float64)
    q = unpack_codes_ref(codes).astype(np.float64)
    M, K = x8.shape
    N = q.shape[0]
    if q.shape[1] != K:
        raise ValueError("x8 and codes disagree on K")
    _check_group(K, G)
    s = bf16_bits_to_f32(scales_bits).astype(np.float64)
    z = bf16_bits_to_f32(zeros_bits).astype(np.float64)
    acc = np.zeros((M, N), dtype=np.float64)
    for g in range(K // G):
        sl = slice(g * G, (g + 1) * G)
        P = x8[:, sl] @ q[:, sl].T              # exact integers
        X = x8[:, sl].sum(axis=1)               # exact integers
        acc += P * s[None, :, g] + X[:, None] * z[None, :, g]
    y = np.asarray(sx, dtype=np.float32).astype(np.float64)[:, None] * acc
    if bias_bits is not None:
        y = y + bf16_bits_to_f32(np.asarray(bias_bits, dtype=np.uint16)).astype(np.float64)
    return y


def linear_rows_ref(x_bits, rows, codes, scales_bits, zeros_bits, G: int,
                    bias_bits=None, cols=None) -> np.ndarray:
    """linear_ref restricted to a subset of output rows m (and optionally
    output columns n): the sampled-output form used at full sizes."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)[np.asarray(rows)]
    if cols is not None:
        cols = np.asarray(cols)
        codes = np.asarray(codes)[cols]
        scales_bits = np.asarray(scales_bits)[cols]
        zeros_bits = np.asarray(zeros_bits)[cols]
        if bias_bits is not None:
            bias_bits = np.asarray(bias_bits)[cols]
    return linear_ref(x_bits, codes, scales_bits, zeros_bits, G, bias_bits)


def rel_frobenius(y, y_ref) -> float:
    """||y - y_ref||_F / ||y_ref||_F in float64."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref)
    num = np.linalg.norm(y - y_ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
