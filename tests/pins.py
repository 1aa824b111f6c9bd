"""Checks that pin the oracle to facts outside itself (brute force, exact
reconstruction, invariants, hand-derived fixtures). Each check takes the
oracle's functions as arguments so the same checks can be run against
deliberately broken copies (see test_oracle_mutants.py)."""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f32_from_bf16(bits):
    """Test-side bf16 decode through torch (independent of the oracle)."""
    t = torch.from_numpy(np.asarray(bits, dtype=np.uint16).astype(np.int16))
    return t.view(torch.bfloat16).to(torch.float32).numpy()


def bf16_from_float(vals):
    t = torch.tensor(np.asarray(vals, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def unpack_test(codes):
    """Test-side nibble unpack: element 2j is the low nibble of byte j."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.zeros((codes.shape[0], codes.shape[1] * 2), dtype=np.int64)
    for j in range(codes.shape[1]):
        out[:, 2 * j] = codes[:, j] % 16
        out[:, 2 * j + 1] = codes[:, j] // 16
    return out


# --- pin 1: hand-derived fixtures -----------------------------------------

def check_golden_halfsteps(quantize):
    g = json.load(open(os.path.join(GOLDEN, "g32_halfsteps.json")))
    W = bf16_from_float(g["values"]).reshape(1, -1)
    codes, s, z = quantize(W, g["G"])
    assert [f"{b:02x}" for b in codes[0]] == g["codes_packed_hex"], "packed codes"
    assert f"{int(s[0, 0]):04x}" == g["scale_bits_hex"], "scale bits"
    assert f"{int(z[0, 0]):04x}" == g["zero_bits_hex"], "zero bits"
    assert list(unpack_test(codes)[0]) == g["codes_unpacked"], "unpacked"


def check_golden_special(quantize):
    g = json.load(open(os.path.join(GOLDEN, "special_groups.json")))
    for case in g["cases"]:
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
        W = bf16_from_float(vals).reshape(1, 32)
        codes, s, z = quantize(W, 32)
        assert f"{int(s[0, 0]):04x}" == case["scale_bits_hex"], case["name"]
        assert f"{int(z[0, 0]):04x}" == case["zero_bits_hex"], case["name"]
        if "codes_packed_hex" in case:
            assert all(f"{b:02x}" == case["codes_packed_hex"] for b in codes[0]), case["name"]
        if "codes_first_two" in case:
            assert list(unpack_test(codes)[0, :2]) == case["codes_first_two"], case["name"]
        if "codes_first" in case:
            n = len(case["codes_first"])
            assert list(unpack_test(codes)[0, :n]) == case["codes_first"], case["name"]


# --- pin 2: brute force nearest code (exact rational arithmetic) -----------

def brute_force_codes(W_bits, G, s_bits, z_bits):
    """For each element pick the code q in 0..15 whose q*s + z is nearest to
    w in exact arithmetic, ties to the even code. Uses the scale and offset
    under test; also returns the exact quotient (w - z)/s per element."""
    w = f32_from_bf16(W_bits).astype(np.float64)
    s = f32_from_bf16(s_bits).astype(np.float64)
    z = f32_from_bf16(z_bits).astype(np.float64)
    N, K = w.shape
    q = np.zeros((N, K), dtype=np.int64)
    quot = np.zeros((N, K), dtype=object)
    for n in range(N):
        for k in range(K):
            sv = Fraction(s[n, k // G])
            zv = Fraction(z[n, k // G])
            wv = Fraction(w[n, k])
            if sv == 0:
                q[n, k] = 0
                quot[n, k] = None
                continue
            best, best_err = None, None
            for c in range(16):
                err = abs(wv - (c * sv + zv))
                if best is None or err < best_err or (err == best_err and c % 2 == 0):
                    best, best_err = c, err
            q[n, k] = best
            quot[n, k] = (wv - zv) / sv
    return q, quot


def check_brute_force(quantize, W_bits, G, tol_rel=2.0**-20):
    """Codes equal the brute-force nearest codes except where the exact
    quotient lies within tol_rel of a half-integer (there float32 rounding of
    the subtraction or the quotient decides, and both neighbours are
    acceptable). Returns the number of such boundary elements."""
    codes, s_bits, z_bits = quantize(W_bits, G)
    q = unpack_test(codes)
    qb, quot = brute_force_codes(W_bits, G, s_bits, z_bits)
    near = 0
    for idx in zip(*np.nonzero(q != qb)):
        t = quot[idx]
        assert t is not None, f"code mismatch at {idx} with zero scale"
        assert t >= 0
        half = math.floor(t) + Fraction(1, 2)
        # an exact tie whose float32 numerator is exact must go to even
        w32 = np.float32(f32_from_bf16(W_bits)[idx])
        z32 = np.float32(f32_from_bf16(z_bits)[idx[0], idx[1] // G])
        exact_num = Fraction(float(np.float32(w32 - z32))) == Fraction(float(w32)) - Fraction(float(z32))
        assert not (t == half and exact_num), f"exact tie at {idx} not rounded to even"
        assert abs(t - half) <= tol_rel * max(abs(t), 1), (
            f"code {q[idx]} != brute force {qb[idx]} at {idx}, quotient {float(t)}")
        assert abs(int(q[idx]) - int(qb[idx])) == 1
        near += 1
    return near


# --- pin 3: invariants -----------------------------------------------------

def check_invariants(quantize, dequant, W_bits, G):
    codes, s_bits, z_bits = quantize(W_bits, G)
    N, K = W_bits.shape
    w = f32_from_bf16(W_bits).astype(np.float64)
    s = f32_from_bf16(s_bits).astype(np.float64)
    z = f32_from_bf16(z_bits).astype(np.float64)
    q = unpack_test(codes)
    assert codes.shape == (N, K // 2) and codes.dtype == np.uint8
    assert s_bits.shape == (N, K // G) and z_bits.shape == (N, K // G)
    assert q.min() >= 0 and q.max() <= 15
    wg = w.reshape(N, K // G, G)
    qg = q.reshape(N, K // G, G)
    # offset is the group minimum (an element of the group)
    assert np.array_equal(z, wg.min(axis=2) + 0.0), "zero != group minimum"
    w_hat = dequant(codes, s_bits, z_bits, G)
    # |w_hat - w| <= s/2 elementwise (s > 0), exact round trip when s == 0
    err = np.abs(w_hat - w).reshape(N, K // G, G)
    pos = s > 0
    assert np.all(err[pos] <= (s[pos] / 2.0)[:, None] * (1 + 1e-12)), "error > s/2"
    cst = wg.max(axis=2) == wg.min(axis=2)
    assert np.all(err[cst] == 0.0), "constant group does not round-trip"
    assert np.all(s[cst] == 0.0)
    # every group with s > 0 uses code 0 (at its minimum) and code 15 (at its max)
    amin = np.argmin(wg, axis=2)
    amax = np.argmax(wg, axis=2)
    ii, jj = np.nonzero(pos)
    assert np.all(qg[ii, jj, amin[ii, jj]] == 0), "minimum not coded 0"
    assert np.all(qg[ii, jj, amax[ii, jj]] == 15), "maximum not coded 15"
    # scale is the bf16 rounding of range/15 (within half a bf16 ulp)
    rng = (wg.max(axis=2) - wg.min(axis=2))[pos] / 15.0
    assert np.all(np.abs(s[pos] - rng) <= rng * 2.0**-8 + 1e-300)


# --- pin 4: exact reconstruction and the linear -----------------------------

def grid_weights(N, K, G, seed, lo_exp=-6, s_exp=-9):
    """W[n, k] = lo[n,g] + j[n,k] * 2^s_exp with j in 0..15 and both 0 and 15
    present in every group, so the quantizer must return exactly j, s and lo.
    lo is a multiple of 2^s_exp (so every grid point is exact in bf16)."""
    rng = np.random.default_rng(seed)
    j = rng.integers(0, 16, size=(N, K // G, G))
    j[:, :, 0] = 0
    j[:, :, 1] = 15
    for n in range(N):                  # shuffle the positions of 0 and 15
        for g in range(K // G):
            rng.shuffle(j[n, g])
    step = 2.0 ** s_exp
    lo = rng.integers(-(2 ** (lo_exp - s_exp)), 2 ** (lo_exp - s_exp),
                      size=(N, K // G)) * step
    w = lo[:, :, None] + j * step
    bits = bf16_from_float(w.reshape(N, K))
    assert np.array_equal(f32_from_bf16(bits).astype(np.float64), w.reshape(N, K))
    return bits, j.reshape(N, K), lo, step


def check_grid_exact(quantize, dequant, linear, M, N, K, G, seed, with_bias):
    W_bits, j, lo, step = grid_weights(N, K, G, seed)
    codes, s_bits, z_bits = quantize(W_bits, G)
    assert np.array_equal(unpack_test(codes), j), "codes != grid indices"
    assert np.all(f32_from_bf16(s_bits) == step), "scale != grid step"
    assert np.array_equal(f32_from_bf16(z_bits).astype(np.float64), lo + 0.0)
    w = f32_from_bf16(W_bits).astype(np.float64)
    assert np.array_equal(dequant(codes, s_bits, z_bits, G), w)
    rng = np.random.default_rng(seed + 1)
    x_bits = bf16_from_float(rng.standard_normal((M, K)))
    b_bits = bf16_from_float(rng.standard_normal(N)) if with_bias else None
    y = linear(x_bits, codes, s_bits, z_bits, G, b_bits)
    # independent reference: torch float64 matmul of the original weights
    xt = torch.from_numpy(f32_from_bf16(x_bits).astype(np.float64))
    yt = xt @ torch.from_numpy(w).T
    if with_bias:
        yt = yt + torch.from_numpy(f32_from_bf16(b_bits).astype(np.float64))
    yt = yt.numpy()
    assert y.shape == (M, N)
    assert np.allclose(y, yt, rtol=1e-12, atol=1e-12), "linear != x @ W^T"


# --- pin 5: bf16 rounding helper against torch -----------------------------

def check_bf16_helper(f32_to_bf16_bits):
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        ((rng.integers(0, 0x7F7F, 5000, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
    ]).astype(np.float32)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), theirs), "bf16 rounding"


# --- pin 6: the fake-quantize round trip --------------------------------------

def check_fake_quant(fake_quant, quantize, W_bits, G):
    """Every element within half a step (plus the roundings to binary32 and
    bf16) of its weight; constant groups unchanged; and the same bits as an
    independent evaluation: torch float64 q * s + z rounded by torch to
    float32 and then to bf16."""
    N, K = W_bits.shape
    fq = fake_quant(W_bits, G)
    assert fq.shape == (N, K) and fq.dtype == np.uint16
    codes, s_bits, z_bits = quantize(W_bits, G)
    q = unpack_test(codes).astype(np.float64)
    s = np.repeat(f32_from_bf16(s_bits).astype(np.float64), G, axis=1)
    z = np.repeat(f32_from_bf16(z_bits).astype(np.float64), G, axis=1)
    exact = q * s + z
    theirs = (torch.from_numpy(exact).to(torch.float32).to(torch.bfloat16)
              .view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(fq, theirs), "fake quant != torch rounding of q s + z"
    w = f32_from_bf16(W_bits).astype(np.float64)
    got = f32_from_bf16(fq).astype(np.float64)
    bound = s / 2 + np.abs(got) * 2.0**-8 + np.abs(exact) * 2.0**-24 + 1e-300
    assert np.all(np.abs(got - w) <= bound), "fake quant further than s/2 from w"
    wg = w.reshape(N, K // G, G)
    const = np.all(wg == wg[:, :, :1], axis=2)
    cmask = np.repeat(const, G, axis=1)
    assert np.array_equal(got[cmask], w[cmask] + 0.0), "constant group changed"


def check_preshuffle(repack, W_codes_seed=17):
    """The pre-shuffled layout (R17), pinned three ways that do not share the
    oracle's index arithmetic:
      * a word worked out by hand: codes k = 0..7 equal to 0..7 give the
        bytes 0x20, 0x64, 0x31, 0x75 (nibbles 0, 2, 4, 6 | 1, 3, 5, 7), and
        sz holds s in the low and z in the high half-word;
      * its purpose: for every word and i = 0..3, ((w >> 4i) & 0x000F000F) |
        0x43004300 read as two bf16 values is (128 + q[8j+2i], 128 +
        q[8j+2i+1]) with q read from the plain codes;
      * it is a rearrangement: per row the multiset of nibbles is unchanged."""
    q = np.tile(np.arange(8, dtype=np.uint8), 4).reshape(1, 32)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    cp, sz = repack(codes, np.array([[0x3F80]], np.uint16), np.array([[0xBF80]], np.uint16), 32)
    assert cp.dtype == np.uint8 and cp.shape == (1, 16)
    assert list(cp[0, :4]) == [0x20, 0x64, 0x31, 0x75], [hex(v) for v in cp[0, :4]]
    assert sz.dtype == np.uint32 and int(sz[0, 0]) == 0xBF803F80
    rng = np.random.default_rng(W_codes_seed)
    for (N, K, G) in ((3, 64, 32), (2, 256, 128), (5, 128, 64)):
        codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
        s_bits = rng.integers(0, 1 << 16, (N, K // G), dtype=np.uint16)
        z_bits = rng.integers(0, 1 << 16, (N, K // G), dtype=np.uint16)
        cp, sz = repack(codes, s_bits, z_bits, G)
        qq = unpack_test(codes).astype(np.uint32)
        words = cp.view("<u4")                      # [N, K / 8]
        for i in range(4):
            pair = ((words >> np.uint32(4 * i)) & np.uint32(0x000F000F)) | np.uint32(0x43004300)
            lo = f32_from_bf16((pair & 0xFFFF).astype(np.uint16))
            hi = f32_from_bf16((pair >> 16).astype(np.uint16))
            assert np.array_equal(lo, 128.0 + qq[:, 2 * i::8]), f"pair {i} low"
            assert np.array_equal(hi, 128.0 + qq[:, 2 * i + 1::8]), f"pair {i} high"
        for n in range(N):
            a = np.sort(np.r_[cp[n] & 15, cp[n] >> 4])
            b = np.sort(np.r_[codes[n] & 15, codes[n] >> 4])
            assert np.array_equal(a, b), "not a rearrangement"
        assert np.array_equal(sz & 0xFFFF, s_bits) and np.array_equal(sz >> 16, z_bits)


def _fl32_of(q: Fraction) -> Fraction:
    """Exact binary32 rounding (nearest, ties to even) of a rational, normal
    and subnormal range."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                            # subnormals share the 2^-149 step
    ulp = Fraction(2) ** (e - 23)
    k = a / ulp
    fl = k.numerator // k.denominator
    rem = k - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def _rne_int(q: Fraction) -> int:
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def check_act_quant(act_quant):
    """Per-token int8 (R18) against exact rational arithmetic on small rows
    (scale = binary32 rounding of max|x| / 127, codes = ties-to-even of the
    binary32 rounding of x / scale, clamped), plus the invariants: |x8| <=
    127, the row maximum maps to +-127, x8 * sx within sx / 2 of x, zero rows
    give zeros, and negating x negates the codes."""
    rng = np.random.default_rng(23)
    V = rng.standard_normal((8, 64)) * 10.0 ** rng.integers(-4, 4, (8, 1))
    V[2] = 0.0
    V[3] = rng.uniform(-1.0, 1.0, 64)
    V[3, :10] = [1.0, -0.5, 0.25, -0.75, 0.0, -0.0, 127.0, 63.5, 2.5, -3.5]   # scale 1: exact ties
    V[4] = np.round(V[4] * 4) / 4
    # half the row maximum lands within an ulp of 63.5: the binary32 quotient
    # and a reciprocal multiply round to different codes here
    V[5] = rng.uniform(-1.0, 1.0, 64)
    V[5, :2] = [43.75, 21.875]
    V[6] = rng.uniform(-1.0, 1.0, 64)
    V[6, :2] = [-89.5, 44.75]
    xb = bf16_from_float(V)
    x8, sx = act_quant(xb)
    assert x8.dtype == np.int8 and sx.dtype == np.float32 and x8.shape == V.shape
    v = f32_from_bf16(xb)
    for m in range(V.shape[0]):
        a = max(abs(Fraction(float(t))) for t in v[m])
        s_exact = _fl32_of(a / 127)
        assert Fraction(float(sx[m])) == s_exact, f"row {m} scale"
        for k in range(V.shape[1]):
            if s_exact == 0:
                want = 0
            else:
                want = max(-127, min(127, _rne_int(_fl32_of(Fraction(float(v[m, k])) / s_exact))))
            assert int(x8[m, k]) == want, f"row {m} k {k}: {int(x8[m, k])} != {want}"
    assert np.all(np.abs(x8.astype(np.int32)) <= 127)
    live = sx > 0
    amax_k = np.abs(v).argmax(axis=1)
    assert np.all(np.abs(x8[np.arange(len(v)), amax_k][live].astype(np.int32)) == 127)
    err = np.abs(x8.astype(np.float64) * sx[:, None].astype(np.float64) - v)
    assert np.all(err <= sx[:, None].astype(np.float64) * (0.5 + 2.0**-20) + 1e-300)
    assert np.all(x8[~live] == 0)
    x8n, sxn = act_quant(bf16_from_float(-V))
    assert np.array_equal(sxn, sx) and np.array_equal(x8n.astype(np.int32), -x8.astype(np.int32))


def check_w4a8_linear(w4a8, linear, quantize):
    """The W4A8 product (R18) two ways: exact rationals on a tiny case, and
    a reduction to the pinned W4A16 oracle: with a power-of-two sx every
    dequantized activation x8 * sx is a bf16 value, and the two products of
    the same weights must agree."""
    rng = np.random.default_rng(29)
    M, N, K, G = 2, 3, 64, 32
    W = bf16_from_float(rng.standard_normal((N, K)) * 0.05)
    codes, s_bits, z_bits = quantize(W, G)
    x8 = rng.integers(-127, 128, (M, K)).astype(np.int8)
    sx = np.array([0.0123, 2.5], dtype=np.float32)
    bias = bf16_from_float(rng.standard_normal((1, N)))[0]
    y = w4a8(x8, sx, codes, s_bits, z_bits, G, bias)
    q = unpack_test(codes)
    sF = [[Fraction(float(t)) for t in r] for r in f32_from_bf16(s_bits)]
    zF = [[Fraction(float(t)) for t in r] for r in f32_from_bf16(z_bits)]
    bF = [Fraction(float(t)) for t in f32_from_bf16(bias)]
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for g in range(K // G):
                P = sum(int(x8[m, k]) * int(q[n, k]) for k in range(g * G, (g + 1) * G))
                X = sum(int(x8[m, k]) for k in range(g * G, (g + 1) * G))
                tot += sF[n][g] * P + zF[n][g] * X
            exact = Fraction(float(sx[m])) * tot + bF[n]
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 10**12), (m, n)
    M, N, K, G = 5, 40, 256, 64
    W = bf16_from_float(rng.standard_normal((N, K)) * 0.05)
    codes, s_bits, z_bits = quantize(W, G)
    x8 = rng.integers(-127, 128, (M, K)).astype(np.int8)
    sx = np.float32(2.0) ** rng.integers(-12, -4, M).astype(np.float32)
    xh = bf16_from_float(x8.astype(np.float64) * sx[:, None].astype(np.float64))
    assert np.array_equal(f32_from_bf16(xh).astype(np.float64),
                          x8.astype(np.float64) * sx[:, None].astype(np.float64))
    y1 = w4a8(x8, sx.astype(np.float32), codes, s_bits, z_bits, G)
    y2 = linear(xh, codes, s_bits, z_bits, G)
    assert np.allclose(y1, y2, rtol=1e-12, atol=1e-12 * np.abs(y2).max())


def _bf16_of_f32(x: Fraction) -> Fraction:
    """Exact bf16 rounding (nearest, ties to even) of a binary32 value."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 7)
    k = a / ulp
    fl = k.numerator // k.denominator
    rem = k - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def check_int8_weights(quantize8, linear8):
    """Int8 weight-only (R19): scales and codes against exact rationals
    (binary32 rounding of max|v| / 127, then bf16 rounding; binary32 rounding
    of v / s, ties to even, clamp), invariants (|q| <= 127, |q s - v| <= s/2,
    zero groups give 0, negating W negates the codes), and the linear
    against an independent float64 product with W itself on weights that are
    exact multiples q * s of a power-of-two scale."""
    rng = np.random.default_rng(31)
    for G in (32, 128):
        V = rng.standard_normal((4, 2 * G)) * 10.0 ** rng.integers(-3, 3, (4, 1))
        V[1, :G] = 0.0
        V[2, :8] = [127.0, 63.5, -0.5, 2.5, -3.5, 0.0, -0.0, 1.5]
        V[2, 8:G] = rng.uniform(-1.0, 1.0, G - 8)
        Wb = bf16_from_float(V)
        q, sb = quantize8(Wb, G)
        assert q.dtype == np.int8 and q.shape == V.shape and sb.dtype == np.uint16
        v = f32_from_bf16(Wb)
        sf = f32_from_bf16(sb)
        for n in range(V.shape[0]):
            for g in range(V.shape[1] // G):
                grp = [Fraction(float(t)) for t in v[n, g * G:(g + 1) * G]]
                s_exact = _bf16_of_f32(_fl32_of(max(abs(t) for t in grp) / 127))
                assert Fraction(float(sf[n, g])) == s_exact, (G, n, g)
                for j, t in enumerate(grp):
                    want = 0 if s_exact == 0 else max(-127, min(127, _rne_int(_fl32_of(t / s_exact))))
                    assert int(q[n, g * G + j]) == want, (G, n, g, j)
        w = np.repeat(sf.astype(np.float64), G, axis=1)
        assert np.all(np.abs(q.astype(np.int32)) <= 127)
        assert np.all(np.abs(q * w - v) <= w * (0.5 + 2.0**-20) + 1e-300)
        assert np.all(q[1, :G] == 0) and np.all(sb[1, 0] == 0)
        qn, sbn = quantize8(bf16_from_float(-V), G)
        assert np.array_equal(sbn, sb) and np.array_equal(qn.astype(np.int32), -q.astype(np.int32))
    # linear on exact grid weights: W = q * 2^-e per group
    M, N, K, G = 3, 20, 256, 64
    qg = rng.integers(-127, 128, (N, K))
    qg[np.arange(N), rng.integers(0, K, N)] = 127          # every row reaches the max
    qg[:, ::G] = 127                                       # every group too
    e = rng.integers(6, 12, (N, K // G))
    W = qg * (2.0 ** -np.repeat(e, G, axis=1))
    Wb = bf16_from_float(W)
    assert np.array_equal(f32_from_bf16(Wb).astype(np.float64), W)
    q, sb = quantize8(Wb, G)
    assert np.array_equal(q.astype(np.int64), qg), "grid weights must encode exactly"
    x = bf16_from_float(rng.standard_normal((M, K)))
    bias = bf16_from_float(rng.standard_normal((1, N)))[0]
    y = linear8(x, q, sb, G, bias)
    theirs = (torch.from_numpy(f32_from_bf16(x).astype(np.float64)) @
              torch.from_numpy(W).T).numpy() + f32_from_bf16(bias).astype(np.float64)
    assert np.allclose(y, theirs, rtol=1e-12, atol=1e-12 * np.abs(theirs).max())


def check_rel_frobenius(rel_frobenius):
    """The acceptance metric ||y - y_ref||_F / ||y_ref||_F against values
    worked out by hand, chosen so that normalising by ||y||, or taking the
    largest element difference, gives a different number."""
    # one difference: |(3, 0)| / |(0, 4)| = 3 / 4
    assert rel_frobenius(np.array([3.0, 4.0]), np.array([0.0, 4.0])) == 0.75
    # two differences (3 and 4): 5 / 4; ||y|| = sqrt(41), max |diff| = 4
    assert rel_frobenius(np.array([3.0, 4.0, 4.0]), np.array([0.0, 4.0, 0.0])) == 1.25
    # matrices: element-wise over all entries, 13 / 5 with diff (5, 12, 0, 0)
    y_ref = np.array([[3.0, 0.0], [0.0, 4.0]])
    y = y_ref + np.array([[5.0, 12.0], [0.0, 0.0]])
    assert rel_frobenius(y, y_ref) == 13.0 / 5.0
    # scale invariance (powers of two keep every step exact) and symmetry in sign
    assert rel_frobenius(y * 1024.0, y_ref * 1024.0) == 13.0 / 5.0
    assert rel_frobenius(-y, -y_ref) == 13.0 / 5.0
    # exact agreement, and the degenerate zero reference
    assert rel_frobenius(y_ref, y_ref) == 0.0
    assert rel_frobenius(np.zeros(3), np.zeros(3)) == 0.0
    assert rel_frobenius(np.ones(3), np.zeros(3)) == float("inf")


def run_all_pins(mod):
    """Every pin against an oracle module-like object."""
    if hasattr(mod, "rel_frobenius"):
        check_rel_frobenius(mod.rel_frobenius)
    check_bf16_helper(mod.f32_to_bf16_bits)
    check_golden_halfsteps(mod.quantize_ref)
    check_golden_special(mod.quantize_ref)
    rng = np.random.default_rng(3)
    for G in (32, 64):
        W = bf16_from_float(rng.standard_normal((2, 2 * G)) * 0.02)
        check_brute_force(mod.quantize_ref, W, G)
        V = rng.standard_normal((6, 2 * G)) * 10.0 ** rng.integers(-3, 3, (6, 1))
        V[1, :G] = 0.25
        check_invariants(mod.quantize_ref, mod.dequant_ref, bf16_from_float(V), G)
    check_grid_exact(mod.quantize_ref, mod.dequant_ref, mod.linear_ref,
                     3, 24, 256, 64, seed=9, with_bias=True)
    if hasattr(mod, "fake_quant_ref"):
        V = rng.standard_normal((8, 256)) * 10.0 ** rng.integers(-3, 3, (8, 1))
        V[2, :32] = -1.5
        check_fake_quant(mod.fake_quant_ref, mod.quantize_ref, bf16_from_float(V), 32)
    if hasattr(mod, "repack_preshuffled_ref"):
        check_preshuffle(mod.repack_preshuffled_ref)
    if hasattr(mod, "quantize_int8_ref"):
        check_int8_weights(mod.quantize_int8_ref, mod.linear_int8_ref)
    if hasattr(mod, "act_quant_ref"):
        check_act_quant(mod.act_quant_ref)
        check_w4a8_linear(mod.w4a8_linear_ref, mod.linear_ref, mod.quantize_ref)
