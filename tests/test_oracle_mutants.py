"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pins catch every one of them."""
import types

import pytest

from oracle import ref
from tests import pins

MUTANTS = {
    "scale_over_16": ("d / np.float32(15.0)", "d / np.float32(16.0)"),
    "no_signed_zero_canon": ("lo = v.min(axis=2) + np.float32(0.0)", "lo = v.min(axis=2)"),
    "zero_is_max": ("z_bits = (lo.view", "z_bits = (hi.view"),
    "round_half_up": ("np.clip(np.rint(quot)", "np.clip(np.floor(quot + 0.5)"),
    "truncate": ("np.clip(np.rint(quot)", "np.clip(np.trunc(quot)"),
    "reciprocal_multiply": (
        "quot = np.divide(num, np.where(zero_scale, np.float32(1.0), s_b),",
        "quot = np.multiply(num, np.float32(1.0) / np.where(zero_scale, np.float32(1.0), s_b),"),
    "scale_truncated_to_bf16": (
        "s_bits = f32_to_bf16_bits(s32)",
        "s_bits = (s32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)"),
    "nibbles_swapped": (
        "codes = (q[:, 0::2] | (q[:, 1::2] << np.uint8(4)))",
        "codes = (q[:, 1::2] | (q[:, 0::2] << np.uint8(4)))"),
    "dequant_drops_zero": (
        "return q * np.repeat(s, G, axis=1) + np.repeat(z, G, axis=1)",
        "return q * np.repeat(s, G, axis=1)"),
    "dequant_wrong_group_index": (
        "return q * np.repeat(s, G, axis=1) + np.repeat(z, G, axis=1)",
        "return q * np.tile(s, (1, G)) + np.tile(z, (1, G))"),
    "linear_reversed_k": ("y[:, n0:n1] = x @ w.T", "y[:, n0:n1] = x @ w[:, ::-1].T"),
    "bias_sign": ("y += bf16_bits_to_f32", "y -= bf16_bits_to_f32"),
    "zero_scale_code_15": ("q = np.where(zero_scale, 0.0, q)", "q = np.where(zero_scale, 15.0, q)"),
    "bf16_round_half_up": (
        "u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))",
        "u = u + np.uint64(0x8000)"),
    "range_min_min": ("hi = v.max(axis=2) + np.float32(0.0)", "hi = v.min(axis=2) + np.float32(1.0)"),
    "fake_quant_drops_zero": ("w = (prod + z).astype(np.float32)", "w = prod.astype(np.float32)"),
    "fake_quant_truncates": (
        "    return f32_to_bf16_bits(w)\n",
        "    return (w.view(np.uint32) >> np.uint32(16)).astype(np.uint16)\n"),
    "fake_quant_scale_unrounded": (
        "    s = np.repeat(bf16_bits_to_f32(s_bits), G, axis=1)\n    z = np.repeat(bf16_bits_to_f32(z_bits), G, axis=1)\n    prod",
        "    s = np.repeat(bf16_bits_to_f32(s_bits) * np.float32(1.0 + 2.0**-9), G, axis=1)\n    z = np.repeat(bf16_bits_to_f32(z_bits), G, axis=1)\n    prod"),
    "preshuffle_odd_first": (
        "nib = np.concatenate([words[:, :, 0::2], words[:, :, 1::2]], axis=2)",
        "nib = np.concatenate([words[:, :, 1::2], words[:, :, 0::2]], axis=2)"),
    "preshuffle_bytes_high_first": (
        "b = (nib[:, :, 0::2] | (nib[:, :, 1::2] << np.uint8(4))).astype(np.uint8)",
        "b = (nib[:, :, 1::2] | (nib[:, :, 0::2] << np.uint8(4))).astype(np.uint8)"),
    "preshuffle_natural_nibbles": (
        "nib = np.concatenate([words[:, :, 0::2], words[:, :, 1::2]], axis=2)",
        "nib = words"),
    "act_scale_over_128": (
        "sx = (a / np.float32(127.0)).astype(np.float32)",
        "sx = (a / np.float32(128.0)).astype(np.float32)"),
    "act_round_half_up": ("code = np.clip(np.rint(ratio), -127.0, 127.0)",
                          "code = np.clip(np.floor(ratio + 0.5), -127.0, 127.0)"),
    "act_truncate": ("code = np.clip(np.rint(ratio), -127.0, 127.0)",
                     "code = np.clip(np.trunc(ratio), -127.0, 127.0)"),
    "act_reciprocal_multiply": (
        "ratio = np.divide(v, np.where(zero, np.float32(1.0), sx)[:, None],\n                      dtype=np.float32)",
        "ratio = np.multiply(v, (np.float32(1.0) / np.where(zero, np.float32(1.0), sx))[:, None],\n                        dtype=np.float32)"),
    "w4a8_drops_zero_term": ("acc += P * s[None, :, g] + X[:, None] * z[None, :, g]",
                             "acc += P * s[None, :, g]"),
    "w4a8_no_token_scale": (
        "y = np.asarray(sx, dtype=np.float32).astype(np.float64)[:, None] * acc",
        "y = acc.copy()"),
    "w4a8_group_shift": ("sl = slice(g * G, (g + 1) * G)", "sl = slice(g * G + 1, (g + 1) * G + 1)"),
    "int8_scale_over_128": ("f32_to_bf16_bits((amax / np.float32(127.0)).astype(np.float32))",
                            "f32_to_bf16_bits((amax / np.float32(128.0)).astype(np.float32))"),
    "int8_scale_unrounded": (
        "sc = np.broadcast_to(bf16_bits_to_f32(scale_bits)[:, :, None], v.shape)",
        "sc = np.broadcast_to((amax / np.float32(127.0)).astype(np.float32)[:, :, None], v.shape)"),
    "int8_round_half_up": ("np.clip(np.rint(t), -127.0, 127.0)", "np.clip(np.floor(t + 0.5), -127.0, 127.0)"),
    "int8_linear_scale_tiled": ("w = q8 * np.repeat(sc, G, axis=1)", "w = q8 * np.tile(sc, (1, G))"),
    "int8_linear_no_bias": (
        "        y = y + bf16_bits_to_f32(np.asarray(bias_bits, dtype=np.uint16)).astype(np.float64)\n    return y\n\n\ndef act_quant_ref",
        "        y = y + 0.0\n    return y\n\n\ndef act_quant_ref"),
    "range_includes_zero": (
        "    lo = v.min(axis=2) + np.float32(0.0)\n    hi = v.max(axis=2) + np.float32(0.0)\n",
        "    lo = np.minimum(v.min(axis=2), np.float32(0.0)) + np.float32(0.0)\n"
        "    hi = np.maximum(v.max(axis=2), np.float32(0.0)) + np.float32(0.0)\n"),
    "clamp_to_14": ("np.clip(np.rint(quot), 0.0, 15.0)", "np.clip(np.rint(quot), 0.0, 14.0)"),
    "dequant_rounded_to_bf16": (
        "return q * np.repeat(s, G, axis=1) + np.repeat(z, G, axis=1)",
        "return bf16_bits_to_f32(f32_to_bf16_bits((q * np.repeat(s, G, axis=1) + "
        "np.repeat(z, G, axis=1)).astype(np.float32))).astype(np.float64)"),
    "rel_frobenius_over_y": ("den = np.linalg.norm(y_ref)", "den = np.linalg.norm(y)"),
    "rel_frobenius_max_abs": ("num = np.linalg.norm(y - y_ref)", "num = np.abs(y - y_ref).max()"),
    "preshuffle_sz_swapped": (
        "return codes_ps, (s | (z << np.uint32(16))).astype(np.uint32)",
        "return codes_ps, (z | (s << np.uint32(16))).astype(np.uint32)"),
}


def _mutant_module(old, new):
    src = open(ref.__file__).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = ref.__file__
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def test_unmutated_oracle_passes_all_pins():
    pins.run_all_pins(ref)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mod = _mutant_module(*MUTANTS[name])
    with pytest.raises((AssertionError, ValueError)):
        pins.run_all_pins(mod)
