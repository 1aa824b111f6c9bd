"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke
check. Holds no arithmetic of the method: it draws normal samples, scales
them and casts to bf16 (torch's own round-to-nearest-even cast), and returns
raw bf16 bits.

The shapes stand in for the workloads the pages name (Llama-3-8B int4
decode, Gemma3-12B, a 32768^2 sweep-scale layer). No weights or datasets are
available, so random layers of the same shapes are used:
W ~ N(0, 0.02), x ~ N(0, 1), both cast to bf16.
"""
from __future__ import annotations

import math

import numpy as np
import torch

# Rows per independently seeded block of a generated matrix: any block of
# rows can be regenerated on its own (sampled checks at full size).
ROW_BLOCK = 256

# Layer shapes [N, K] (out_features, in_features).
LLAMA3_8B = {           # decode layer set of a Llama-3-8B-shaped block
    "qkv": (6144, 4096),
    "o": (4096, 4096),
    "gate_up": (28672, 4096),
    "down": (4096, 14336),
}
GEMMA3_12B = {          # hidden 3840, 16 heads x 256, 8 KV heads, MLP 15360
    "q": (4096, 3840),
    "k": (2048, 3840),
    "v": (2048, 3840),
    "o": (3840, 4096),
    "gate": (15360, 3840),
    "up": (15360, 3840),
    "down": (3840, 15360),
}
SQUARE = {"square": (32768, 32768)}

CONFIGS = {
    1: dict(name="tiny", layers={"linear": (512, 512)}, G=(32,), M=(1,),
            outliers=False),
    2: dict(name="llama3_8b_decode", layers=LLAMA3_8B, G=(128,), M=(1,),
            outliers=False),
    3: dict(name="llama3_8b_m16_outliers", layers=LLAMA3_8B, G=(32, 64),
            M=(16,), outliers=True),
    4: dict(name="gemma3_12b_prefill", layers=GEMMA3_12B, G=(128,),
            M=(2048,), outliers=False),
    5: dict(name="square_32768", layers=SQUARE, G=(64,), M=(1, 32768),
            outliers=False),
}


def w_seed(config: int) -> int:
    """Config i (1-based) draws its weights from seed i - 1."""
    return config - 1


def x_seed(config: int) -> int:
    return 1000 + config - 1


def _block_generator(seed: int, block: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed((seed * 1_000_003 + block * 7919 + 12345) % (2**63 - 1))
    return g


def outlier_columns(K: int, seed: int) -> np.ndarray:
    """round(1% of K) distinct input columns, chosen by a seeded permutation."""
    n_out = int(round(0.01 * K))
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 424242)
    perm = torch.randperm(K, generator=g)
    return np.sort(perm[:n_out].numpy())


def normal_bf16_rows(N: int, K: int, std: float, seed: int,
                     row0: int = 0, row1: int | None = None,
                     outlier_cols: np.ndarray | None = None,
                     outlier_factor: float = 20.0) -> np.ndarray:
    """Rows [row0, row1) of an [N, K] matrix of bf16 bits.

    Each block of ROW_BLOCK rows has its own generator, so a row subset is
    reproduced without drawing the rest. Outlier columns are multiplied in
    float32 before the bf16 cast.
    """
    if row1 is None:
        row1 = N
    out = np.empty((row1 - row0, K), dtype=np.uint16)
    b0 = row0 // ROW_BLOCK
    b1 = (row1 + ROW_BLOCK - 1) // ROW_BLOCK
    for b in range(b0, b1):
        r0 = b * ROW_BLOCK
        r1 = min(N, r0 + ROW_BLOCK)
        t = torch.randn(r1 - r0, K, generator=_block_generator(seed, b),
                        dtype=torch.float32) * std
        if outlier_cols is not None and len(outlier_cols):
            t[:, torch.from_numpy(np.asarray(outlier_cols))] *= outlier_factor
        bits = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        lo = max(r0, row0)
        hi = min(r1, row1)
        out[lo - row0:hi - row0] = bits[lo - r0:hi - r0]
    return out


def weight_bits(config: int, layer: str, rows=None) -> np.ndarray:
    """bf16 bits of the synthetic weight W[N, K] of a config's layer."""
    cfg = CONFIGS[config]
    N, K = cfg["layers"][layer]
    names = sorted(cfg["layers"])
    seed = w_seed(config) * 100 + names.index(layer)
    oc = outlier_columns(K, seed) if cfg["outliers"] else None
    if rows is None:
        return normal_bf16_rows(N, K, 0.02, seed, outlier_cols=oc)
    return normal_bf16_rows(N, K, 0.02, seed, rows[0], rows[1], outlier_cols=oc)


def activation_bits(config: int, M: int, K: int, rows=None) -> np.ndarray:
    """bf16 bits of the synthetic activation x[M, K] ~ N(0, 1)."""
    seed = x_seed(config) * 100 + (K % 97) + 13 * int(math.log2(max(M, 1)) + 1)
    if rows is None:
        return normal_bf16_rows(M, K, 1.0, seed)
    return normal_bf16_rows(M, K, 1.0, seed, rows[0], rows[1])


def random_bf16(shape, std: float, seed: int) -> np.ndarray:
    """Small ad-hoc bf16 matrices for edge-case tests."""
    N, K = shape
    return normal_bf16_rows(N, K, std, seed)
