"""Independent helpers for the tests: decoding through numpy/torch, brute-force
selection by pair enumeration, and small random input families.  Nothing here
calls the oracle or the GPU library."""
from __future__ import annotations

import itertools

import numpy as np
import torch

PAIRS = list(itertools.combinations(range(4), 2))   # (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
VALID_NIBBLES = {p | (q << 2) for p, q in PAIRS}     # {0x4, 0x8, 0xC, 0x9, 0xD, 0xE}


def to_f64(dt: str, a: np.ndarray) -> np.ndarray:
    """Values of raw storage as float64, decoded by numpy (fp16) or torch (bf16)."""
    a = np.ascontiguousarray(a)
    if dt == "i8":
        return a.astype(np.float64)
    if dt == "f16":
        return a.view(np.float16).astype(np.float64)
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def to_i64(a: np.ndarray) -> np.ndarray:
    return np.asarray(a).astype(np.int64)


def brute_pair(mags) -> tuple:
    """Kept positions of one group by enumerating all 6 pairs: the pair whose
    (larger, smaller) magnitude pair is greatest; among equals, the
    lexicographically smallest positions."""
    best = None
    for p, q in PAIRS:
        key = (max(mags[p], mags[q]), min(mags[p], mags[q]))
        if best is None or key > best[0]:
            best = (key, (p, q))
    return best[1]


def brute_keep_mask(dt: str, A: np.ndarray) -> np.ndarray:
    """Boolean keep mask [M, K] by pair enumeration (python loops: small inputs)."""
    mag = np.abs(to_f64(dt, A))
    M, K = A.shape
    keep = np.zeros((M, K), dtype=bool)
    for m in range(M):
        for g in range(K // 4):
            p, q = brute_pair(list(mag[m, 4 * g:4 * g + 4]))
            keep[m, 4 * g + p] = keep[m, 4 * g + q] = True
    return keep


def store_dtype(dt: str):
    return np.int8 if dt == "i8" else np.uint16


def encode(dt: str, values) -> np.ndarray:
    """Raw storage of float values (exactly representable ones) in dt."""
    v = np.asarray(values, dtype=np.float64)
    if dt == "i8":
        return v.astype(np.int8)
    if dt == "f16":
        return v.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def random_matrix(dt: str, M: int, K: int, family: str, seed: int) -> np.ndarray:
    """Raw storage of a random [M, K] matrix.

    families: "normal" (continuous), "ties" (few distinct magnitudes, zeros and
    -0), "sparse" (about half the entries +0), "extreme" (int8 -128/127 or
    large/small fp magnitudes)."""
    rng = np.random.default_rng(seed)
    if dt == "i8":
        if family == "normal":
            a = rng.integers(-127, 128, size=(M, K))
        elif family == "ties":
            a = rng.choice([-2, -1, 0, 1, 2], size=(M, K))
        elif family == "sparse":
            a = rng.integers(-127, 128, size=(M, K)) * (rng.random((M, K)) < 0.5)
        else:
            a = rng.choice([-128, -127, 127, 0, 1, -1], size=(M, K))
        return a.astype(np.int8)
    if family == "normal":
        v = rng.standard_normal((M, K))
    elif family == "ties":
        v = rng.choice([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0], size=(M, K))
    elif family == "sparse":
        v = rng.standard_normal((M, K)) * (rng.random((M, K)) < 0.5)
    else:
        v = rng.choice([-60000.0, 60000.0, 1e-7, -1e-7, 0.0, -0.0, 1.0], size=(M, K))
    if dt == "bf16" and family == "extreme":
        v = rng.choice([-3e38, 3e38, 1e-40, -1e-40, 0.0, -0.0, 1.0], size=(M, K))
    return encode(dt, v)


def is_zero(dt: str, a: np.ndarray) -> np.ndarray:
    return to_f64(dt, a) == 0.0
