"""Independent helpers for the tests: decoding through numpy/torch, brute-force
selection by pair enumeration, and small random input families.  Nothing here
calls the oracle or the GPU library."""
from __future__ import annotations

import itertools

import numpy as np
import torch

from workloads import TORCH_DTYPE, encode, random_matrix, store_dtype  # noqa: F401  (seeded input families)

PAIRS = list(itertools.combinations(range(4), 2))   # (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
VALID_NIBBLES = {p | (q << 2) for p, q in PAIRS}     # {0x4, 0x8, 0xC, 0x9, 0xD, 0xE}


def to_f64(dt: str, a: np.ndarray) -> np.ndarray:
    """Values of raw storage as float64, decoded by numpy (fp16) or torch (bf16, fp8)."""
    a = np.ascontiguousarray(a)
    if dt == "i4":                                   # two 4-bit integers per byte, low nibble first
        lo = (a & 0xF).astype(np.int64)
        hi = (a >> 4).astype(np.int64)
        v = np.stack([lo, hi], axis=-1).reshape(a.shape[0], -1)
        return np.where(v >= 8, v - 16, v).astype(np.float64)
    if dt == "i8":
        return a.astype(np.float64)
    if dt == "f16":
        return a.view(np.float16).astype(np.float64)
    if dt in ("e4m3", "e5m2"):
        t = torch.from_numpy(a.view(np.uint8).copy()).view(TORCH_DTYPE[dt])
        return t.to(torch.float64).numpy()
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


def is_zero(dt: str, a: np.ndarray) -> np.ndarray:
    return to_f64(dt, a) == 0.0


NM_PATTERNS = [(1, 4), (2, 4), (2, 8), (4, 8)]     # the N:M patterns the GPU library implements


def brute_subset(mags, n: int) -> tuple:
    """Kept positions of one group of len(mags) by enumerating every n-subset:
    the subset whose magnitudes, sorted descending, are greatest; among
    equals, the lexicographically smallest positions (itertools yields the
    subsets in that order, so the first best one is kept)."""
    best = None
    for sub in itertools.combinations(range(len(mags)), n):
        key = tuple(sorted((mags[p] for p in sub), reverse=True))
        if best is None or key > best[0]:
            best = (key, sub)
    return best[1]


def brute_keep_mask_nm(dt: str, A: np.ndarray, n: int, m: int) -> np.ndarray:
    """Boolean N:M keep mask [M, K] by subset enumeration (python loops: small inputs)."""
    mag = np.abs(to_f64(dt, A))
    M, K = mag.shape
    keep = np.zeros((M, K), dtype=bool)
    for r in range(M):
        for g in range(K // m):
            for p in brute_subset(list(mag[r, m * g:m * g + m]), n):
                keep[r, m * g + p] = True
    return keep


def mask_bits(mask: np.ndarray, K: int) -> np.ndarray:
    """Boolean [M, K] of a per-row bitmask (bit k % 8 of byte k / 8)."""
    return np.unpackbits(np.ascontiguousarray(mask, dtype=np.uint8), axis=1, bitorder="little")[:, :K].astype(bool)
