"""Seeded synthetic inputs for the 2:4 SpMM workloads.

This module generates dense inputs only: it holds none of the method's
arithmetic (no selection, compression or product).  Both the GPU path's
callers (tests, bench) and the CPU oracle's callers draw their inputs here,
so the two sides see bit-identical data.

Recipe, per workload:
* a torch CPU generator per operand, seeded ``1000 + i`` for A, ``2000 + i``
  for B and ``3000 + i`` for the mask of workload ``i``;
* floating-point values are drawn in fp32 (``randn`` times the stated sigma)
  and rounded to nearest-even into fp16 / bf16;
* int8 values are drawn with ``randint`` over the stated closed range;
* 8-bit float (OCP E4M3 / E5M2) values are drawn in fp32 and converted by
  torch's round-to-nearest-even;
* the moderately-unstructured workload keeps each A element independently
  with probability 0.5 (``rand < 0.5``); dropped elements are set to +0 with
  ``torch.where`` so a negative value never turns into -0.

The shapes follow LLM projection layers: 11008 x 4096 is a 7B-class FFN
weight and 28672 x 8192 a 70B-class FFN weight; 16 columns of B is a decode
batch, 2048 a prefill chunk.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch

TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8,
               "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2,
               "i4": torch.uint8}   # 4-bit integers, two per byte (storage only)
FP8 = ("e4m3", "e5m2")


@dataclass(frozen=True)
class Workload:
    key: str
    title: str
    dtype: str            # "f16" | "bf16" | "i8" | "e4m3" | "e5m2" | "i4" (weights only)
    M: int
    K: int
    N: int
    index: int            # seeds are 1000+index, 2000+index, 3000+index
    a_sigma: float = 1.0  # fp: A ~ N(0, a_sigma^2)
    a_range: tuple = (-127, 127)   # int8: A uniform over this closed range
    b_range: tuple = (-128, 127)   # int8: B uniform over this closed range
    keep_prob: Optional[float] = None   # moderately-unstructured mask
    klass: str = "latency"              # "latency" | "large_n" | "small_n"
    b_dtype: Optional[str] = None       # B's element type when it differs from A's (4-bit weights: fp16)

    def with_shape(self, M=None, K=None, N=None) -> "Workload":
        """Same distribution and seeds at another shape (for reduced-size tests)."""
        return replace(self, M=self.M if M is None else M, K=self.K if K is None else K,
                       N=self.N if N is None else N)

    @property
    def residual(self) -> bool:
        return self.keep_prob is not None


WORKLOADS = {
    "c1": Workload("c1", "fp16 2:4 SpMM M=256 K=256 N=64", "f16", 256, 256, 64, 1, a_sigma=1.0),
    "c2": Workload("c2", "int8 2:4 SpMM M=K=N=4096", "i8", 4096, 4096, 4096, 2, klass="large_n"),
    "c3": Workload("c3", "fp16 decode-shape SpMM M=11008 K=4096 N=16", "f16", 11008, 4096, 16, 3,
                   a_sigma=0.02, klass="small_n"),
    "c4": Workload("c4", "bf16 prefill-shape SpMM M=28672 K=8192 N=2048", "bf16", 28672, 8192, 2048, 4,
                   a_sigma=0.02, klass="large_n"),
    "c5": Workload("c5", "fp16 moderately-unstructured SpMM M=K=8192 N=16 (50% mask, 2:4 + residual)",
                   "f16", 8192, 8192, 16, 5, a_sigma=0.02, keep_prob=0.5, klass="small_n"),
    # the decode and prefill shapes again with 8-bit float (OCP E4M3) operands
    "c3f8": Workload("c3f8", "fp8 (E4M3) decode-shape SpMM M=11008 K=4096 N=16", "e4m3", 11008, 4096, 16, 6,
                     a_sigma=0.02, klass="small_n"),
    "c4f8": Workload("c4f8", "fp8 (E4M3) prefill-shape SpMM M=28672 K=8192 N=2048", "e4m3", 28672, 8192, 2048, 7,
                     a_sigma=0.02, klass="large_n"),
    # the decode shape as the dense weight that N:M patterns other than 2:4
    # (1:4, 2:8, 4:8) are selected from
    "c3nm": Workload("c3nm", "fp16 N:M decode-shape SpMM M=11008 K=4096 N=16", "f16", 11008, 4096, 16, 8,
                     a_sigma=0.02, klass="small_n"),
    # the decode shape with 4-bit weights (uniform over [-8, 7]) and fp16 activations
    "c3w4": Workload("c3w4", "4-bit-weight N:M decode-shape SpMM M=11008 K=4096 N=16 (fp16 activations)", "i4",
                     11008, 4096, 16, 9, klass="small_n", b_dtype="f16"),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def pack_i4(v) -> np.ndarray:
    """4-bit two's-complement storage of integers in [-8, 7]: element k of a
    row in the low nibble of byte k/2 for even k, the high nibble for odd k."""
    v = np.asarray(v, dtype=np.int64)
    if v.shape[-1] % 2 or (v < -8).any() or (v > 7).any():
        raise ValueError("pack_i4 takes an even number of columns of values in [-8, 7]")
    u = (v & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def gen_a(w: Workload) -> torch.Tensor:
    """Dense A [M, K] on the CPU (before any pruning); 4-bit weights as
    [M, K/2] bytes."""
    g = _gen(1000 + w.index)
    if w.dtype == "i4":
        a = torch.randint(-8, 8, (w.M, w.K), generator=g, dtype=torch.int8)
        return torch.from_numpy(pack_i4(a.numpy()))
    if w.dtype == "i8":
        lo, hi = w.a_range
        a = torch.randint(lo, hi + 1, (w.M, w.K), generator=g, dtype=torch.int8)
    else:
        a = (torch.randn((w.M, w.K), generator=g, dtype=torch.float32) * w.a_sigma).to(TORCH_DTYPE[w.dtype])
    if w.keep_prob is not None:
        keep = torch.rand((w.M, w.K), generator=_gen(3000 + w.index)) < w.keep_prob
        a = torch.where(keep, a, torch.zeros((), dtype=a.dtype))
    return a


def gen_b(w: Workload) -> torch.Tensor:
    """Dense B [K, N] on the CPU."""
    g = _gen(2000 + w.index)
    bt = w.b_dtype or w.dtype
    if bt == "i8":
        lo, hi = w.b_range
        return torch.randint(lo, hi + 1, (w.K, w.N), generator=g, dtype=torch.int8)
    return torch.randn((w.K, w.N), generator=g, dtype=torch.float32).to(TORCH_DTYPE[bt])


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a CPU tensor as numpy: uint16 bit patterns for fp16/bf16, int8 as is."""
    t = t.contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.int8, torch.uint8):
        return t.numpy()
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        return t.view(torch.uint8).numpy()
    raise TypeError("unsupported dtype %s" % (t.dtype,))


def from_bits(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Inverse of bits(): a CPU tensor of the named dtype sharing nothing with a."""
    a = np.ascontiguousarray(a)
    if dtype == "i8":
        return torch.from_numpy(a.astype(np.int8, copy=True))
    if dtype == "i4":
        return torch.from_numpy(a.astype(np.uint8, copy=True))
    if dtype in FP8:
        return torch.from_numpy(a.astype(np.uint8, copy=True)).view(TORCH_DTYPE[dtype])
    return torch.from_numpy(a.astype(np.uint16, copy=True).view(np.int16)).view(TORCH_DTYPE[dtype])


# ---------------------------------------------------------------- small random families for tests

def store_dtype(dt: str):
    return np.int8 if dt == "i8" else (np.uint8 if dt in FP8 or dt == "i4" else np.uint16)


def encode(dt: str, values) -> np.ndarray:
    """Raw storage (numpy) of float values in dt, rounded to nearest-even."""
    v = np.asarray(values, dtype=np.float64)
    if dt == "i8":
        return v.astype(np.int8)
    if dt == "i4":
        return pack_i4(v.astype(np.int64))
    if dt == "f16":
        return v.astype(np.float16).view(np.uint16)
    if dt in FP8:
        # fp32 first, then torch's round-to-nearest-even into the 8-bit format
        t = torch.from_numpy(v.astype(np.float32)).to(TORCH_DTYPE[dt])
        return t.view(torch.uint8).numpy().copy()
    t = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def random_matrix(dt: str, M: int, K: int, family: str, seed: int) -> np.ndarray:
    """Raw storage of a random [M, K] matrix.

    families: "normal" (continuous), "ties" (few distinct magnitudes, zeros and
    -0), "sparse" (about half the entries +0), "extreme" (int8 -128/127 or
    large/small fp magnitudes)."""
    rng = np.random.default_rng(seed)
    if dt == "i4":                                   # [M, K/2] bytes
        if family == "normal":
            a = rng.integers(-8, 8, size=(M, K))
        elif family == "ties":
            a = rng.choice([-2, -1, 0, 1, 2], size=(M, K))
        elif family == "sparse":
            a = rng.integers(-8, 8, size=(M, K)) * (rng.random((M, K)) < 0.5)
        else:
            a = rng.choice([-8, -7, 7, 0, 1, -1], size=(M, K))
        return pack_i4(a)
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
    if dt == "e4m3" and family == "extreme":
        v = rng.choice([-448.0, 448.0, 2.0 ** -9, -2.0 ** -9, 0.0, -0.0, 1.0], size=(M, K))
    if dt == "e5m2" and family == "extreme":
        v = rng.choice([-57344.0, 57344.0, 2.0 ** -16, -2.0 ** -16, 0.0, -0.0, 1.0], size=(M, K))
    return encode(dt, v)


