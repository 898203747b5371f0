"""Seeded synthetic inputs for the exact-attention path: shapes, seeds, draws, rounding.

This module holds none of the attention arithmetic. It only fixes *which* bits the
two sides of every parity check see: the HIP path (through torch device tensors)
and the fp64 CPU oracle (through an exact upcast of the same bits). Neither side's
arithmetic lives here, and nothing here imports either side.

Recipe (fixed before any result was seen):

* numpy ``Generator(PCG64(seed))``, ``standard_normal`` in float64, drawn in the
  order Q, K, V, dO, each of shape (B, H, N, d);
* the long-context workload multiplies Q by 4 before rounding (exact: a power of
  two), which makes logits large and stresses the running-max rescale;
* each tensor is rounded ONCE, round-to-nearest-even, straight from float64 to
  the storage type (fp16 or bf16) -- no intermediate float32 step, so there is no
  double rounding.

The workload shapes follow the pages: the single-head and small causal cases,
the GPT-2-medium shape of the FlashAttention v1 IO table ("FlashAttention·FA4·FP4",
section on the cost of computing vs storing N x N, Figure 2 left table: B=64, H=16,
N=1024, d=64), and the d=128 shapes of the FA4 forward plots (same page, section on
what remains after HBM is saved, Figure 4).
"""
from __future__ import annotations

import dataclasses
from typing import Iterator

import numpy as np

FP16 = "fp16"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    label: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: tuple  # which mask settings the workload is run with
    seed: int
    q_mult: float = 1.0

    @property
    def shape(self) -> tuple:
        return (self.B, self.H, self.N, self.d)

    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.d))


WORKLOADS = {
    "single_head": Workload("single_head", "B=1 H=1 N=256 d=64 fp16 (non-causal and causal)",
                            1, 1, 256, 64, FP16, (False, True), 1001),
    "small_causal": Workload("small_causal", "B=1 H=8 N=1024 d=64 fp16 causal",
                             1, 8, 1024, 64, FP16, (True,), 1002),
    "gpt2_medium": Workload("gpt2_medium", "B=64 H=16 N=1024 d=64 fp16 non-causal",
                            64, 16, 1024, 64, FP16, (False,), 1003),
    "llm_layer": Workload("llm_layer", "B=4 H=32 N=4096 d=128 bf16 causal",
                          4, 32, 4096, 128, BF16, (True,), 1004),
    "long_context": Workload("long_context", "B=1 H=16 N=16384 d=128 bf16 causal, Q scaled by 4",
                             1, 16, 16384, 128, BF16, (True,), 1005, q_mult=4.0),
}
HEADLINE = "llm_layer"


# ----------------------------------------------------------------------------- rounding

_TWO_M126 = 2.0 ** -126


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 -> bfloat16 (round-to-nearest-even, one rounding), return uint16 bits.

    Normal range: round the 52-bit fp64 mantissa to bf16's 7 stored bits directly on
    the fp64 bit pattern (add 2^44-1 plus the lowest kept bit, truncate); a mantissa
    carry rolls into the exponent, which is the correct result. The rounded value has
    at most 8 significant bits, so converting it to float32 is exact and the top 16
    bits of that float32 are the bf16 encoding. Values below 2^-126 in magnitude
    (bf16 subnormals) are quantised to multiples of 2^-133 with numpy's rint (RNE).
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    rounded = (bits + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    y = rounded.view(np.float64)
    tiny = np.abs(x) < _TWO_M126
    if np.any(tiny):
        y = y.copy()
        y[tiny] = np.ldexp(np.rint(np.ldexp(x[tiny], 133)), -133)
    with np.errstate(over="ignore"):
        f32 = y.astype(np.float32)
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to float64."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 -> IEEE binary16 with round-to-nearest-even (numpy's direct conversion)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def fp16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return f64_to_bf16_bits(x)
    if dtype == FP16:
        return f64_to_fp16_bits(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def bits_to_f64(b: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return bf16_bits_to_f64(b)
    if dtype == FP16:
        return fp16_bits_to_f64(b)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# ----------------------------------------------------------------------------- draws

TENSOR_ORDER = ("q", "k", "v", "do")


def draw_bits(shape, dtype: str, seed: int, q_mult: float = 1.0) -> dict:
    """Draw Q, K, V, dO ~ N(0,1) (Q times q_mult) in that order and round each once.

    Returns a dict of uint16 bit arrays of the given (B, H, N, d) shape.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name in TENSOR_ORDER:
        x = rng.standard_normal(size=shape, dtype=np.float64)
        if name == "q" and q_mult != 1.0:
            x *= q_mult
        out[name] = round_bits(x, dtype)
        del x
    return out


def draw_bits_rect(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, seed: int) -> dict:
    """Inputs with Nq query rows and Nk key rows: draw_bits over max(Nq, Nk) rows, then Q and
    dO keep their first Nq rows and K and V their first Nk (contiguous copies)."""
    bits = draw_bits((B, H, max(Nq, Nk), d), dtype, seed)
    rows = {"q": Nq, "k": Nk, "v": Nk, "do": Nq}
    return {n: np.ascontiguousarray(bits[n][:, :, :rows[n]]) for n in TENSOR_ORDER}


def draw_workload(w: Workload) -> dict:
    return draw_bits(w.shape, w.dtype, w.seed, w.q_mult)


def edge_shapes() -> Iterator[tuple]:
    """Extra parity shapes: ragged N (not a multiple of any tile), B*H=1, tiny N.

    Yields (B, H, N, d, dtype, causal, seed). Seeds are fixed here.
    """
    seed = 2000
    for d in (64, 128):
        for dtype in (FP16, BF16):
            for N in (1, 17, 257, 1000):
                for causal in (False, True):
                    seed += 1
                    yield (1, 2, N, d, dtype, causal, seed)


def varlen_lengths(n_seq: int, n_max: int, seed: int) -> np.ndarray:
    """A seeded mix of sequence lengths for variable-length batches: n_seq lengths drawn
    uniformly from [n_max // 8, n_max] (numpy PCG64), the last forced to n_max so the
    longest sequence is always present. Returns int64 lengths."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = rng.integers(max(1, n_max // 8), n_max + 1, size=n_seq)
    lengths[-1] = n_max
    return lengths.astype(np.int64)
