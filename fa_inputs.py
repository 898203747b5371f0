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


LOGIT_PATTERNS = ("far_negative", "rising", "dominant_last", "near_tau")


def draw_bits_logit_pattern(pattern: str, B: int, H: int, N: int, d: int, dtype: str, seed: int) -> dict:
    """Inputs whose scaled logits s = Q K^T / sqrt(d) take a chosen shape, for the range
    limits of the exponential. Safe softmax subtracts the row max so that the result is the
    same for any shift of a row's logits ("FlashAttentionを1から", section "タイリングを阻む、
    softmaxという壁"); these recipes put rows where a kernel's running max and its rescale
    factors are pushed to their limits. The shapes, with e0 the first coordinate:

    * far_negative: Q = -4 + 0.5 z, K = 4 + 0.5 z elementwise, so every logit lies near
      -16 sqrt(d) (-128 at d = 64, -181 at d = 128), with a spread of about 3: exp of any
      of them underflows in float32, and a running max that starts at 0 is ~180 too high.
    * rising: Q = 128 e0 + 0.25 z; K[:, 0] a ramp over the keys, centred on zero, rising by
      12 logit units per 64 keys (other coordinates z): a row's max rises by 12 (17 in
      log2 units) on every 64-key tile, so any tiled pass has to move its reference on every
      tile; at N = 1000 the first keys sit near -94, below the float32 range of exp.
    * dominant_last: Q = 8 e0 + 0.25 z, K = 0.25 z except the last key, K[N-1, 0] = 40 in
      logit units: every row that sees the last key is dominated by it (its softmax weight
      is ~1 and the others' are ~e^-40); the reference jumps by ~40 at the last tile.
    * near_tau: Q = 8 e0 + 0.05 z, K = 0.25 z, with K[:, 0] a step of 5.4 logit units
      between the first 64 keys and the rest, centred so that the keys' mean is zero: the
      later keys exceed the first 64 by 5.4 (just under 8 in log2 units), so a pass that moves
      its reference only when a tile's max exceeds it by more than 2^8 accumulates
      probabilities close to 2^8 against the first tile's reference.

    z ~ N(0, 1) from numpy Generator(PCG64(seed)), drawn in the order Q, K, V, dO, each of
    shape (B, H, N, d); V and dO are z itself. Every tensor is rounded once to `dtype`.
    Apart from far_negative (whose keys must share a large common part), the keys that a row's
    softmax weights most differ from each other by more than they share, so that the
    gradient dQ_i = scale sum_j dS_ij K_j, which cancels any part common to the keys, is not
    dominated by the rounding of dS against that common part.
    """
    if pattern not in LOGIT_PATTERNS:
        raise ValueError(f"unknown logit pattern {pattern!r}")
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    z = {name: rng.standard_normal(size=shape, dtype=np.float64) for name in TENSOR_ORDER}
    root = float(np.sqrt(d))  # logit = (q . k) / root
    q, k = z["q"], z["k"]
    if pattern == "far_negative":
        q = -4.0 + 0.5 * q
        k = 4.0 + 0.5 * k
    elif pattern == "rising":
        a = 128.0
        q = 0.25 * q
        q[..., 0] = a
        k[..., 0] = (12.0 / 64.0) * (np.arange(N) - (N - 1) / 2.0) * root / a
    elif pattern == "dominant_last":
        a = 8.0
        q = 0.25 * q
        q[..., 0] = a
        k = 0.25 * k
        k[..., N - 1, 0] = 40.0 * root / a
    else:  # near_tau
        a = 8.0
        q = 0.05 * q
        q[..., 0] = a
        k = 0.25 * k
        frac = max(N - 64, 0) / N  # share of keys past the first 64
        k[..., :64, 0] = -5.4 * frac * root / a
        k[..., 64:, 0] = 5.4 * (1.0 - frac) * root / a
    return {"q": round_bits(q, dtype), "k": round_bits(k, dtype), "v": round_bits(z["v"], dtype),
            "do": round_bits(z["do"], dtype)}


def varlen_lengths(n_seq: int, n_max: int, seed: int) -> np.ndarray:
    """A seeded mix of sequence lengths for variable-length batches: n_seq lengths drawn
    uniformly from [n_max // 8, n_max] (numpy PCG64), the last forced to n_max so the
    longest sequence is always present. Returns int64 lengths."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = rng.integers(max(1, n_max // 8), n_max + 1, size=n_seq)
    lengths[-1] = n_max
    return lengths.astype(np.int64)
