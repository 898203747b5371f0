"""Shared test helpers: locating/building the HIP library and moving seeded bits to the GPU."""
import os
import re

import numpy as np

import fa_inputs as FI

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def ensure_built():
    """Load libfa.so, building it first only when no built library exists."""
    import exact_attention_27_amd as fa
    if not os.path.exists(fa.LIB_PATH):
        from exact_attention_27_amd import build
        build.build()
    return fa.load_library()


def header_functions():
    """Names of every function declared in include/fa.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(fa_\w+)\s*\(", text, flags=re.M)))


def to_device(bits: np.ndarray, dtype: str, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)
    return t.view(torch.bfloat16 if dtype == FI.BF16 else torch.float16)


def from_device(t, dtype: str) -> np.ndarray:
    import torch
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return FI.bits_to_f64(bits, dtype)


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of each (already rounded) 16-bit value."""
    mant_bits = 7 if dtype == FI.BF16 else 10
    _, e = np.frexp(np.abs(x))
    ulp = np.ldexp(1.0, e - 1 - mant_bits)
    if dtype == FI.FP16:
        ulp = np.maximum(ulp, 2.0 ** -24)
    ulp = np.where(x == 0, 2.0 ** -24 if dtype == FI.FP16 else 2.0 ** -133, ulp)
    return 0.5 * ulp


def map_threads(fn, items, workers: int = 8):
    """[fn(x) for x in items] on a small thread pool (numpy releases the GIL in its matrix
    products and large elementwise operations, so oracle calls on separate heads overlap)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=max(1, min(workers, len(items)))) as ex:
        return list(ex.map(fn, items))
