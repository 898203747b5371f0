"""GPU parity of the split-KV forward (fa_forward_splitkv) against the fp64 oracle.

The split forward computes softmax states over disjoint key ranges and merges them; the result
is the same exact attention as the single-pass forward, so the forward tolerances apply
unchanged: max(|O_gpu - O_ref| - half_ulp(O_gpu)) <= 1e-2 and max|LSE_gpu - LSE_ref| <= 1e-3.
Outputs and the workspace are pre-filled with NaN, so a partial state or output row that is
never written cannot pass. Split counts include 1 (one range: the merge of a single state)
and counts above the number of key tiles (empty ranges, merged with weight zero).
"""
import numpy as np
import pytest

import fa_inputs as FI
from oracle import attention as ORACLE
from tests import _lib

pytestmark = pytest.mark.gpu

TOL_O = 1e-2
TOL_LSE = 1e-3


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    _lib.ensure_built()
    import exact_attention_27_amd as fa_mod
    return fa_mod


def split_forward(fa, bits, dtype, causal, scale, splits):
    import torch
    q, k, v = (_lib.to_device(bits[n], dtype) for n in ("q", "k", "v"))
    B, H, N, d = q.shape
    nan = float("nan")
    o = torch.full_like(q, nan)
    lse = torch.full((B, H, N), nan, dtype=torch.float32, device=q.device)
    nbytes = fa.fa_forward_splitkv_workspace_bytes(B, H, N, d, splits)
    ws = torch.full((nbytes // 4,), nan, dtype=torch.float32, device=q.device)
    fa.fa_forward_splitkv(q, k, v, o, lse, causal, scale, splits, ws)
    torch.cuda.synchronize()
    o_np, lse_np = _lib.from_device(o, dtype), lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o_np)) and np.all(np.isfinite(lse_np)), "unwritten or non-finite output"
    return o_np, lse_np


def check_heads(o, lse, bits, dtype, causal, scale, heads, label):
    for b, h in heads:
        q, k, v = (FI.bits_to_f64(bits[n][b, h], dtype) for n in ("q", "k", "v"))
        o_ref, lse_ref = ORACLE.forward(q, k, v, scale, causal)
        gate = float((np.abs(o[b, h] - o_ref) - _lib.half_ulp(o[b, h], dtype)).max())
        lerr = float(np.abs(lse[b, h] - lse_ref).max())
        print(f"{label} b{b}h{h}: o_gate={gate:.3g} lse={lerr:.3g}", flush=True)
        assert gate <= TOL_O and lerr <= TOL_LSE, (label, b, h, gate, lerr)


CASES = [("single_head", False, 1), ("single_head", False, 3), ("single_head", True, 2),
         ("single_head", True, 16), ("small_causal", True, 4), ("small_causal", True, 7)]


@pytest.mark.parametrize("key,causal,splits", CASES,
                         ids=[f"{k}-{'c' if c else 'f'}-s{s}" for k, c, s in CASES])
def test_split_forward_small_workloads(fa, key, causal, splits):
    w = FI.WORKLOADS[key]
    bits = FI.draw_workload(w)
    o, lse = split_forward(fa, bits, w.dtype, causal, w.scale(), splits)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    check_heads(o, lse, bits, w.dtype, causal, w.scale(), heads, f"{key} causal={causal} splits={splits}")


EDGES = [s for s in FI.edge_shapes() if s[2] in (17, 257, 1000)]


@pytest.mark.parametrize("shape", EDGES, ids=[f"N{s[2]}-d{s[3]}-{s[4]}-{'c' if s[5] else 'f'}" for s in EDGES])
def test_split_forward_edge_shapes(fa, shape):
    B, H, N, d, dtype, causal, seed = shape
    bits = FI.draw_bits((B, H, N, d), dtype, seed)
    for splits in (2, 5):
        o, lse = split_forward(fa, bits, dtype, causal, d ** -0.5, splits)
        check_heads(o, lse, bits, dtype, causal, d ** -0.5, [(0, h) for h in range(H)],
                    f"edge {shape} splits={splits}")


def test_split_matches_single_pass(fa):
    """Same inputs through fa_forward and fa_forward_splitkv. P is rounded to 16 bits against
    each pass's own reference max (the split ranges start fresh), so the two differ by that
    rounding (relative 2^-9 per probability), not bit for bit: they must agree within the
    forward tolerances above."""
    import torch
    bits = FI.draw_bits((2, 3, 777, 128), FI.BF16, 81)
    q, k, v = (_lib.to_device(bits[n], FI.BF16) for n in ("q", "k", "v"))
    o1, lse1 = fa.attention_forward(q, k, v, True)
    o2 = torch.empty_like(q)
    lse2 = torch.empty_like(lse1)
    fa.fa_forward_splitkv(q, k, v, o2, lse2, True, 128 ** -0.5, 3)
    torch.cuda.synchronize()
    a, b = _lib.from_device(o1, FI.BF16), _lib.from_device(o2, FI.BF16)
    diff = float(np.abs(a - b).max())
    ldiff = float((lse1 - lse2).abs().max())
    print(f"split vs single pass: max|dO|={diff:.3g} max|dLSE|={ldiff:.3g}", flush=True)
    assert diff <= TOL_O and ldiff <= TOL_LSE


@pytest.mark.timeout(600)
def test_split_forward_full_size_sampled(fa):
    """The headline shape with 2 splits: two heads compared row by row on sampled rows."""
    w = FI.WORKLOADS["llm_layer"]
    bits = FI.draw_workload(w)
    o, lse = split_forward(fa, bits, w.dtype, True, w.scale(), 2)
    rows = np.concatenate([np.arange(128), np.random.Generator(np.random.PCG64(11)).integers(128, w.N, 256)])
    for b, h in ((0, 0), (3, 31)):
        q, k, v = (FI.bits_to_f64(bits[n][b, h], w.dtype) for n in ("q", "k", "v"))
        o_ref, lse_ref = ORACLE.forward_rows(q, k, v, w.scale(), True, rows)
        gate = float((np.abs(o[b, h][rows] - o_ref) - _lib.half_ulp(o[b, h][rows], w.dtype)).max())
        lerr = float(np.abs(lse[b, h][rows] - lse_ref).max())
        print(f"llm_layer splits=2 b{b}h{h} sampled rows: o_gate={gate:.3g} lse={lerr:.3g}", flush=True)
        assert gate <= TOL_O and lerr <= TOL_LSE
