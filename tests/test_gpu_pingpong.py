"""GPU parity of the two-group ping-pong forward (fa_forward_pingpong).

The ping-pong schedule reorders which waves run which half of a step and when tiles are
copied, never the arithmetic of a row: every query row goes through the same products,
exponentials and sums in the same order as in fa_forward. Its O and LSE are therefore
compared with fa_forward's bit for bit, over shapes that exercise one partial tile, ragged
tails, the causal diagonal, both dtypes, head dims that run the 128-wide tiles (d = 96, 128)
and ones that fall back to the default schedule (d = 64, 256), and grids with and without
the causal heavy + light pairing. fa_forward is itself compared with the fp64 oracle by the
other parity tests; one case here is also compared with the oracle directly, and the
exponent-range patterns of the extreme-logit tests are run through both entry points.
Outputs are pre-filled with NaN.
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


def both(fa, bits, dtype, causal, scale):
    import torch
    q, k, v = (_lib.to_device(bits[n], dtype) for n in ("q", "k", "v"))
    B, H, N, d = q.shape
    nan = float("nan")
    outs = []
    for fn in (fa.fa_forward, fa.fa_forward_pingpong):
        o = torch.full_like(q, nan)
        lse = torch.full((B, H, N), nan, dtype=torch.float32, device=q.device)
        fn(q, k, v, o, lse, causal, scale)
        outs.append((o, lse))
    torch.cuda.synchronize()
    return outs


# (B, H, N, d): one partial tile, ragged tails around the 256-row tile, several tiles, the
# 128-wide kernel at d = 96, the default schedule at d = 64 and 256, a grid that pairs causal
# tiles (B*H*8 pairs >= 2 per CU), one that pairs them with an odd middle tile running alone
# (three 256-row tiles per head), and one that does not pair
SHAPES = [(1, 2, 1, 128), (1, 2, 37, 128), (2, 3, 255, 128), (1, 2, 257, 128), (1, 3, 1000, 96),
          (1, 2, 700, 64), (1, 2, 300, 256), (2, 8, 2048, 128), (4, 32, 4096, 128), (1, 512, 600, 128)]
CASES = [(s, dt, c) for s in SHAPES for dt in (FI.BF16, FI.FP16) for c in (False, True)
         if not (s[0] * s[1] * s[2] >= 4 * 32 * 4096 and dt == FI.FP16)]


@pytest.mark.parametrize("shape,dtype,causal", CASES,
                         ids=[f"{'x'.join(map(str, s))}-{dt}-{'c' if c else 'f'}" for s, dt, c in CASES])
def test_bit_identical_to_forward(fa, shape, dtype, causal):
    seed = 9100 + SHAPES.index(shape) * 4 + 2 * (dtype == FI.BF16) + causal
    print(f"case {shape} {dtype} causal={causal} seed={seed}", flush=True)
    bits = FI.draw_bits(shape, dtype, seed)
    (o0, l0), (o1, l1) = both(fa, bits, dtype, causal, shape[3] ** -0.5)
    assert not o1.isnan().any() and not l1.isnan().any(), "unwritten output"
    assert o0.equal(o1), "O differs from fa_forward"
    assert l0.equal(l1), "LSE differs from fa_forward"


def test_against_oracle(fa):
    shape, dtype, causal = (1, 2, 300, 128), FI.BF16, True
    bits = FI.draw_bits(shape, dtype, 9199)
    scale = shape[3] ** -0.5
    (_, _), (o, lse) = both(fa, bits, dtype, causal, scale)
    o_np, lse_np = _lib.from_device(o, dtype), lse.cpu().numpy().astype(np.float64)
    for h in range(shape[1]):
        q, k, v = (FI.bits_to_f64(bits[n][0, h], dtype) for n in ("q", "k", "v"))
        o_ref, lse_ref = ORACLE.forward(q, k, v, scale, causal)
        gate = float((np.abs(o_np[0, h] - o_ref) - _lib.half_ulp(o_np[0, h], dtype)).max())
        lerr = float(np.abs(lse_np[0, h] - lse_ref).max())
        print(f"h{h}: o_gate={gate:.3g} lse={lerr:.3g}", flush=True)
        assert gate <= TOL_O and lerr <= TOL_LSE, (h, gate, lerr)


@pytest.mark.parametrize("pattern", FI.LOGIT_PATTERNS)
def test_extreme_logits_bit_identical(fa, pattern):
    for dtype in (FI.BF16, FI.FP16):
        for causal in (False, True):
            bits = FI.draw_bits_logit_pattern(pattern, 1, 2, 1000, 128, dtype, 9300 + causal)
            (o0, l0), (o1, l1) = both(fa, bits, dtype, causal, 128 ** -0.5)
            assert o0.equal(o1) and l0.equal(l1), (pattern, dtype, causal)
