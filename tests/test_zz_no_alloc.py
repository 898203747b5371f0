"""fa_backward_noalloc (the backward whose delta workspace is the library's own device array)
against fa_backward, through the C ABI, on two calls in a row -- the second with a smaller
problem, so it reuses the array the first one filled -- and one more large call after it.
The two entry points run the same kernels on the same inputs, so dQ, dK and dV must agree bit
for bit; the first call is also checked against the fp64 oracle on two heads at the parity
gates. Outputs are pre-filled with NaN."""
import numpy as np
import pytest

import fa_inputs as FI
from oracle import attention as ORACLE
from tests import _lib

pytestmark = pytest.mark.gpu

TOL_GRAD = 2e-2


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    _lib.ensure_built()
    import exact_attention_27_amd as fa_mod
    return fa_mod


def _problem(fa, shape, dtype, causal, seed):
    import torch
    bits = FI.draw_bits(shape, dtype, seed)
    q, k, v, do = (_lib.to_device(bits[n], dtype) for n in FI.TENSOR_ORDER)
    scale = shape[3] ** -0.5
    o, lse = fa.attention_forward(q, k, v, causal, scale)
    return bits, (q, k, v, do, o, lse), scale


def _both(fa, tens, causal, scale):
    import torch
    q, k, v, do, o, lse = tens
    nan = float("nan")
    ref = [torch.full_like(q, nan) for _ in range(3)]
    delta = torch.full(lse.shape, nan, dtype=torch.float32, device=q.device)
    fa.fa_backward(q, k, v, o, do, lse, *ref, delta, causal, scale)
    got = [torch.full_like(q, nan) for _ in range(3)]
    fa.fa_backward_noalloc(q, k, v, o, do, lse, *got, causal, scale)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dtype,causal", [(FI.BF16, True), (FI.FP16, False)])
def test_noalloc_matches_fa_backward(fa, dtype, causal):
    import torch
    shapes = [(2, 4, 1000, 128, 9401), (1, 3, 129, 64, 9402), (4, 8, 2048, 96, 9403)]
    for i, (B, H, N, d, seed) in enumerate(shapes):
        print(f"call {i}: B={B} H={H} N={N} d={d} {dtype} causal={causal} seed={seed}", flush=True)
        bits, tens, scale = _problem(fa, (B, H, N, d), dtype, causal, seed)
        ref, got = _both(fa, tens, causal, scale)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert bool(torch.isfinite(b).all()), (i, name)
            assert torch.equal(a, b), (i, name, float((a.float() - b.float()).abs().max()))
        if i == 0:
            for b_, h in ((0, 0), (B - 1, H - 1)):
                q, k, v, do = (FI.bits_to_f64(bits[n][b_, h], dtype) for n in FI.TENSOR_ORDER)
                r = ORACLE.backward(q, k, v, do, scale, causal)
                for name, t in zip(("dq", "dk", "dv"), got):
                    g = _lib.from_device(t, dtype)[b_, h]
                    rel = float(np.linalg.norm(g - r[name]) / np.linalg.norm(r[name]))
                    assert rel <= TOL_GRAD, (name, b_, h, rel)


def test_noalloc_limit(fa):
    import torch
    limit = fa.fa_backward_noalloc_max_rows()
    assert limit == 1 << 22
    # B*H*N one row past the array: refused before anything is enqueued
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 1, 8, dtype=torch.float32, device="cuda")
    lib = fa.load_library()
    import ctypes
    vp = ctypes.c_void_p
    p = vp(q.data_ptr())
    st = lib.fa_backward_noalloc(p, p, p, p, p, vp(lse.data_ptr()), p, p, p, 1, 1, limit + 1, 64, 0, 0.125,
                                 fa.FA_BF16, vp(0))
    assert st == fa.FA_ERR_UNSUPPORTED
