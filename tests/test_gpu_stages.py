"""GPU: the backward stages called one by one, against fa_backward and the fp64 oracle.

fa_backward runs two launches: dQ, whose workgroups also compute D_i = sum_c dO_ic O_ic for
their own rows and write delta (fa_backward_dq_delta), then dK/dV (fa_backward_dkv). The
pages' three-kernel split ("Triton 05: Flash Attention", section "3단계 커널 구조") stays
available as fa_backward_preprocess, fa_backward_dkv and fa_backward_dq. For each problem:

  * fa_backward_dq_delta then fa_backward_dkv give, bit for bit, what fa_backward gives (the
    same kernels in the same order);
  * the three-stage form matches the oracle to the parity tolerances of
    tests/test_gpu_parity.py (dQ, dK, dV relative Frobenius error <= 2e-2; delta within 1e-2
    of ||dO_i|| ||O_i||);
  * the two forms' delta agree to fp32 summation order: |D_a - D_b| <= 1e-5 (||dO_i|| ||O_i||)
    (each is a sum of d products of 16-bit values in fp32, in a different order).

Outputs are pre-filled with NaN.
"""
import numpy as np
import pytest

import fa_inputs as FI
from oracle import attention as ORACLE
from tests import _lib

pytestmark = pytest.mark.gpu

TOL_GRAD = 2e-2
TOL_DELTA = 1e-2


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    _lib.ensure_built()
    import exact_attention_27_amd as fa_mod
    return fa_mod


CASES = [((1, 2, 1, 64), FI.BF16, True), ((2, 3, 200, 64), FI.FP16, False), ((1, 2, 300, 128), FI.BF16, True),
         ((1, 2, 257, 128), FI.FP16, True), ((2, 2, 130, 96), FI.BF16, False), ((1, 2, 150, 256), FI.BF16, True),
         ((1, 512, 300, 128), FI.BF16, True)]


@pytest.mark.parametrize("shape,dtype,causal", CASES,
                         ids=[f"{'x'.join(map(str, s))}-{dt}-{'c' if c else 'f'}" for s, dt, c in CASES])
def test_stages(fa, shape, dtype, causal):
    import torch
    seed = 9500 + CASES.index((shape, dtype, causal))
    print(f"case {shape} {dtype} causal={causal} seed={seed}", flush=True)
    bits = FI.draw_bits(shape, dtype, seed)
    B, H, N, d = shape
    scale = d ** -0.5
    q, k, v, do = (_lib.to_device(bits[n], dtype) for n in FI.TENSOR_ORDER)
    nan = float("nan")
    o = torch.full_like(q, nan)
    lse = torch.full((B, H, N), nan, dtype=torch.float32, device=q.device)
    fa.fa_forward(q, k, v, o, lse, causal, scale)

    def fresh():
        return ([torch.full_like(q, nan) for _ in range(3)]
                + [torch.full((B, H, N), nan, dtype=torch.float32, device=q.device)])

    dq_b, dk_b, dv_b, de_b = fresh()
    fa.fa_backward(q, k, v, o, do, lse, dq_b, dk_b, dv_b, de_b, causal, scale)
    dq_c, dk_c, dv_c, de_c = fresh()
    fa.fa_backward_dq_delta(q, k, v, o, do, lse, dq_c, de_c, causal, scale)
    fa.fa_backward_dkv(q, k, v, do, lse, de_c, dk_c, dv_c, causal, scale)
    dq_a, dk_a, dv_a, de_a = fresh()
    fa.fa_backward_preprocess(o, do, de_a)
    fa.fa_backward_dkv(q, k, v, do, lse, de_a, dk_a, dv_a, causal, scale)
    fa.fa_backward_dq(q, k, v, do, lse, de_a, dq_a, causal, scale)
    torch.cuda.synchronize()

    for x, y, name in ((dq_b, dq_c, "dq"), (dk_b, dk_c, "dk"), (dv_b, dv_c, "dv"), (de_b, de_c, "delta")):
        assert x.equal(y), f"{name}: the two stage calls differ from fa_backward"

    o_np = _lib.from_device(o, dtype)
    got = {"dq": _lib.from_device(dq_a, dtype), "dk": _lib.from_device(dk_a, dtype),
           "dv": _lib.from_device(dv_a, dtype)}
    d_a, d_b = de_a.cpu().numpy().astype(np.float64), de_b.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(d_a)) and np.all(np.isfinite(d_b))
    for arr in got.values():
        assert np.all(np.isfinite(arr))
    for b in range(B):
        for h in ([0, H // 2, H - 1] if H > 8 else range(H)):
            qf, kf, vf, dof = (FI.bits_to_f64(bits[n][b, h], dtype) for n in FI.TENSOR_ORDER)
            ref = ORACLE.backward(qf, kf, vf, dof, scale, causal)
            # (one key: dQ = dK = 0 exactly, up to the rounding difference between the two
            # evaluations of dO.V; compared absolutely, as in the parity tests)
            rel = {g: float(np.linalg.norm(got[g][b, h] - ref[g]) / np.linalg.norm(ref[g]))
                   if np.linalg.norm(ref[g]) > 1e-12 else float(np.abs(got[g][b, h]).max()) * TOL_GRAD / 1e-3
                   for g in got}
            norm = np.linalg.norm(dof, axis=1) * np.linalg.norm(o_np[b, h], axis=1) + 1e-30
            dref = float((np.abs(d_a[b, h] - ref["delta"]) / norm).max())
            dab = float((np.abs(d_a[b, h] - d_b[b, h]) / norm).max())
            print(f"  b{b}h{h}: " + " ".join(f"{g}={r:.3g}" for g, r in rel.items())
                  + f" delta={dref:.3g} delta_two_forms={dab:.3g}", flush=True)
            for g, r in rel.items():
                assert r <= TOL_GRAD, (g, r)
            assert dref <= TOL_DELTA, dref
            assert dab <= 1e-5, dab
