"""GPU: head dims other than 64 and 128 (multiples of 8 up to 256).

Such a head dim runs on the 64-, 128- or 256-wide kernels with the columns past d zero on chip
(loads past d read zero, stores past d are skipped), which leaves every dot product
unchanged. Checked here:
  * parity with the fp64 oracle on every head, forward and backward, to the tolerances of
    tests/test_gpu_parity.py (ragged N, both masks, both element types);
  * nothing is written past column d: the outputs sit in buffers whose extra columns (and
    extra rows after the tensor) are NaN before the call and must still be NaN after it;
  * the split-KV forward at such a head dim.
"""
import numpy as np
import pytest

import fa_inputs as FI
from oracle import attention as ORACLE
from tests import _lib
from tests.test_gpu_parity import check, head_metrics, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    _lib.ensure_built()
    import exact_attention_27_amd as fa_mod
    return fa_mod


CASES = [
    # d, N, dtype, causal
    (8, 70, FI.BF16, True),
    (32, 190, FI.BF16, True),
    (32, 129, FI.FP16, False),
    (40, 257, FI.FP16, True),
    (72, 100, FI.BF16, False),
    (96, 333, FI.BF16, True),
    (96, 64, FI.FP16, False),
    (120, 150, FI.BF16, True),
    (136, 100, FI.FP16, True),
    (192, 257, FI.BF16, False),
    (256, 300, FI.BF16, True),
    (256, 129, FI.FP16, False),
]


@pytest.mark.parametrize("case", CASES, ids=[f"d{c[0]}-N{c[1]}-{c[2]}-{'c' if c[3] else 'f'}" for c in CASES])
def test_head_dim_parity(fa, case):
    d, N, dtype, causal = case
    B, H = 1, 2
    bits = FI.draw_bits((B, H, N, d), dtype, 5000 + d + N)
    scale = d ** -0.5
    gpu = run_gpu(fa, bits, dtype, causal, scale)
    for h in range(H):
        check(head_metrics(gpu, bits, dtype, 0, h, scale, causal), f"d={d} N={N} {dtype} causal={causal} h{h}")


def test_nothing_written_past_head_dim(fa):
    import torch
    B, H, N, d, pad, dtype, causal = 2, 2, 150, 96, 32, FI.BF16, True
    bits = FI.draw_bits((B, H, N, d), dtype, 5100)
    q, k, v, do = (_lib.to_device(bits[n], dtype) for n in FI.TENSOR_ORDER)
    scale = d ** -0.5

    def padded():
        # (B, N, H, d) view of a (B, N, H, d + pad) NaN buffer, with 4 spare NaN rows after it
        buf = torch.full((B * N * H * (d + pad) + 4 * H * (d + pad),), float("nan"), dtype=q.dtype, device=q.device)
        return buf, buf[: B * N * H * (d + pad)].view(B, N, H, d + pad)[..., :d]

    def load(t):
        buf, view = padded()
        view.copy_(t.transpose(1, 2))
        return view

    qs, ks, vs, dos = (load(t) for t in (q, k, v, do))
    (ob, o), (dqb, dq), (dkb, dk), (dvb, dv) = padded(), padded(), padded(), padded()
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    delta = torch.full_like(lse, float("nan"))
    fa.fa_forward_ex(qs, ks, vs, o, lse, causal, scale, layout="bnhd")
    fa.fa_backward_ex(qs, ks, vs, o, dos, lse, dq, dk, dv, delta, causal, scale, layout="bnhd")
    torch.cuda.synchronize()
    for name, buf, view in (("o", ob, o), ("dq", dqb, dq), ("dk", dkb, dk), ("dv", dvb, dv)):
        assert torch.isfinite(view).all(), name
        body = buf[: B * N * H * (d + pad)].view(B, N, H, d + pad)
        assert torch.isnan(body[..., d:]).all(), f"{name}: a column past d was written"
        assert torch.isnan(buf[B * N * H * (d + pad):]).all(), f"{name}: a row past the tensor was written"
    assert torch.isfinite(lse).all() and torch.isfinite(delta).all()
    # the values: oracle on one head
    o_np = _lib.from_device(o.transpose(1, 2), dtype)
    qf, kf, vf = (FI.bits_to_f64(bits[n][1, 1], dtype) for n in ("q", "k", "v"))
    o_ref, lse_ref = ORACLE.forward(qf, kf, vf, scale, causal)
    gate = float((np.abs(o_np[1, 1] - o_ref) - _lib.half_ulp(o_np[1, 1], dtype)).max())
    assert gate <= 1e-2 and float(np.abs(lse[1, 1].cpu().numpy() - lse_ref).max()) <= 1e-3


@pytest.mark.parametrize("d,splits", [(40, 3), (96, 2), (256, 2)])
def test_head_dim_splitkv(fa, d, splits):
    import torch
    B, H, N, dtype, causal = 1, 2, 300, FI.BF16, True
    bits = FI.draw_bits((B, H, N, d), dtype, 5200 + d)
    q, k, v = (_lib.to_device(bits[n], dtype) for n in ("q", "k", "v"))
    scale = d ** -0.5
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    nbytes = fa.fa_forward_splitkv_workspace_bytes(B, H, N, d, splits)
    assert nbytes == splits * B * H * N * ((64 if d <= 64 else 128 if d <= 128 else 256) + 2) * 4
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=q.device)
    fa.fa_forward_splitkv(q, k, v, o, lse, causal, scale, splits, ws)
    torch.cuda.synchronize()
    o_np = _lib.from_device(o, dtype)
    for h in range(H):
        qf, kf, vf = (FI.bits_to_f64(bits[n][0, h], dtype) for n in ("q", "k", "v"))
        o_ref, lse_ref = ORACLE.forward(qf, kf, vf, scale, causal)
        gate = float((np.abs(o_np[0, h] - o_ref) - _lib.half_ulp(o_np[0, h], dtype)).max())
        lerr = float(np.abs(lse[0, h].cpu().numpy() - lse_ref).max())
        print(f"split d={d} s={splits} h{h}: o_gate={gate:.3g} lse={lerr:.3g}", flush=True)
        assert gate <= 1e-2 and lerr <= 1e-3


@pytest.mark.parametrize("d", [64, 96, 256])
def test_paired_tiles_many_heads(fa, d):
    """Many heads make the causal grid large enough for tile pairing (a heavy and a light Q or
    K tile per workgroup; N = 300 gives an odd middle tile that runs alone), which the other
    small shapes here do not reach. Sampled heads against the oracle, forward and backward;
    every head finite."""
    import torch
    B, H, N, dtype, causal = 1, 512, 300, FI.BF16, True
    bits = FI.draw_bits((B, H, N, d), dtype, 5300 + d)
    scale = d ** -0.5
    gpu = run_gpu(fa, bits, dtype, causal, scale)
    for h in (0, 257, 511):
        check(head_metrics(gpu, bits, dtype, 0, h, scale, causal), f"paired d={d} h{h}")
