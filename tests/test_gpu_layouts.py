"""GPU: strided operands and variable-length batches (fa_forward_ex / fa_backward_ex).

Two kinds of checks:
  * bit-identity with the contiguous path. A strided operand changes only where rows are
    read and written, and a packed sequence is computed with the same tiles as the same
    sequence alone, so O, LSE, dQ, dK, dV and delta must be equal bit for bit;
  * parity with the fp64 oracle per sequence and head for variable lengths, to the same
    tolerances as tests/test_gpu_parity.py.
Every output buffer is pre-filled with NaN, so an unwritten row cannot pass.
"""
import numpy as np
import pytest

import fa_inputs as FI
from oracle import attention as ORACLE
from tests import _lib

pytestmark = pytest.mark.gpu

TOL_O = 1e-2
TOL_LSE = 1e-3
TOL_GRAD = 2e-2


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    _lib.ensure_built()
    import exact_attention_27_amd as fa_mod
    return fa_mod


def nan_like(t):
    import torch
    return torch.full_like(t, float("nan"))


def contiguous_run(fa, q, k, v, do, causal, scale):
    """fa_forward + fa_backward on contiguous (B, H, N, d) tensors."""
    import torch
    B, H, N, _ = q.shape
    o = nan_like(q)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    fa.fa_forward(q, k, v, o, lse, causal, scale)
    dq, dk, dv = nan_like(q), nan_like(k), nan_like(v)
    delta = nan_like(lse)
    fa.fa_backward(q, k, v, o, do, lse, dq, dk, dv, delta, causal, scale)
    return o, lse, dq, dk, dv, delta


def bnhd_views(base, shape_bnhd, pad):
    """(B, N, H, d) views of `base`'s values whose rows sit in a larger buffer (pad extra
    elements after each head's d values), i.e. strides that are neither contiguous nor dense."""
    import torch
    B, N, H, d = shape_bnhd
    buf = torch.full((B, N, H, d + pad), float("nan"), dtype=base.dtype, device=base.device)
    view = buf[..., :d]
    view.copy_(base)
    return view


LAYOUT_CASES = [
    # B, H, N, d, dtype, causal, pad
    (2, 3, 333, 64, FI.BF16, True, 0),
    (2, 3, 333, 128, FI.FP16, False, 0),
    (1, 4, 257, 128, FI.BF16, True, 8),
    (3, 2, 64, 64, FI.FP16, True, 16),
]


@pytest.mark.parametrize("case", LAYOUT_CASES, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}-{c[4]}-{'c' if c[5] else 'f'}-pad{c[6]}"
                                                   for c in LAYOUT_CASES])
def test_bnhd_layout_bit_identical(fa, case):
    import torch
    B, H, N, d, dtype, causal, pad = case
    bits = FI.draw_bits((B, H, N, d), dtype, 4100 + N + d)
    q, k, v, do = (_lib.to_device(bits[n], dtype) for n in FI.TENSOR_ORDER)
    scale = d ** -0.5
    ref = contiguous_run(fa, q, k, v, do, causal, scale)
    # (B, N, H, d) views, optionally with padded rows
    qs, ks, vs, dos = (bnhd_views(t.transpose(1, 2), (B, N, H, d), pad) for t in (q, k, v, do))
    o = bnhd_views(torch.full_like(qs, float("nan")), (B, N, H, d), pad)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    fa.fa_forward_ex(qs, ks, vs, o, lse, causal, scale, layout="bnhd")
    dq, dk, dv = (bnhd_views(torch.full_like(qs, float("nan")), (B, N, H, d), pad) for _ in range(3))
    delta = torch.full_like(lse, float("nan"))
    fa.fa_backward_ex(qs, ks, vs, o, dos, lse, dq, dk, dv, delta, causal, scale, layout="bnhd")
    torch.cuda.synchronize()
    got = (o.transpose(1, 2), lse, dq.transpose(1, 2), dk.transpose(1, 2), dv.transpose(1, 2), delta)
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv", "delta"), got, ref):
        assert torch.equal(a.contiguous().view(torch.int16) if a.dtype != torch.float32 else a,
                           b.contiguous().view(torch.int16) if b.dtype != torch.float32 else b), name


def test_packed_qkv_and_packed_gradient(fa):
    """Q, K, V as slices of one (B, N, 3, H, d) tensor, and dQ, dK, dV as slices of another:
    inputs overlap freely; the three output slices share no element and are accepted."""
    import torch
    B, H, N, d, dtype, causal = 2, 2, 190, 128, FI.BF16, True
    bits = FI.draw_bits((B, H, N, d), dtype, 4200)
    q, k, v, do = (_lib.to_device(bits[n], dtype) for n in FI.TENSOR_ORDER)
    scale = d ** -0.5
    ref = contiguous_run(fa, q, k, v, do, causal, scale)
    qkv = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).contiguous()  # (B, N, 3, H, d)
    qs, ks, vs = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    o = torch.full((B, N, H, d), float("nan"), dtype=q.dtype, device=q.device)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    fa.fa_forward_ex(qs, ks, vs, o, lse, causal, scale, layout="bnhd")
    dqkv = torch.full_like(qkv, float("nan"))
    delta = torch.full_like(lse, float("nan"))
    fa.fa_backward_ex(qs, ks, vs, o, do.transpose(1, 2).contiguous(), lse, dqkv[:, :, 0], dqkv[:, :, 1],
                      dqkv[:, :, 2], delta, causal, scale, layout="bnhd")
    torch.cuda.synchronize()
    assert torch.equal(o.transpose(1, 2).contiguous().view(torch.int16), ref[0].view(torch.int16))
    assert torch.equal(lse, ref[1]) and torch.equal(delta, ref[5])
    for i in range(3):
        assert torch.equal(dqkv[:, :, i].transpose(1, 2).contiguous().view(torch.int16), ref[2 + i].view(torch.int16))


def test_aliasing_outputs_refused(fa):
    import torch
    B, H, N, d = 1, 2, 64, 64
    q = torch.zeros(B, N, H, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(B, H, N, dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fa_forward_ex(q, q, q, q, lse, False, 0.125, layout="bnhd")
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    g = torch.zeros_like(q)
    with pytest.raises(fa.FAError) as e:
        fa.fa_backward_ex(q, q, q, torch.zeros_like(q), torch.zeros_like(q), lse, g, g, torch.zeros_like(q),
                          torch.zeros_like(lse), False, 0.125, layout="bnhd")
    assert e.value.status == fa.FA_ERR_INVALID_ARG


# --------------------------------------------------------------------- variable lengths

VARLEN_CASES = [
    # lengths, H, d, dtype, causal
    ((37, 1, 200, 0, 128, 65), 3, 64, FI.BF16, True),
    ((37, 1, 200, 0, 128, 65), 3, 128, FI.FP16, False),
    ((300, 5, 64), 2, 128, FI.BF16, True),
    ((1,), 1, 64, FI.FP16, True),
    ((37, 1, 130), 2, 96, FI.BF16, True),
    ((70, 200), 2, 256, FI.FP16, True),
]


def draw_varlen(lengths, H, d, dtype, seed):
    """Per-sequence seeded bits, each (1, H, n, d); returns them and the packed (T, H, d) bits."""
    seqs = [FI.draw_bits((1, H, n, d), dtype, seed + i) if n > 0 else None for i, n in enumerate(lengths)]
    packed = {}
    for name in FI.TENSOR_ORDER:
        parts = [s[name][0].transpose(1, 0, 2) for s in seqs if s is not None]  # (n, H, d)
        packed[name] = np.ascontiguousarray(np.concatenate(parts, axis=0))
    return seqs, packed


def run_varlen(fa, packed, lengths, dtype, causal, scale):
    import torch
    q, k, v, do = (_lib.to_device(packed[n], dtype) for n in FI.TENSOR_ORDER)
    T, H, d = q.shape
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=q.device)
    nmax = max(max(lengths), 1)
    o = nan_like(q)
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device=q.device)
    fa.fa_forward_ex(q, k, v, o, lse, causal, scale, cu_seqlens=cu, max_seqlen=nmax)
    dq, dk, dv = nan_like(q), nan_like(k), nan_like(v)
    delta = nan_like(lse)
    fa.fa_backward_ex(q, k, v, o, do, lse, dq, dk, dv, delta, causal, scale, cu_seqlens=cu, max_seqlen=nmax)
    torch.cuda.synchronize()
    return (q, k, v, do), (o, lse, dq, dk, dv, delta)


@pytest.mark.parametrize("case", VARLEN_CASES, ids=[f"L{'-'.join(map(str, c[0]))}-H{c[1]}d{c[2]}-{c[3]}-{'c' if c[4] else 'f'}"
                                                   for c in VARLEN_CASES])
def test_varlen_oracle_and_bit_identical(fa, case):
    import torch
    lengths, H, d, dtype, causal = case
    scale = d ** -0.5
    seqs, packed = draw_varlen(lengths, H, d, dtype, 4300 + d + len(lengths))
    _, (o, lse, dq, dk, dv, delta) = run_varlen(fa, packed, lengths, dtype, causal, scale)
    out = {"o": _lib.from_device(o, dtype), "dq": _lib.from_device(dq, dtype), "dk": _lib.from_device(dk, dtype),
           "dv": _lib.from_device(dv, dtype), "lse": lse.cpu().numpy().astype(np.float64)}
    for name in ("o", "dq", "dk", "dv", "lse"):
        assert np.all(np.isfinite(out[name])), name
    row0 = 0
    for i, n in enumerate(lengths):
        if n == 0:
            continue
        s = seqs[i]
        rows = slice(row0, row0 + n)
        # the same sequence alone through the contiguous path: bit for bit
        t = [_lib.to_device(s[nm], dtype) for nm in FI.TENSOR_ORDER]
        ref = contiguous_run(fa, *t, causal, scale)
        torch.cuda.synchronize()
        for name, got, r in (("o", o, ref[0]), ("dq", dq, ref[2]), ("dk", dk, ref[3]), ("dv", dv, ref[4])):
            assert torch.equal(got[rows].transpose(0, 1).contiguous().view(torch.int16), r[0].view(torch.int16)), (i, name)
        assert torch.equal(lse[:, rows], ref[1][0]) and torch.equal(delta[:, rows], ref[5][0]), i
        # and the oracle, head by head
        for h in range(H):
            qf, kf, vf, dof = (FI.bits_to_f64(s[nm][0, h], dtype) for nm in FI.TENSOR_ORDER)
            r = ORACLE.backward(qf, kf, vf, dof, scale, causal)
            og = out["o"][rows, h]
            gate = float((np.abs(og - r["o"]) - _lib.half_ulp(og, dtype)).max())
            lerr = float(np.abs(out["lse"][h, rows] - r["lse"]).max())
            msg = f"seq {i} (n={n}) h{h}: o_gate={gate:.3g} lse={lerr:.3g}"
            grads = {}
            for g in ("dq", "dk", "dv"):
                nref = np.linalg.norm(r[g])
                grads[g] = float(np.linalg.norm(out[g][rows, h] - r[g]) / nref) if nref > 0 else float(
                    np.abs(out[g][rows, h]).max())
            print(msg + " " + " ".join(f"{g}={e:.3g}" for g, e in grads.items()), flush=True)
            assert gate <= TOL_O and lerr <= TOL_LSE, msg
            if n == 1:
                # one key: dQ = dK = 0 up to the rounding gap between the two evaluations of dO.V
                assert grads["dq"] <= 1e-3 and grads["dk"] <= 1e-3, msg
                assert np.array_equal(out["dv"][rows, h], FI.bits_to_f64(s["do"][0, h], dtype)), msg
            else:
                for g in ("dq", "dk", "dv"):
                    assert grads[g] <= TOL_GRAD, (msg, g)
        row0 += n


def test_varlen_padding_rows_untouched(fa):
    """Packed rows past cu_seqlens[B] belong to no sequence: nothing writes them."""
    import torch
    lengths, H, d, dtype = (50, 70), 2, 64, FI.BF16
    seqs, packed = draw_varlen(lengths, H, d, dtype, 4400)
    q, k, v = (_lib.to_device(packed[n], dtype) for n in ("q", "k", "v"))
    T = q.shape[0]
    extra = 30
    qx, kx, vx = (torch.cat([t, torch.zeros(extra, H, d, dtype=t.dtype, device=t.device)]) for t in (q, k, v))
    cu = torch.tensor([0, 50, 120], dtype=torch.int32, device=q.device)
    o = torch.full_like(qx, float("nan"))
    lse = torch.full((H, T + extra), float("nan"), dtype=torch.float32, device=q.device)
    fa.fa_forward_ex(qx, kx, vx, o, lse, True, d ** -0.5, cu_seqlens=cu, max_seqlen=70)
    torch.cuda.synchronize()
    assert torch.isfinite(o[:T]).all() and torch.isnan(o[T:]).all()
    assert torch.isfinite(lse[:, :T]).all() and torch.isnan(lse[:, T:]).all()


# ---------------------------------------------------------------------------- autograd

def test_flash_attn_func_matches_contiguous(fa):
    import torch
    B, H, N, d, dtype = 2, 3, 150, 64, FI.FP16
    bits = FI.draw_bits((B, H, N, d), dtype, 4500)
    q, k, v, do = (_lib.to_device(bits[n], dtype) for n in FI.TENSOR_ORDER)
    ref = contiguous_run(fa, q, k, v, do, True, d ** -0.5)
    qs, ks, vs = (t.transpose(1, 2).contiguous().requires_grad_(True) for t in (q, k, v))
    o = fa.flash_attn_func(qs, ks, vs, causal=True)
    o.backward(do.transpose(1, 2).contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o.detach().transpose(1, 2).contiguous().view(torch.int16), ref[0].view(torch.int16))
    for t, r in zip((qs, ks, vs), ref[2:5]):
        assert torch.equal(t.grad.transpose(1, 2).contiguous().view(torch.int16), r.view(torch.int16))


def test_flash_attn_varlen_func_autograd(fa):
    import torch
    lengths, H, d, dtype, causal = (90, 3, 130), 2, 128, FI.BF16, True
    scale = d ** -0.5
    _, packed = draw_varlen(lengths, H, d, dtype, 4600)
    (q, k, v, do), (o_ref, _, dq_ref, dk_ref, dv_ref, _) = run_varlen(fa, packed, lengths, dtype, causal, scale)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=q.device)
    qg, kg, vg = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = fa.flash_attn_varlen_func(qg, kg, vg, cu, max(lengths), causal=causal)
    o.backward(do)
    torch.cuda.synchronize()
    assert torch.equal(o.detach().view(torch.int16), o_ref.view(torch.int16))
    for t, r in zip((qg, kg, vg), (dq_ref, dk_ref, dv_ref)):
        assert torch.equal(t.grad.view(torch.int16), r.view(torch.int16))


def test_malformed_cu_seqlens_stay_inside(fa):
    """Offsets that break the rules (decreasing, past total, negative; a length above
    max_seqlen) are clamped on the device: no write lands outside the operands. Each output
    sits between NaN guard regions, which must come back untouched."""
    import torch
    H, d, T, G = 2, 64, 300, 4096
    bits = FI.draw_bits((1, H, T, d), FI.BF16, 4700)
    q, k, v, do = (_lib.to_device(bits[n][0].transpose(1, 0, 2), FI.BF16) for n in FI.TENSOR_ORDER)

    def guarded(shape, dtype):
        n = int(np.prod(shape))
        buf = torch.full((G + n + G,), float("nan"), dtype=dtype, device=q.device)
        return buf, buf[G:G + n].view(*shape)

    cases = [
        [0, 200, 100, 300],      # decreasing offsets
        [0, 150, 5000],          # an offset past total
        [-50, 120, 300],         # a negative offset
        [0, 300],                # one sequence longer than max_seqlen (128)
    ]
    for cu_list in cases:
        cu = torch.tensor(cu_list, dtype=torch.int32, device=q.device)
        (ob, o), (lb, lse) = guarded((T, H, d), q.dtype), guarded((H, T), torch.float32)
        (dqb, dq), (dkb, dk), (dvb, dv) = (guarded((T, H, d), q.dtype) for _ in range(3))
        (db, delta) = guarded((H, T), torch.float32)
        fa.fa_forward_ex(q, k, v, o, lse, True, d ** -0.5, cu_seqlens=cu, max_seqlen=128)
        fa.fa_backward_ex(q, k, v, o, do, lse, dq, dk, dv, delta, True, d ** -0.5, cu_seqlens=cu, max_seqlen=128)
        torch.cuda.synchronize()
        for name, buf in (("o", ob), ("lse", lb), ("dq", dqb), ("dk", dkb), ("dv", dvb), ("delta", db)):
            assert torch.isnan(buf[:G]).all() and torch.isnan(buf[-G:]).all(), (cu_list, name)


def test_malformed_cu_seqlens_k_stay_inside(fa):
    """The same for the key offsets (cu_seqlens_k, separate from the query offsets): clamped
    on the device to [0, total_k] with lengths cut to max_seqlen_k, so no write lands outside
    the operands, through the forward, the backward and the split-KV forward."""
    import torch
    H, d, T, Tk, G = 2, 64, 300, 400, 4096
    bits = FI.draw_bits_rect(1, H, T, Tk, d, FI.BF16, 4800)
    q, do = (_lib.to_device(bits[n][0].transpose(1, 0, 2), FI.BF16) for n in ("q", "do"))
    k, v = (_lib.to_device(bits[n][0].transpose(1, 0, 2), FI.BF16) for n in ("k", "v"))
    cu = torch.tensor([0, 100, 200, 300], dtype=torch.int32, device=q.device)

    def guarded(shape, dtype):
        n = int(np.prod(shape))
        buf = torch.full((G + n + G,), float("nan"), dtype=dtype, device=q.device)
        return buf, buf[G:G + n].view(*shape)

    cases = [
        [0, 300, 150, 400],      # decreasing offsets
        [0, 150, 9000, 400],     # an offset past total_k
        [-70, 120, 250, 400],    # a negative offset
        [0, 10, 20, 400],        # a sequence longer than max_seqlen_k (128)
    ]
    for cuk_list in cases:
        cuk = torch.tensor(cuk_list, dtype=torch.int32, device=q.device)
        kw = dict(cu_seqlens=cu, max_seqlen=100, cu_seqlens_k=cuk, max_seqlen_k=128)
        (ob, o), (lb, lse) = guarded((T, H, d), q.dtype), guarded((H, T), torch.float32)
        (dqb, dq), (db, delta) = guarded((T, H, d), q.dtype), guarded((H, T), torch.float32)
        (dkb, dk), (dvb, dv) = guarded((Tk, H, d), q.dtype), guarded((Tk, H, d), q.dtype)
        (o2b, o2), (l2b, lse2) = guarded((T, H, d), q.dtype), guarded((H, T), torch.float32)
        need = fa.fa_forward_splitkv_ex_workspace_bytes(q, k, 3, **kw)
        wsb, ws = guarded((need // 4,), torch.float32)
        fa.fa_forward_ex(q, k, v, o, lse, True, d ** -0.5, **kw)
        fa.fa_backward_ex(q, k, v, o, do, lse, dq, dk, dv, delta, True, d ** -0.5, **kw)
        fa.fa_forward_splitkv_ex(q, k, v, o2, lse2, True, d ** -0.5, 3, ws, **kw)
        torch.cuda.synchronize()
        for name, buf in (("o", ob), ("lse", lb), ("dq", dqb), ("delta", db), ("dk", dkb), ("dv", dvb),
                          ("o split", o2b), ("lse split", l2b), ("workspace", wsb)):
            assert torch.isnan(buf[:G]).all() and torch.isnan(buf[-G:]).all(), (cuk_list, name)


@pytest.mark.timeout(600)
def test_varlen_full_size_sampled(fa):
    """A packed batch of the shape bench.py --sweep times (8 sequences, lengths
    varlen_lengths(8, 4096, 3001), 22030 tokens, H=32, d=128, causal bf16; values drawn per
    sequence here), in the same launch configuration: three
    (sequence, head) pairs against the oracle element by element, forward and backward,
    including the longest (4096-row) sequence, and on every head of every sequence the
    invariants sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i."""
    H, d, dtype, causal = 32, 128, FI.BF16, True
    lengths = [int(n) for n in FI.varlen_lengths(8, 4096, 3001)]
    scale = d ** -0.5
    seqs, packed = draw_varlen(lengths, H, d, dtype, 4900)
    _, (o, lse, dq, dk, dv, delta) = run_varlen(fa, packed, lengths, dtype, causal, scale)
    out = {n: _lib.from_device(t, dtype) for n, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv))}
    lse_np, delta_np = lse.cpu().numpy().astype(np.float64), delta.cpu().numpy().astype(np.float64)
    for n in out:
        assert np.all(np.isfinite(out[n])), n
    cu = np.concatenate([[0], np.cumsum(lengths)])
    longest = int(np.argmax(lengths))
    for b, h in ((0, 0), (3, 17), (longest, 31)):
        rows = slice(cu[b], cu[b + 1])
        q, k, v, do = (FI.bits_to_f64(seqs[b][n][0, h], dtype) for n in FI.TENSOR_ORDER)
        ref = ORACLE.backward(q, k, v, do, scale, causal)
        gpu = {"o": out["o"][rows, h], "lse": lse_np[h, rows], "dq": out["dq"][rows, h], "dk": out["dk"][rows, h],
               "dv": out["dv"][rows, h], "delta": delta_np[h, rows]}
        m = {"o_gate": float((np.abs(gpu["o"] - ref["o"]) - _lib.half_ulp(gpu["o"], dtype)).max()),
             "lse": float(np.abs(gpu["lse"] - ref["lse"]).max())}
        for g in ("dq", "dk", "dv"):
            m[g] = float(np.linalg.norm(gpu[g] - ref[g]) / np.linalg.norm(ref[g]))
        norm = np.linalg.norm(do, axis=1) * np.linalg.norm(ref["o"], axis=1) + 1e-30
        m["delta"] = float((np.abs(gpu["delta"] - ref["delta"]) / norm).max())
        print(f"varlen full size seq{b} (n={lengths[b]}) h{h}: " + " ".join(f"{k}={x:.3g}" for k, x in m.items()),
              flush=True)
        assert m["o_gate"] <= 1e-2 and m["lse"] <= 1e-3 and m["delta"] <= 1e-2, m
        assert max(m["dq"], m["dk"], m["dv"]) <= 2e-2, m
    do_all = FI.bits_to_f64(packed["do"], dtype)
    for b in range(len(lengths)):
        rows = slice(cu[b], cu[b + 1])
        dk_b, dv_b = out["dk"][rows], out["dv"][rows]  # (n, H, d)
        dk_sum = np.abs(dk_b.sum(axis=0)).max() / np.abs(dk_b).sum(axis=0).max()
        dv_gap = np.abs(dv_b.sum(axis=0) - do_all[rows].sum(axis=0)).max() / np.abs(dv_b).sum(axis=0).max()
        assert dk_sum <= 1e-2 and dv_gap <= 1e-2, (b, dk_sum, dv_gap)
