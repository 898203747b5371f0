"""GPU: a seeded random sweep over the strided, packed and rectangular entry points.

Each draw (numpy PCG64, seed 8000 + index, fixed before any result) picks:
  * fixed lengths (B, H, N_q, N_k) or a packed batch with its own query and key lengths per
    sequence (zero lengths included), with shared or separate key offsets;
  * a head dim (any multiple of 8 up to 256), fp16 or bf16, causal or not, and a scale;
  * the storage layout: (B,H,N,d), or (B,N,H,d) / packed rows with padding columns after d.
It runs fa_forward_ex + fa_backward_ex, and for half of the draws also fa_forward_splitkv_ex;
for contiguous fixed-length draws with as many keys as queries, fa_forward_pingpong too (bit
for bit against fa_forward_ex).
Every head of every sequence is compared with the fp64 oracle to the tolerances of
tests/test_gpu_parity.py. Rows that see no key must be exactly O = 0, LSE = -inf, dQ = 0. Keys
that no query sees must get dK = dV = 0.
"""
import numpy as np
import pytest

import fa_inputs as FI
from oracle import attention as ORACLE
from tests import _lib
from tests.test_gpu_rectangular import compare_head

pytestmark = pytest.mark.gpu

N_DRAWS = 520


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    _lib.ensure_built()
    import exact_attention_27_amd as fa_mod
    return fa_mod


def draw_problem(i):
    rng = np.random.Generator(np.random.PCG64(8000 + i))
    p = {"d": int(8 * rng.integers(1, 33)), "dtype": FI.BF16 if rng.random() < 0.5 else FI.FP16,
         "causal": bool(rng.random() < 0.5), "H": int(rng.integers(1, 4)), "pad": int(rng.choice([0, 8, 24])),
         "split": int(rng.integers(1, 9)) if rng.random() < 0.5 else 0}
    p["scale"] = float(p["d"] ** -0.5 * rng.uniform(0.5, 2.0))
    if rng.random() < 0.4:
        B = int(rng.integers(1, 5))
        lq = rng.integers(0, 300, size=B)
        shared = rng.random() < 0.5
        lk = lq.copy() if shared else rng.integers(0, 300, size=B)
        lq[rng.integers(0, B)] = max(1, lq.max())  # at least one query row and one key row
        if shared:
            lk = lq.copy()
        else:
            lk[rng.integers(0, B)] = max(1, lk.max())
        p.update(varlen=True, B=B, lq=lq, lk=lk, shared=shared)
    else:
        B = int(rng.integers(1, 3))
        nq = int(rng.integers(1, 400))
        nk = nq if rng.random() < 0.5 else int(rng.integers(1, 400))
        p.update(varlen=False, B=B, nq=nq, nk=nk, layout="bhnd" if rng.random() < 0.5 else "bnhd")
    return p


def label_of(p):
    shape = (f"varlen{'-shared' if p['shared'] else ''} q{[int(x) for x in p['lq']]} k{[int(x) for x in p['lk']]}" if p["varlen"]
             else f"{p['layout']} B{p['B']} q{p['nq']} k{p['nk']}")
    return (f"{shape} H{p['H']} d{p['d']} {p['dtype']} {'causal' if p['causal'] else 'full'} pad{p['pad']} "
            f"split{p['split']}")


def padded(torch, t, pad):
    """t in a buffer with `pad` NaN columns after the head dim (same shape, wider row stride)."""
    if pad == 0:
        return t.contiguous()
    buf = torch.full(t.shape[:-1] + (t.shape[-1] + pad,), float("nan"), dtype=t.dtype, device=t.device)
    view = buf[..., : t.shape[-1]]
    view.copy_(t)
    return view


@pytest.mark.parametrize("i", range(N_DRAWS))
def test_random_problem(fa, i):
    import torch
    p = draw_problem(i)
    label = label_of(p)
    print(f"draw {i}: {label}", flush=True)
    d, dtype, H, scale, causal = p["d"], p["dtype"], p["H"], p["scale"], p["causal"]
    nan = float("nan")
    if p["varlen"]:
        lq, lk = p["lq"], p["lk"]
        cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
        Tq, Tk = int(cq[-1]), int(ck[-1])
        bits = FI.draw_bits_rect(1, H, Tq, Tk, d, dtype, 8500 + i)
        pk = {n: np.ascontiguousarray(bits[n][0].transpose(1, 0, 2)) for n in FI.TENSOR_ORDER}
        q, k, v, do = (padded(torch, _lib.to_device(pk[n], dtype), p["pad"]) for n in FI.TENSOR_ORDER)
        cu_q = torch.tensor(cq, dtype=torch.int32, device=q.device)
        kw = dict(cu_seqlens=cu_q, max_seqlen=int(max(1, lq.max())))
        if not p["shared"]:
            kw.update(cu_seqlens_k=torch.tensor(ck, dtype=torch.int32, device=q.device),
                      max_seqlen_k=int(max(1, lk.max())))
        sshape = (H, Tq)
        # (sequence, head) -> (query rows, key rows) of the packed operands
        cases = [(b, h, (slice(cq[b], cq[b + 1]), h), (slice(ck[b], ck[b + 1]), h), (h, slice(cq[b], cq[b + 1])))
                 for b in range(p["B"]) for h in range(H)]
    else:
        B, nq, nk, layout = p["B"], p["nq"], p["nk"], p["layout"]
        bits = FI.draw_bits_rect(B, H, nq, nk, d, dtype, 8500 + i)
        dev = [_lib.to_device(bits[n], dtype) for n in FI.TENSOR_ORDER]
        if layout == "bnhd":
            dev = [padded(torch, t.transpose(1, 2), p["pad"]) for t in dev]
        q, k, v, do = dev
        kw = dict(layout=layout)
        sshape = (B, H, nq)
        cases = [(b, h, (b, h), (b, h), (b, h)) for b in range(B) for h in range(H)]

    def to_np(t):
        # back to the (B,H,N,d) / packed (T,H,d) index order the cases use
        a = _lib.from_device(t, dtype)
        return a.transpose(0, 2, 1, 3) if (not p["varlen"] and p["layout"] == "bnhd") else a

    def bits_np(n):
        return FI.bits_to_f64(pk[n] if p["varlen"] else bits[n], dtype)

    qb, kb, vb, dob = (bits_np(n) for n in FI.TENSOR_ORDER)

    o = padded(torch, torch.full_like(q, nan), p["pad"]) if p["pad"] else torch.full_like(q, nan)
    lse = torch.full(sshape, nan, dtype=torch.float32, device=q.device)
    fa.fa_forward_ex(q, k, v, o, lse, causal, scale, **kw)
    dq = torch.full_like(q, nan)
    dk, dv = torch.full_like(k, nan), torch.full_like(v, nan)
    delta = torch.full_like(lse, nan)
    fa.fa_backward_ex(q, k, v, o, do, lse, dq, dk, dv, delta, causal, scale, **kw)
    torch.cuda.synchronize()
    g = {n: to_np(t) for n, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv))}
    g_lse, g_delta = lse.cpu().numpy().astype(np.float64), delta.cpu().numpy().astype(np.float64)

    split = None
    if p["split"]:
        o2 = torch.full_like(o, nan)
        lse2 = torch.full_like(lse, nan)
        fa.fa_forward_splitkv_ex(q, k, v, o2, lse2, causal, scale, p["split"], None, **kw)
        torch.cuda.synchronize()
        split = (to_np(o2), lse2.cpu().numpy().astype(np.float64))

    if not p["varlen"] and p["layout"] == "bhnd" and p["pad"] == 0 and p["nq"] == p["nk"]:
        # the ping-pong forward on the same contiguous problem: bit for bit what fa_forward_ex gave
        o3 = torch.full_like(q, nan)
        lse3 = torch.full_like(lse, nan)
        fa.fa_forward_pingpong(q, k, v, o3, lse3, causal, scale)
        torch.cuda.synchronize()
        assert o3.equal(o) and lse3.equal(lse), f"draw {i}: ping-pong forward differs"

    for b, h, qi, ki, si in cases:
        qf, dof, kf, vf = qb[qi], dob[qi], kb[ki], vb[ki]
        lab = f"draw {i} seq/batch {b} h{h}"
        if kf.shape[0] == 0:
            assert np.all(g["o"][qi] == 0.0) and np.all(g["dq"][qi] == 0.0), lab
            assert np.all(g_lse[si] == -np.inf), lab
            continue
        if qf.shape[0] == 0:
            assert np.all(g["dk"][ki] == 0.0) and np.all(g["dv"][ki] == 0.0), lab
            continue
        ref = ORACLE.backward(qf, kf, vf, dof, scale, causal)
        got = {"o": g["o"][qi], "lse": g_lse[si], "dq": g["dq"][qi], "dk": g["dk"][ki], "dv": g["dv"][ki],
               "delta": g_delta[si], "do_in": dof}
        compare_head(got, ref, dtype, lab, inputs=(qf, kf, vf, dof, scale, causal))
        if split is not None:
            compare_head({"o": split[0][qi], "lse": split[1][si]}, {"o": ref["o"], "lse": ref["lse"]}, dtype,
                         f"{lab} split={p['split']}", grads=False)
