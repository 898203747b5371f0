"""GPU: queries and keys of different lengths (cross-attention, decode against a key cache).

With N_q query rows and N_k key rows the causal mask aligns the queries with the last N_q
key positions: query i sees key j iff j <= i + (N_k - N_q). A query that sees no key gets
O = 0, LSE = -inf and dQ = 0; a key that no query sees gets dK = dV = 0. Checked here,
against the fp64 oracle on every head, to the tolerances of tests/test_gpu_parity.py:
  * forward and backward through fa_forward_ex / fa_backward_ex for N_q < N_k (down to one
    query) and N_q > N_k (rows that see no key), both masks, d = 64 / 96 / 128 / 256;
  * the split-KV forward on decode shapes (one query, a few thousand keys) and on
    rectangular ones, every split count giving the same answer, and batched decode over
    ragged key caches (packed sequences of 1-3 queries, one cache empty);
  * packed variable-length batches whose key offsets differ from the query offsets,
    including a sequence with no queries and one with no keys;
  * the autograd wrapper on K and V sliced out of a packed (B, N_k, 2, H, d) tensor;
  * the d <= 64 forward's three-slot K/V ring: 1 to 7 key tiles, single-pass and split.
"""
import numpy as np
import pytest

import fa_inputs as FI
from oracle import attention as ORACLE
from tests import _lib
from tests.test_gpu_parity import TOL_DELTA, TOL_GRAD, TOL_LSE, TOL_O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    _lib.ensure_built()
    import exact_attention_27_amd as fa_mod
    return fa_mod


def _nan_like(t, shape=None):
    import torch
    if shape is None:
        return torch.full_like(t, float("nan"))
    return torch.full(shape, float("nan"), dtype=torch.float32, device=t.device)


def compare_head(got, ref, dtype, label, grads=True, inputs=None):
    """Oracle comparison of one head. got / ref: dicts of float64 arrays (o, lse[, dq, dk, dv,
    delta]). Rows the oracle gives LSE = -inf must be exactly O = 0 / LSE = -inf / dQ = 0.

    inputs (q, k, v, dO, scale, causal as float64): when dQ or dK misses the gate, the head is
    also compared with the oracle's backward that takes D from the GPU's stored O (reading of
    the pages: the preprocess step uses the saved O). It passes only if the rounding of that O
    moves the reference by more than half the gate (dS is then a small difference of rounded
    terms: a row with two or three visible keys, say) and the GPU meets the gate against it."""
    m = {}
    err = np.abs(got["o"] - ref["o"])
    m["o_gate"] = float((err - _lib.half_ulp(got["o"], dtype)).max()) if err.size else 0.0
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(np.isfinite(got["lse"]), fin), f"{label}: rows with LSE = -inf differ"
    assert np.all(got["lse"][~fin] == -np.inf), label
    assert np.all(got["o"][~fin] == 0.0), f"{label}: a row that sees no key has O != 0"
    m["lse"] = float(np.abs(got["lse"][fin] - ref["lse"][fin]).max()) if fin.any() else 0.0
    if grads:
        assert np.all(got["dq"][~fin] == 0.0), f"{label}: a row that sees no key has dQ != 0"
        for g in ("dq", "dk", "dv"):
            nrm = np.linalg.norm(ref[g])
            if nrm == 0.0:
                if g == "dv":
                    # dV_j = sum_i P_ij dO_i: zero only when no query sees the key, which the
                    # kernel writes as exact zeros
                    assert np.all(got[g] == 0.0), f"{label}: {g} should be zero"
                else:
                    # A sequence with one visible key has dS = P (dP - D) = 0 exactly, but the
                    # kernels take dP = dO.V from the matrix cores and D = dO.O from the stored
                    # O (reading of the pages: D comes from the saved O), two fp32 sums of the
                    # same products in different orders: dQ and dK are then rounding-sized,
                    # as in the one-key case of the parity tests.
                    assert np.abs(got[g]).max() <= 1e-3, f"{label}: {g} should be (rounding-)zero"
                m[g] = 0.0
            else:
                m[g] = float(np.linalg.norm(got[g] - ref[g]) / nrm)
        norm = np.linalg.norm(got["do_in"], axis=1) * np.linalg.norm(ref["o"], axis=1) + 1e-30
        m["delta"] = float((np.abs(got["delta"] - ref["delta"]) / norm).max()) if norm.size else 0.0
    print(f"{label}: " + " ".join(f"{k}={v:.3g}" for k, v in m.items()), flush=True)
    assert m["o_gate"] <= TOL_O and m["lse"] <= TOL_LSE, (label, m)
    if grads:
        alt = None
        for g in ("dq", "dk", "dv"):
            if m[g] <= TOL_GRAD or g == "dv" or inputs is None:
                assert m[g] <= TOL_GRAD, (label, g, m)
                continue
            if alt is None:
                alt = ORACLE.backward(*inputs, o_stored=got["o"])
            shift = float(np.linalg.norm(alt[g] - ref[g]) / np.linalg.norm(ref[g]))
            r2 = float(np.linalg.norm(got[g] - alt[g]) / np.linalg.norm(alt[g]))
            print(f"{label}: {g} against D from the stored O: {r2:.3g} (the stored O moves the "
                  f"reference by {shift:.3g})", flush=True)
            assert shift > TOL_GRAD / 2 and r2 <= TOL_GRAD, (label, g, m, shift, r2)
        assert m["delta"] <= TOL_DELTA, (label, m)


# ------------------------------------------------------------------ fixed-length rectangles

RECT = [
    # B, H, Nq, Nk, d, dtype, causal
    (2, 2, 1, 1000, 128, FI.BF16, True),
    (1, 2, 1, 1000, 64, FI.FP16, False),
    (1, 2, 7, 300, 64, FI.BF16, True),
    (1, 2, 100, 300, 128, FI.BF16, True),
    (1, 2, 100, 300, 128, FI.FP16, False),
    (1, 2, 300, 100, 64, FI.BF16, True),
    (1, 2, 300, 100, 128, FI.FP16, False),
    (1, 2, 257, 1000, 128, FI.BF16, True),
    (1, 2, 1000, 257, 64, FI.BF16, True),
    (1, 2, 130, 64, 96, FI.BF16, True),
    (1, 2, 200, 700, 256, FI.BF16, True),
    (1, 2, 333, 129, 256, FI.FP16, True),
]


def run_rect(fa, bits, dtype, causal, scale):
    import torch
    q, k, v, do = (_lib.to_device(bits[n], dtype) for n in FI.TENSOR_ORDER)
    B, H, Nq, _ = q.shape
    o, lse = _nan_like(q), _nan_like(q, (B, H, Nq))
    fa.fa_forward_ex(q, k, v, o, lse, causal, scale, layout="bhnd")
    dq, dk, dv, delta = _nan_like(q), _nan_like(k), _nan_like(v), _nan_like(q, (B, H, Nq))
    fa.fa_backward_ex(q, k, v, o, do, lse, dq, dk, dv, delta, causal, scale, layout="bhnd")
    torch.cuda.synchronize()
    out = {n: _lib.from_device(t, dtype) for n, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv))}
    out["lse"] = lse.cpu().numpy().astype(np.float64)
    out["delta"] = delta.cpu().numpy().astype(np.float64)
    for n in ("o", "dq", "dk", "dv", "delta"):
        assert np.all(np.isfinite(out[n])), f"non-finite GPU {n}"
    assert not np.any(np.isnan(out["lse"])), "LSE left unwritten"
    return out


@pytest.mark.parametrize("case", RECT, ids=[f"q{c[2]}-k{c[3]}-d{c[4]}-{c[5]}-{'c' if c[6] else 'f'}" for c in RECT])
def test_rectangular_parity(fa, case):
    B, H, Nq, Nk, d, dtype, causal = case
    bits = FI.draw_bits_rect(B, H, Nq, Nk, d, dtype, 6000 + Nq + 3 * Nk + d)
    scale = d ** -0.5
    gpu = run_rect(fa, bits, dtype, causal, scale)
    for b in range(B):
        for h in range(H):
            q, k, v, do = (FI.bits_to_f64(bits[n][b, h], dtype) for n in FI.TENSOR_ORDER)
            ref = ORACLE.backward(q, k, v, do, scale, causal)
            got = {n: gpu[n][b, h] for n in ("o", "lse", "dq", "dk", "dv", "delta")}
            got["do_in"] = do
            compare_head(got, ref, dtype, f"Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal} b{b}h{h}")


# ------------------------------------------------------------------------ split-KV decode

SPLIT = [
    # B, H, Nq, Nk, d, causal, split counts
    (2, 4, 1, 4000, 128, True, (1, 4, 16, 63)),
    (2, 4, 1, 4096, 64, False, (2, 32)),
    (1, 2, 1, 1000, 256, True, (3,)),
    (1, 2, 100, 300, 128, True, (3, 8)),
    (1, 2, 300, 100, 64, True, (2, 5)),
]


@pytest.mark.parametrize("case", SPLIT, ids=[f"q{c[2]}-k{c[3]}-d{c[4]}-{'c' if c[5] else 'f'}" for c in SPLIT])
def test_splitkv_rectangular(fa, case):
    import torch
    B, H, Nq, Nk, d, causal, split_counts = case
    dtype = FI.BF16
    bits = FI.draw_bits_rect(B, H, Nq, Nk, d, dtype, 6500 + Nq + Nk + d)
    q, k, v = (_lib.to_device(bits[n], dtype) for n in ("q", "k", "v"))
    scale = d ** -0.5
    refs = {}
    for b in range(B):
        for h in range(H):
            qf, kf, vf = (FI.bits_to_f64(bits[n][b, h], dtype) for n in ("q", "k", "v"))
            refs[b, h] = ORACLE.forward(qf, kf, vf, scale, causal)
    for splits in split_counts:
        o, lse = _nan_like(q), _nan_like(q, (B, H, Nq))
        need = fa.fa_forward_splitkv_ex_workspace_bytes(q, k, splits, layout="bhnd")
        w = 64 if d <= 64 else 128 if d <= 128 else 256
        assert need == splits * B * H * Nq * (w + 2) * 4
        ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=q.device)
        fa.fa_forward_splitkv_ex(q, k, v, o, lse, causal, scale, splits, ws, layout="bhnd")
        torch.cuda.synchronize()
        o_np, lse_np = _lib.from_device(o, dtype), lse.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(o_np)) and not np.any(np.isnan(lse_np))
        for (b, h), (o_ref, lse_ref) in refs.items():
            compare_head({"o": o_np[b, h], "lse": lse_np[b, h]}, {"o": o_ref, "lse": lse_ref}, dtype,
                         f"split={splits} Nq={Nq} Nk={Nk} d={d} causal={causal} b{b}h{h}", grads=False)



RING_NK = [1, 63, 64, 65, 128, 129, 191, 192, 193, 256, 257, 320, 385]
RING_CASES = [(dt, d, c) for dt in (FI.FP16, FI.BF16) for d in (64, 40) for c in (False, True)]


@pytest.mark.parametrize("dtype,d,causal", RING_CASES, ids=[f"{dt}-d{d}-{'c' if c else 'f'}" for dt, d, c in RING_CASES])
def test_forward_ring_residues(fa, dtype, d, causal):
    """The forward at d <= 64 rotates three K and V slots, so the slot of the last key tile
    depends on the tile count modulo 3. 1 to 7 key tiles (N_k from 1 to 385, 100 queries),
    single-pass and split into 2 and 3 key ranges (ranges start at other tiles and hold 0-3
    tiles), against the oracle on every head."""
    import torch
    B, H, Nq = 1, 2, 100
    scale = d ** -0.5
    for nk in RING_NK:
        bits = FI.draw_bits_rect(B, H, Nq, nk, d, dtype, 6700 + nk + d)
        q, k, v = (_lib.to_device(bits[n], dtype) for n in ("q", "k", "v"))
        refs = {}
        for h in range(H):
            qf, kf, vf = (FI.bits_to_f64(bits[n][0, h], dtype) for n in ("q", "k", "v"))
            refs[h] = ORACLE.forward(qf, kf, vf, scale, causal)
        for splits in (0, 2, 3):
            o, lse = _nan_like(q), _nan_like(q, (B, H, Nq))
            if splits:
                need = fa.fa_forward_splitkv_ex_workspace_bytes(q, k, splits, layout="bhnd")
                ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=q.device)
                fa.fa_forward_splitkv_ex(q, k, v, o, lse, causal, scale, splits, ws, layout="bhnd")
            else:
                fa.fa_forward_ex(q, k, v, o, lse, causal, scale, layout="bhnd")
            torch.cuda.synchronize()
            o_np, lse_np = _lib.from_device(o, dtype), lse.cpu().numpy().astype(np.float64)
            for h in range(H):
                o_ref, lse_ref = refs[h]
                compare_head({"o": o_np[0, h], "lse": lse_np[0, h]}, {"o": o_ref, "lse": lse_ref}, dtype,
                             f"Nk={nk} splits={splits} h{h}", grads=False)

# ------------------------------------------------------ variable lengths, separate key offsets

def test_varlen_separate_key_offsets(fa):
    import torch
    H, d, dtype = 2, 64, FI.BF16
    # one query against 500 keys; equal lengths; keys only; more queries than keys; queries only
    lq = [1, 37, 0, 200, 150]
    lk = [500, 37, 64, 120, 0]
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    Tq, Tk = int(cq[-1]), int(ck[-1])
    bits = FI.draw_bits_rect(1, H, Tq, Tk, d, dtype, 6900)
    # packed (total, H, d) operands
    pk = {n: np.ascontiguousarray(bits[n][0].transpose(1, 0, 2)) for n in FI.TENSOR_ORDER}
    q, k, v, do = (_lib.to_device(pk[n], dtype) for n in FI.TENSOR_ORDER)
    cu_q = torch.tensor(cq, dtype=torch.int32, device=q.device)
    cu_k = torch.tensor(ck, dtype=torch.int32, device=q.device)
    scale = d ** -0.5
    for causal in (False, True):
        o, lse = _nan_like(q), _nan_like(q, (H, Tq))
        kw = dict(cu_seqlens=cu_q, max_seqlen=max(lq), cu_seqlens_k=cu_k, max_seqlen_k=max(lk))
        fa.fa_forward_ex(q, k, v, o, lse, causal, scale, **kw)
        dq, dk, dv, delta = _nan_like(q), _nan_like(k), _nan_like(v), _nan_like(q, (H, Tq))
        fa.fa_backward_ex(q, k, v, o, do, lse, dq, dk, dv, delta, causal, scale, **kw)
        torch.cuda.synchronize()
        g = {n: _lib.from_device(t, dtype) for n, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv))}
        g_lse, g_delta = lse.cpu().numpy().astype(np.float64), delta.cpu().numpy().astype(np.float64)
        for n in ("o", "dq", "dk", "dv"):
            assert np.all(np.isfinite(g[n])), n
        for b in range(len(lq)):
            rq, rk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
            for h in range(H):
                qf, dof = (FI.bits_to_f64(pk[n][rq, h], dtype) for n in ("q", "do"))
                kf, vf = (FI.bits_to_f64(pk[n][rk, h], dtype) for n in ("k", "v"))
                label = f"varlen causal={causal} seq{b} (q{lq[b]}, k{lk[b]}) h{h}"
                if lk[b] == 0:
                    # no key at all: every row is empty (the definition's empty softmax)
                    assert np.all(g["o"][rq, h] == 0.0) and np.all(g["dq"][rq, h] == 0.0), label
                    assert np.all(g_lse[h, rq] == -np.inf) and np.all(g_delta[h, rq] == 0.0), label
                    continue
                if lq[b] == 0:
                    # no query: nothing flows into the keys
                    assert np.all(g["dk"][rk, h] == 0.0) and np.all(g["dv"][rk, h] == 0.0), label
                    continue
                ref = ORACLE.backward(qf, kf, vf, dof, scale, causal)
                got = {"o": g["o"][rq, h], "lse": g_lse[h, rq], "dq": g["dq"][rq, h], "dk": g["dk"][rk, h],
                       "dv": g["dv"][rk, h], "delta": g_delta[h, rq], "do_in": dof}
                compare_head(got, ref, dtype, label)


# -------------------------------------------------------------------- autograd, strided K/V

def test_autograd_packed_kv(fa):
    import torch
    B, H, Nq, Nk, d, dtype, causal = 2, 2, 90, 250, 128, FI.BF16, True
    bits = FI.draw_bits_rect(B, H, Nq, Nk, d, dtype, 7100)
    qd, kd, vd, dod = (_lib.to_device(bits[n], dtype) for n in FI.TENSOR_ORDER)
    # (B, N, H, d) query and a (B, Nk, 2, H, d) packed key/value tensor
    q = qd.transpose(1, 2).contiguous().requires_grad_(True)
    kv = torch.stack([kd.transpose(1, 2), vd.transpose(1, 2)], dim=2).contiguous().requires_grad_(True)
    o = fa.flash_attn_func(q, kv[:, :, 0], kv[:, :, 1], causal=causal)
    o.backward(dod.transpose(1, 2))
    torch.cuda.synchronize()
    o_np = _lib.from_device(o.detach().transpose(1, 2), dtype)
    dq_np = _lib.from_device(q.grad.transpose(1, 2), dtype)
    dk_np = _lib.from_device(kv.grad[:, :, 0].transpose(1, 2), dtype)
    dv_np = _lib.from_device(kv.grad[:, :, 1].transpose(1, 2), dtype)
    scale = d ** -0.5
    for b in range(B):
        for h in range(H):
            qf, kf, vf, dof = (FI.bits_to_f64(bits[n][b, h], dtype) for n in FI.TENSOR_ORDER)
            ref = ORACLE.backward(qf, kf, vf, dof, scale, causal)
            label = f"autograd packed kv b{b}h{h}"
            gate = float((np.abs(o_np[b, h] - ref["o"]) - _lib.half_ulp(o_np[b, h], dtype)).max())
            assert gate <= TOL_O, (label, gate)
            for name, got in (("dq", dq_np), ("dk", dk_np), ("dv", dv_np)):
                rel = float(np.linalg.norm(got[b, h] - ref[name]) / np.linalg.norm(ref[name]))
                print(f"{label}: {name}={rel:.3g}", flush=True)
                assert rel <= TOL_GRAD, (label, name, rel)


def test_splitkv_varlen_decode(fa):
    """Batched decode over ragged key caches: packed sequences of 1-3 queries, each against its
    own cache length (one empty), through the split-KV forward with separate key offsets."""
    import torch
    H, d, dtype = 4, 128, FI.BF16
    lq = [1, 1, 3, 1, 1, 2]
    lk = [1, 100, 777, 2048, 0, 3000]
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    Tq, Tk = int(cq[-1]), int(ck[-1])
    bits = FI.draw_bits_rect(1, H, Tq, Tk, d, dtype, 7300)
    pk = {n: np.ascontiguousarray(bits[n][0].transpose(1, 0, 2)) for n in ("q", "k", "v")}
    q, k, v = (_lib.to_device(pk[n], dtype) for n in ("q", "k", "v"))
    cu_q = torch.tensor(cq, dtype=torch.int32, device=q.device)
    cu_k = torch.tensor(ck, dtype=torch.int32, device=q.device)
    scale = d ** -0.5
    kw = dict(cu_seqlens=cu_q, max_seqlen=max(lq), cu_seqlens_k=cu_k, max_seqlen_k=max(lk))
    for causal in (True, False):
        refs = {}
        for b in range(len(lq)):
            if lk[b] == 0:
                continue
            for h in range(H):
                qf = FI.bits_to_f64(pk["q"][cq[b]:cq[b + 1], h], dtype)
                kf, vf = (FI.bits_to_f64(pk[n][ck[b]:ck[b + 1], h], dtype) for n in ("k", "v"))
                refs[b, h] = ORACLE.forward(qf, kf, vf, scale, causal)
        for splits in (1, 5, 16):
            o, lse = _nan_like(q), _nan_like(q, (H, Tq))
            need = fa.fa_forward_splitkv_ex_workspace_bytes(q, k, splits, **kw)
            assert need == splits * H * Tq * (128 + 2) * 4
            ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=q.device)
            fa.fa_forward_splitkv_ex(q, k, v, o, lse, causal, scale, splits, ws, **kw)
            torch.cuda.synchronize()
            o_np, lse_np = _lib.from_device(o, dtype), lse.cpu().numpy().astype(np.float64)
            assert np.all(np.isfinite(o_np)) and not np.any(np.isnan(lse_np))
            for b in range(len(lq)):
                rq = slice(cq[b], cq[b + 1])
                label = f"varlen decode causal={causal} splits={splits} seq{b} (q{lq[b]}, k{lk[b]})"
                if lk[b] == 0:
                    assert np.all(o_np[rq] == 0.0) and np.all(lse_np[:, rq] == -np.inf), label
                    continue
                for h in range(H):
                    o_ref, lse_ref = refs[b, h]
                    compare_head({"o": o_np[rq, h], "lse": lse_np[h, rq]}, {"o": o_ref, "lse": lse_ref}, dtype,
                                 f"{label} h{h}", grads=False)
