"""Pins for the fp64 oracle: what the pages and the mathematics fix, independent of the oracle.

Each check below is written as a function of the forward/backward callables, so the
same checks also run against deliberately broken copies of the oracle (the
"mutants" at the end) and must reject every one of them -- a dropped term, a wrong
sign or index, an off-by-one mask, a transposed operand, a base-2 LSE. That shows
the pins constrain the oracle rather than restate it.

Sources of the pinned values:
* the worked examples printed on the pages (fixtures in tests/golden/, with citations);
* closed forms (N = 1, all keys equal, causal row 0 and the last causal row);
* invariants (rows of P sum to 1, permutation invariance, gradient sums);
* a second algorithm (the blocked online recurrence) whose result the pages state is
  independent of the block split;
* library routines that define the same quantity independently (scipy's logsumexp,
  torch's float64 CPU scaled_dot_product_attention with autograd);
* central finite differences of the forward for every gradient.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import online as OL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(seed, *shape, scale=1.0):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape) * scale


# ----------------------------------------------------------------------------- checks
# Each check returns a list of failure strings (empty = pass) so mutants can be scored.

def check_worked_example_30(fwd, bwd):
    g = _golden("online_softmax_30.json")
    s = np.array([0.0, math.log(2.0), math.log(4.0)])
    q = np.ones((1, 1))
    k = s.reshape(3, 1)
    v = np.array(g["values"]).reshape(3, 1)
    o, lse = fwd(q, k, v, 1.0, False)
    errs = []
    if not abs(o[0, 0] - g["output_every_split"]) < 1e-12:
        errs.append(f"worked example 30: got {o[0, 0]}")
    if not abs(lse[0] - math.log(7.0)) < 1e-12:  # ln(1 + 2 + 4)
        errs.append(f"worked example 30 LSE: got {lse[0]}")
    return errs


def check_worked_example_fa2(fwd, bwd):
    g = _golden("fa2_trace_example.json")
    s = np.array(g["scores"])
    v = np.array(g["values"]).reshape(4, 1)
    o, lse = fwd(np.ones((1, 1)), s.reshape(4, 1), v, 1.0, False)
    errs = []
    e = np.exp(s - 5.0)
    exact = float((e * np.array(g["values"])).sum() / e.sum())
    if not abs(o[0, 0] - exact) < 1e-12:
        errs.append(f"fa2 example closed form: {o[0, 0]} vs {exact}")
    if not abs(o[0, 0] - g["page_values"]["output"]) <= g["printed_precision_abs"]:
        errs.append(f"fa2 example page value: {o[0, 0]}")
    denom = math.exp(lse[0] - g["page_values"]["global_max"])
    if not abs(denom - g["page_values"]["denominator"]) <= 1e-4 + 1e-12:
        errs.append(f"fa2 example denominator: {denom}")
    return errs


def check_causal_row0_and_last(fwd, bwd):
    errs = []
    N, d = 9, 5
    q, k, v = _rand(11, N, d), _rand(12, N, d), _rand(13, N, 3)
    scale = 0.37
    o, lse = fwd(q, k, v, scale, True)
    if not np.allclose(o[0], v[0], atol=1e-13, rtol=0):
        errs.append("causal row 0 != V[0]")
    if not abs(lse[0] - scale * float(q[0] @ k[0])) < 1e-13:
        errs.append("causal LSE_0 != scale q0.k0")
    o_nc, lse_nc = fwd(q, k, v, scale, False)
    if not (np.allclose(o[-1], o_nc[-1], atol=1e-13) and abs(lse[-1] - lse_nc[-1]) < 1e-13):
        errs.append("last causal row != non-causal last row")
    # every causal row i equals non-causal attention over the prefix of keys 0..i
    for i in (1, 4, 7):
        oi, li = fwd(q[i:i + 1], k[:i + 1], v[:i + 1], scale, False)
        if not (np.allclose(o[i], oi[0], atol=1e-13) and abs(lse[i] - li[0]) < 1e-13):
            errs.append(f"causal row {i} != prefix attention")
    return errs


def check_single_key(fwd, bwd):
    errs = []
    q, k, v = _rand(21, 1, 4), _rand(22, 1, 4), _rand(23, 1, 4)
    for causal in (False, True):
        o, lse = fwd(q, k, v, 0.5, causal)
        if not np.allclose(o, v, atol=1e-15):
            errs.append(f"N=1 O != V (causal={causal})")
        if not abs(lse[0] - 0.5 * float(q[0] @ k[0])) < 1e-14:
            errs.append(f"N=1 LSE (causal={causal})")
    return errs


def check_equal_keys(fwd, bwd):
    N, d = 7, 6
    q = _rand(31, N, d)
    k = np.tile(_rand(32, 1, d), (N, 1))
    v = _rand(33, N, d)
    scale = 0.8
    o, lse = fwd(q, k, v, scale, False)
    errs = []
    if not np.allclose(o, np.tile(v.mean(axis=0), (N, 1)), atol=1e-13):
        errs.append("equal keys: O != mean(V)")
    if not np.allclose(lse, scale * (q @ k[0]) + math.log(N), atol=1e-13):
        errs.append("equal keys: LSE != s + ln N")
    return errs


def check_permutations(fwd, bwd):
    N, d = 8, 4
    q, k, v = _rand(41, N, d), _rand(42, N, d), _rand(43, N, d)
    perm_k = np.random.Generator(np.random.PCG64(44)).permutation(N)
    perm_q = np.random.Generator(np.random.PCG64(45)).permutation(N)
    o, lse = fwd(q, k, v, 0.6, False)
    o2, lse2 = fwd(q, k[perm_k], v[perm_k], 0.6, False)
    o3, lse3 = fwd(q[perm_q], k, v, 0.6, False)
    errs = []
    if not (np.allclose(o, o2, atol=1e-13) and np.allclose(lse, lse2, atol=1e-13)):
        errs.append("permuting K,V rows together changed O")
    if not (np.allclose(o[perm_q], o3, atol=1e-13) and np.allclose(lse[perm_q], lse3, atol=1e-13)):
        errs.append("permuting Q rows did not permute O")
    return errs


def check_block_invariance(fwd, bwd):
    """Blocked online recurrence equals the direct result for every block width."""
    errs = []
    N, d = 70, 16
    q, k, v = _rand(51, N, d, scale=4.0), _rand(52, N, d), _rand(53, N, d)
    scale = 1.0 / math.sqrt(d)
    for causal in (False, True):
        o, lse = fwd(q, k, v, scale, causal)
        for bn in (1, 3, 16, 64, N):
            ob, lb = OL.forward_blocked(q, k, v, scale, causal, bn)
            if not (np.allclose(o, ob, atol=1e-12, rtol=0) and np.allclose(lse, lb, atol=1e-12, rtol=0)):
                errs.append(f"blocked Bc={bn} causal={causal} differs from direct")
    return errs


def check_library_logsumexp(fwd, bwd):
    from scipy.special import logsumexp
    errs = []
    N, d = 12, 8
    q, k, v = _rand(61, N, d, scale=3.0), _rand(62, N, d), _rand(63, N, d)
    scale = 0.3
    for causal in (False, True):
        _, lse = fwd(q, k, v, scale, causal)
        s = scale * (q @ k.T)
        if causal:
            s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
        if not np.allclose(lse, logsumexp(s, axis=1), atol=1e-12):
            errs.append(f"LSE != scipy logsumexp (causal={causal})")
    return errs


def check_torch_sdpa(fwd, bwd):
    """torch's float64 CPU scaled_dot_product_attention + autograd: an independent library definition."""
    import torch
    errs = []
    for causal in (False, True):
        N, d = 11, 8
        qn, kn, vn, don = _rand(71, N, d), _rand(72, N, d), _rand(73, N, d), _rand(74, N, d)
        scale = 0.41
        q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (qn, kn, vn))
        o = torch.nn.functional.scaled_dot_product_attention(
            q[None, None], k[None, None], v[None, None], is_causal=causal, scale=scale)[0, 0]
        o.backward(torch.tensor(don, dtype=torch.float64))
        r = bwd(qn, kn, vn, don, scale, causal)
        for name, ref in (("o", o.detach()), ("dq", q.grad), ("dk", k.grad), ("dv", v.grad)):
            if not np.allclose(r[name], ref.numpy(), atol=1e-12, rtol=1e-10):
                errs.append(f"{name} != torch sdpa (causal={causal})")
    return errs


def check_finite_differences(fwd, bwd):
    """Central differences of L = sum(O * dO) w.r.t. every input element."""
    errs = []
    h = 1e-6
    for causal in (False, True):
        N, d = 6, 5
        q, k, v, do = _rand(81, N, d), _rand(82, N, d), _rand(83, N, d), _rand(84, N, d)
        scale = 0.7
        r = bwd(q, k, v, do, scale, causal)

        def loss(qq, kk, vv):
            o, _ = fwd(qq, kk, vv, scale, causal)
            return float((o * do).sum())

        for name, idx in (("dq", 0), ("dk", 1), ("dv", 2)):
            args = [q.copy(), k.copy(), v.copy()]
            num = np.zeros_like(args[idx])
            for pos in np.ndindex(*num.shape):
                plus = [a.copy() for a in args]
                minus = [a.copy() for a in args]
                plus[idx][pos] += h
                minus[idx][pos] -= h
                num[pos] = (loss(*plus) - loss(*minus)) / (2 * h)
            if not np.allclose(r[name], num, atol=1e-7, rtol=1e-6):
                errs.append(f"{name} != finite differences (causal={causal}), "
                            f"max err {np.abs(r[name] - num).max():.3g}")
    return errs


def check_gradient_invariants(fwd, bwd):
    errs = []
    for causal in (False, True):
        N, d = 10, 6
        q, k, v, do = _rand(91, N, d), _rand(92, N, d), _rand(93, N, d), _rand(94, N, d)
        r = bwd(q, k, v, do, 0.45, causal)
        # O is unchanged by K_j -> K_j + c for all j at once, so sum_j dK_j = 0.
        if not np.allclose(r["dk"].sum(axis=0), 0.0, atol=1e-12):
            errs.append(f"sum_j dK_j != 0 (causal={causal})")
        # rows of P sum to 1, so sum_j dV_j = sum_i dO_i.
        if not np.allclose(r["dv"].sum(axis=0), do.sum(axis=0), atol=1e-12):
            errs.append(f"sum_j dV_j != sum_i dO_i (causal={causal})")
        # D_i = rowsum(dO_i * O_i) equals sum_k P_ik dP_ik with dP = dO V^T.
        o, lse = fwd(q, k, v, 0.45, causal)
        s = 0.45 * (q @ k.T)
        if causal:
            s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
        p = np.exp(s - lse[:, None])
        if not np.allclose(r["delta"], (p * (do @ v.T)).sum(axis=1), atol=1e-12):
            errs.append(f"delta != sum_k P dP (causal={causal})")
        if not np.allclose(p.sum(axis=1), 1.0, atol=1e-14):
            errs.append(f"rows of exp(S - LSE) do not sum to 1 (causal={causal})")
    # N = 1: dV = dO, dQ = dK = 0.
    q, k, v, do = _rand(95, 1, 4), _rand(96, 1, 4), _rand(97, 1, 4), _rand(98, 1, 4)
    r = bwd(q, k, v, do, 0.5, True)
    if not (np.allclose(r["dv"], do, atol=1e-15) and np.allclose(r["dq"], 0, atol=1e-15)
            and np.allclose(r["dk"], 0, atol=1e-15)):
        errs.append("N=1 gradients")
    return errs


def check_rectangular_causal(fwd, bwd):
    """Nq != Nk with the causal mask: the queries are the last Nq positions.

    * a rectangular problem is the last Nq rows of the square one (O, LSE, dQ), and its
      dK, dV are the square problem's with dO zero on the rows it lacks (the loss is
      linear in dO);
    * one causal query sees every key: it equals the unmasked result;
    * Nq > Nk: the first Nq - Nk rows see no key (O = 0, LSE = -inf, dQ = 0) and the
      rest are the square problem on the last Nk queries;
    * a tiny case written out with scalar loops.
    """
    errs = []
    nk, d = 12, 5
    qf, k, v, dof = _rand(121, nk, d), _rand(122, nk, d), _rand(123, nk, d), _rand(124, nk, d)
    o_sq, lse_sq = fwd(qf, k, v, 0.6, True)
    for nq in (1, 5):
        o, lse = fwd(qf[-nq:], k, v, 0.6, True)
        if not (np.allclose(o, o_sq[-nq:], atol=1e-13) and np.allclose(lse, lse_sq[-nq:], atol=1e-13)):
            errs.append(f"rectangular causal (nq={nq}) != last rows of the square problem")
        r = bwd(qf[-nq:], k, v, dof[-nq:], 0.6, True)
        do_pad = dof.copy()
        do_pad[:-nq] = 0.0
        rs = bwd(qf, k, v, do_pad, 0.6, True)
        if not (np.allclose(r["dq"], rs["dq"][-nq:], atol=1e-12) and np.allclose(r["dk"], rs["dk"], atol=1e-12)
                and np.allclose(r["dv"], rs["dv"], atol=1e-12)):
            errs.append(f"rectangular causal gradients (nq={nq}) != square problem with dO zero-padded")
    o1, l1 = fwd(qf[:1], k, v, 0.6, True)
    o2, l2 = fwd(qf[:1], k, v, 0.6, False)
    if not (np.allclose(o1, o2, atol=1e-14) and np.allclose(l1, l2, atol=1e-14)):
        errs.append("a single causal query does not see every key")
    # Nq > Nk
    q8 = _rand(125, 8, d)
    o, lse = fwd(q8, k[:5], v[:5], 0.6, True)
    o5, lse5 = fwd(q8[3:], k[:5], v[:5], 0.6, True)
    if not (np.all(o[:3] == 0.0) and np.all(lse[:3] == -np.inf)):
        errs.append("rows that see no key: O != 0 or LSE != -inf")
    if not (np.allclose(o[3:], o5, atol=1e-14) and np.allclose(lse[3:], lse5, atol=1e-14)):
        errs.append("Nq > Nk: visible rows != square problem on the last Nk queries")
    r = bwd(q8, k[:5], v[:5], dof[:8], 0.6, True)
    r5 = bwd(q8[3:], k[:5], v[:5], dof[3:8], 0.6, True)
    if not (np.all(r["dq"][:3] == 0.0) and np.allclose(r["dk"], r5["dk"], atol=1e-12)
            and np.allclose(r["dv"], r5["dv"], atol=1e-12)):
        errs.append("Nq > Nk gradients")
    # scalar loops: 3 queries, 7 keys, query i sees keys j <= i + 4
    q3, k7, v7 = _rand(126, 3, 2), _rand(127, 7, 2), _rand(128, 7, 2)
    o, lse = fwd(q3, k7, v7, 0.9, True)
    for i in range(3):
        sc = [0.9 * sum(q3[i, c] * k7[j, c] for c in range(2)) for j in range(i + 5)]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        tot = sum(w)
        for c in range(2):
            ref = sum(w[j] * v7[j, c] for j in range(len(w))) / tot
            if not abs(o[i, c] - ref) < 1e-13:
                errs.append(f"scalar-loop rectangular causal row {i}")
        if not abs(lse[i] - (mx + math.log(tot))) < 1e-13:
            errs.append(f"scalar-loop rectangular causal LSE row {i}")
    return errs


ALL_CHECKS = [
    check_worked_example_30, check_worked_example_fa2, check_causal_row0_and_last,
    check_single_key, check_equal_keys, check_permutations, check_block_invariance,
    check_library_logsumexp, check_torch_sdpa, check_finite_differences,
    check_gradient_invariants, check_rectangular_causal,
]


def _oracle_fwd(q, k, v, scale, causal):
    return A.forward(q, k, v, scale, causal)


def _oracle_bwd(q, k, v, do, scale, causal):
    return A.backward(q, k, v, do, scale, causal)


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    errs = check(_oracle_fwd, _oracle_bwd)
    assert not errs, errs


# ----------------------------------------------------------------------------- pages' blocked traces

def test_online_softmax_30_every_split_and_control():
    g = _golden("online_softmax_30.json")
    s = [0.0, math.log(2.0), math.log(4.0)]
    for splits in ([3], [2, 1], [1, 2], [1, 1, 1]):
        assert abs(OL.forward_blocked_split(s, g["values"], splits) - 30.0) < 1e-12
    assert abs(OL.forward_blocked_split(s, g["values"], [2, 1], rescale=False)
               - g["no_rescale_control_split_2_1"]) < 1e-12
    # intermediate state after the first two-element block
    m, l, u = OL.online_state(np.ones((1, 1)), np.array(s).reshape(3, 1),
                              np.array(g["values"]).reshape(3, 1), 1.0, False, 2, key_range=(0, 2))
    fb = g["first_block_two_elements"]
    assert abs(m[0] - math.log(2.0)) < 1e-15 and abs(l[0] - fb["l"]) < 1e-12 and abs(u[0, 0] - fb["u"]) < 1e-12


def test_fa2_trace_intermediates_to_printed_precision():
    g = _golden("fa2_trace_example.json")
    s = np.array(g["scores"]).reshape(4, 1)
    v = np.array(g["values"]).reshape(4, 1)
    tol = g["printed_precision_abs"]
    pv = g["page_values"]
    m1, l1, u1 = OL.online_state(np.ones((1, 1)), s, v, 1.0, False, 2, key_range=(0, 2))
    assert m1[0] == pv["block1"]["m"]
    assert abs(l1[0] - pv["block1"]["l"]) <= tol and abs(u1[0, 0] - pv["block1"]["o_unnormalised"]) <= tol
    m2, l2, u2 = OL.online_state(np.ones((1, 1)), s, v, 1.0, False, 2)
    assert m2[0] == pv["block2"]["m"]
    assert abs(l2[0] - pv["block2"]["l"]) <= tol and abs(u2[0, 0] - pv["block2"]["o_unnormalised"]) <= tol
    assert abs(u2[0, 0] / l2[0] - pv["output"]) <= tol


def test_rescale_factor_example():
    g = _golden("rescale_factor_example.json")
    # scores [score, chunk1_max] then [chunk2_max]; value 1 on the first key only
    s = np.array([g["score"], g["chunk1_max"], g["chunk2_max"]]).reshape(3, 1)
    v = np.array([1.0, 0.0, 0.0]).reshape(3, 1)
    _, _, u1 = OL.online_state(np.ones((1, 1)), s, v, 1.0, False, 2, key_range=(0, 2))
    assert abs(u1[0, 0] - g["exp_under_chunk1_max"]) <= g["printed_precision_abs"]
    _, _, u2 = OL.online_state(np.ones((1, 1)), s, v, 1.0, False, 2)
    assert abs(u2[0, 0] - g["exp_under_chunk2_max"]) <= g["printed_precision_abs"]
    assert abs(u2[0, 0] - math.exp(g["score"] - g["chunk2_max"])) < 1e-15


def test_split_merge_equals_direct():
    N, d = 40, 8
    q, k, v = _rand(101, N, d, scale=3.0), _rand(102, N, d), _rand(103, N, d)
    for causal in (False, True):
        o, lse = A.forward(q, k, v, 0.35, causal)
        parts = [OL.online_state(q, k, v, 0.35, causal, 7, key_range=r) for r in ((0, 13), (13, 30), (30, 40))]
        # rows that see no key of a part keep m = -inf there; the merge ignores them
        om, lm = OL.merge_partials(parts)
        assert np.allclose(o, om, atol=1e-12) and np.allclose(lse, lm, atol=1e-12)


def test_forward_rows_matches_full():
    N, d = 33, 8
    q, k, v = _rand(111, N, d), _rand(112, N, d), _rand(113, N, d)
    rows = [0, 5, 32]
    for causal in (False, True):
        o, lse = A.forward(q, k, v, 0.5, causal)
        orow, lrow = A.forward_rows(q, k, v, 0.5, causal, rows)
        assert np.array_equal(o[rows], orow) and np.array_equal(lse[rows], lrow)


def test_backward_with_stored_o_d():
    """D from a stored O (the page's preprocess definition) against the Jacobian form: with
    the exact O the identity sum_k P_ik dP_ik = dO_i . O_i makes the two agree; with O
    perturbed, the gradients move by exactly the induced dS = -P diag(dD) (a closed form)."""
    rng = np.random.Generator(np.random.PCG64(611))
    for nq, nk, causal in ((7, 7, True), (5, 9, False), (9, 3, True)):
        q, k, v, do = (rng.standard_normal((n, 6)) for n in (nq, nk, nk, nq))
        ref = A.backward(q, k, v, do, 0.4, causal)
        same = A.backward(q, k, v, do, 0.4, causal, o_stored=ref["o"])
        for g in ("dq", "dk", "dv"):
            assert np.allclose(same[g], ref[g], rtol=0, atol=1e-12)
        eps = 1e-3 * rng.standard_normal(ref["o"].shape)
        moved = A.backward(q, k, v, do, 0.4, causal, o_stored=ref["o"] + eps)
        _, _, p = A.forward(q, k, v, 0.4, causal, return_p=True)
        dd = (do * eps).sum(axis=1, keepdims=True)
        assert np.allclose(moved["dq"] - ref["dq"], -0.4 * (p * dd) @ k, rtol=0, atol=1e-12)
        assert np.allclose(moved["dk"] - ref["dk"], -0.4 * (p * dd).T @ q, rtol=0, atol=1e-12)
        assert np.array_equal(moved["dv"], ref["dv"])


def test_dq_rows_matches_full():
    # rows of the full backward's dQ, with fewer queries than keys and rows that see no key
    for nq, nk in ((33, 33), (20, 45), (45, 20)):
        q, do = _rand(121, nq, 8), _rand(122, nq, 8)
        k, v = _rand(123, nk, 8), _rand(124, nk, 8)
        rows = [0, 7, nq - 1]
        for causal in (False, True):
            full = A.backward(q, k, v, do, 0.5, causal)["dq"]
            assert np.allclose(A.dq_rows(q, k, v, do, 0.5, causal, rows), full[rows], rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------- mutants

def _mutant_forward(kind):
    def fwd(q, k, v, scale, causal):
        q = np.asarray(q, float)
        k = np.asarray(k, float)
        v = np.asarray(v, float)
        s = scale * (q @ k.T)
        if kind == "no_scale":
            s = q @ k.T
        if causal:
            nq, nk = s.shape
            jj, ii = np.arange(nk)[None, :], np.arange(nq)[:, None] + (nk - nq)
            hidden = jj >= ii if kind == "mask_hides_diagonal" else (jj > ii + 1 if kind == "mask_shows_next" else jj > ii)
            if kind == "mask_transposed":
                hidden = jj < ii
            if kind == "mask_top_left":
                hidden = jj > np.arange(nq)[:, None]
            s = np.where(hidden, -np.inf, s)
        p, m, l = A.softmax_rows(s)
        o = p @ v
        with np.errstate(divide="ignore"):
            lse = m + (np.log2(l) if kind == "lse_base2" else np.log(l))
            if kind == "lse_missing_max":
                lse = np.log(l)
        return o, lse
    return fwd


def _mutant_backward(kind):
    fwd_ok = _oracle_fwd

    def bwd(q, k, v, do, scale, causal):
        q, k, v, do = (np.asarray(x, float) for x in (q, k, v, do))
        s = A.scores(q, k, scale, causal)
        p, m, l = A.softmax_rows(s)
        o = p @ v
        dv = p.T @ do
        dp = do @ v.T
        if kind == "dp_uses_k":
            dp = do @ k.T
        corr = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - corr)
        if kind == "drop_jacobian_term":
            ds = p * dp
        if kind == "jacobian_sign":
            ds = p * (dp + corr)
        dq = scale * (ds @ k)
        dk = scale * (ds.T @ q)
        if kind == "dk_not_transposed":
            dk = scale * (ds @ q)
        if kind == "dq_missing_scale":
            dq = ds @ k
        if kind == "dv_not_transposed":
            dv = p @ do
        delta = (do * o).sum(axis=1)
        return {"o": o, "lse": m + np.log(l), "dq": dq, "dk": dk, "dv": dv, "delta": delta}
    return fwd_ok, bwd


FWD_MUTANTS = ["no_scale", "mask_hides_diagonal", "mask_shows_next", "mask_transposed",
               "lse_base2", "lse_missing_max", "mask_top_left"]
BWD_MUTANTS = ["dp_uses_k", "drop_jacobian_term", "jacobian_sign", "dk_not_transposed",
               "dq_missing_scale", "dv_not_transposed"]


def _run_all(fwd, bwd):
    failures = []
    for check in ALL_CHECKS:
        try:
            failures += check(fwd, bwd)
        except Exception as exc:  # a broken mutant may also crash a check
            failures.append(f"{check.__name__} raised {type(exc).__name__}")
    return failures


@pytest.mark.parametrize("kind", FWD_MUTANTS)
def test_pins_reject_forward_mutant(kind):
    fwd = _mutant_forward(kind)

    def bwd(q, k, v, do, scale, causal):  # backward built on the mutated forward's O
        r = A.backward(q, k, v, do, scale, causal)
        r["o"], r["lse"] = fwd(q, k, v, scale, causal)
        return r
    with np.errstate(all="ignore"):
        assert _run_all(fwd, bwd), f"no pin caught forward mutant {kind}"


@pytest.mark.parametrize("kind", BWD_MUTANTS)
def test_pins_reject_backward_mutant(kind):
    fwd, bwd = _mutant_backward(kind)
    with np.errstate(all="ignore"):
        assert _run_all(fwd, bwd), f"no pin caught backward mutant {kind}"
