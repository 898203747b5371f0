"""fp64 CPU oracle for exact attention, forward and backward.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module. The HIP library and its Python binding
never import it, share no code with it, and never fall back to it.

This is the *plain definition* the tiled method reaches exactly (up to rounding
order): "FlashAttentionを1から" (ta-paperlens), section "最適化なのに、計算が増える",
and "FlashAttention·FA4·FP4", section "첫 번째 비용", both state that the tiled
algorithm is not an approximation and returns the same answer as standard attention.
So the oracle materialises the full N x N score matrix S and probability matrix P,
in float64, with numpy's matmul as the only library primitive.

Definitions followed (the formula images on the pages were lost in extraction; the
surrounding prose fixes them, and the readings are listed in the design notes):

* scores  S = scale * Q K^T ("Triton 05: Flash Attention", section "코드 라인별 설명
  (Forward)", inner-loop step 1; "FlashAttention·FA4·FP4", section "첫 번째 비용":
  S = QK^T/sqrt(d)); the scale is applied before masking and the row max;
* causal mask: key j is visible to query i iff j <= i + (Nk - Nq) ("Triton 05", section
  "Causal Masking": future tokens are blocked by -inf). With Nq = Nk this is j <= i. With
  Nq != Nk the queries are read as the last Nq positions of the Nk-long sequence
  (bottom-right alignment), the reading under which a decode query -- one new token
  against the whole cache ("FlashAttentionを1から", section "その後の版と、推論での事情")
  -- sees every key;
* a row that sees no key (Nq > Nk, causal) has P = 0, O = 0 and LSE = -inf;
* safe softmax along each row: P_ij = exp(S_ij - m_i) / sum_k exp(S_ik - m_i),
  m_i = max_k S_ik ("FlashAttentionを1から", section "タイリングを阻む、softmaxという壁");
* output O = P V, and the saved row statistic LSE_i = m_i + ln sum_j exp(S_ij - m_i),
  natural log ("Triton 05", section "LSE로 P 재계산 (Recomputation)");
* backward, for an upstream gradient dO:
    dV = P^T dO,  dP = dO V^T,
    dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)      (the softmax Jacobian, written out),
    dQ = scale * dS K,  dK = scale * dS^T Q.
  ("Triton 05", sections "Softmax Gradient", "dKV 커널 수식", "dQ 커널 수식").
  The oracle deliberately uses the Jacobian form sum_k P_ik dP_ik rather than the
  shortcut D_i = rowsum(dO_i * O_i) the page introduces, so that the GPU's D vector
  is checked against an independent computation; D is returned separately, computed
  from its definition on the page, for that comparison.

All arrays are per head: q (Nq, d), k (Nk, d), v (Nk, dv), do (Nq, dv).
"""
from __future__ import annotations

import numpy as np


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def causal_hidden(rows, nq: int, nk: int) -> np.ndarray:
    """Boolean (len(rows), nk): key j hidden from query row i iff j > i + (nk - nq)."""
    return np.arange(nk)[None, :] > np.asarray(rows)[:, None] + (nk - nq)


def scores(q, k, scale: float, causal: bool) -> np.ndarray:
    """S = scale * Q K^T, with S_ij = -inf where the causal mask hides key j from query i."""
    q = _as_f64(q)
    k = _as_f64(k)
    s = scale * (q @ k.T)
    if causal:
        nq, nk = s.shape
        s[causal_hidden(np.arange(nq), nq, nk)] = -np.inf
    return s


def softmax_rows(s: np.ndarray):
    """Safe softmax over each row. Returns (P, m, l) with m the row max, l = sum exp(s - m).

    A row with every entry -inf (it sees no key) gets P = 0, m = -inf, l = 0."""
    m = s.max(axis=1)
    empty = m == -np.inf
    e = np.exp(s - np.where(empty, 0.0, m)[:, None])
    l = e.sum(axis=1)
    return e / np.where(empty, 1.0, l)[:, None], m, l


def _lse(m, l):
    """LSE = m + ln l, and -inf for a row that sees no key."""
    empty = m == -np.inf
    return np.where(empty, -np.inf, np.where(empty, 0.0, m) + np.log(np.where(empty, 1.0, l)))


def forward(q, k, v, scale: float, causal: bool, return_p: bool = False):
    """Exact attention forward for one head. Returns (O, LSE[, P]) in float64."""
    s = scores(q, k, scale, causal)
    p, m, l = softmax_rows(s)
    o = p @ _as_f64(v)
    lse = _lse(m, l)
    if return_p:
        return o, lse, p
    return o, lse


def forward_rows(q, k, v, scale: float, causal: bool, rows):
    """Forward restricted to the query rows ``rows`` (same definition, fewer rows).

    Row i of O and LSE depends only on q_i and all of K, V, so this is the plain
    definition evaluated for a sample of rows -- used for spot checks at sizes
    where materialising every row of S would be needlessly slow.
    """
    rows = np.asarray(rows, dtype=np.int64)
    q = _as_f64(q)
    k = _as_f64(k)
    s = scale * (q[rows] @ k.T)
    if causal:
        s[causal_hidden(rows, q.shape[0], k.shape[0])] = -np.inf
    p, m, l = softmax_rows(s)
    return p @ _as_f64(v), _lse(m, l)


def dq_rows(q, k, v, do, scale: float, causal: bool, rows):
    """dQ restricted to the query rows ``rows`` (same definition, fewer rows).

    Row i of dQ = scale * dS_i K needs only row i of S, P and dP ("Triton 05", section
    "dQ 커널 수식"), so this is the plain definition evaluated for a sample of rows -- for
    spot checks at lengths where the N x N matrices would not fit in memory.
    """
    rows = np.asarray(rows, dtype=np.int64)
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    s = scale * (q[rows] @ k.T)
    if causal:
        s[causal_hidden(rows, q.shape[0], k.shape[0])] = -np.inf
    p, _, _ = softmax_rows(s)
    dp = do[rows] @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return scale * (ds @ k)


def backward(q, k, v, do, scale: float, causal: bool, o_stored=None):
    """Exact attention backward for one head.

    Returns a dict with o, lse, dq, dk, dv and delta (D_i = rowsum(dO_i * O_i)),
    all float64.

    o_stored: None for the softmax Jacobian form above. Otherwise the output as a
    kernel stored it (16-bit values, as float64): dS then uses D_i = rowsum(dO_i * O_i)
    of that stored O, the preprocess step of "Triton 05", section "3단계 커널 구조",
    evaluated exactly. With the exact O the two forms agree (sum_k P_ik dP_ik =
    dO_i . (P V)_i); they differ by the rounding of the stored O, which dominates dS
    where dS is a small difference (a row with two or three visible keys, say).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    o, lse, p = forward(q, k, v, scale, causal, return_p=True)
    dv = p.T @ do
    dp = do @ v.T
    if o_stored is None:
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    else:
        ds = p * (dp - (do * _as_f64(o_stored)).sum(axis=1, keepdims=True))
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    delta = (do * o).sum(axis=1)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "delta": delta}
