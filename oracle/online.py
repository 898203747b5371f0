"""Blocked online-softmax forward in fp64 -- a test-only second algorithm.

TEST INFRASTRUCTURE (same import rule as ``oracle.attention``).

This is not the oracle. It walks the key/value blocks left to right keeping, per
query row, the running max m, the running denominator l and the unnormalised
accumulator u, as "FlashAttentionを1から" (ta-paperlens) describes in sections
"オンラインsoftmax" and "擬似コードで書くと", and "FlashAttention·FA4·FP4" in section
"온라인 softmax가 블록 사이의 값을 어떻게 이어 주나":

    m' = max(m, max of the new block's scores)
    l' = exp(m - m') * l + sum_j exp(s_j - m')
    u' = exp(m - m') * u + sum_j exp(s_j - m') * v_j
    output = u / l, once, after the last block.

Its job in the tests is to pin the oracle from another direction: the pages state
that the blocked result does not depend on where the block boundaries fall, so
the blocked result for every block width must equal the direct definition in
``oracle.attention``. ``rescale=False`` drops the exp(m - m') factor; it exists
only as the negative control the second page's worked example describes (the
result then changes with the block split).

A row whose scores in the current block are all masked contributes nothing; a row
that has seen no visible key yet keeps m = -inf, and exp(m - m') is then taken as
0 (the page's trace in "GPU에서 Attention은 실제로 어떻게 실행되는가", section 3-2,
starts from m = -inf, l = 0 and notes exp(-inf) = 0 wipes the initial term).
"""
from __future__ import annotations

import numpy as np


def _rescale_factor(m_old: np.ndarray, m_new: np.ndarray) -> np.ndarray:
    # exp(m_old - m_new); both -inf (nothing seen yet) gives 0 instead of NaN.
    out = np.zeros_like(m_new)
    seen = np.isfinite(m_old)
    out[seen] = np.exp(m_old[seen] - m_new[seen])
    return out


def online_state(q, k, v, scale: float, causal: bool, block_n: int,
                 key_range=None, rescale: bool = True):
    """Run the recurrence over keys [j_start, j_end) in blocks of ``block_n``.

    Returns the per-row state (m, l, u) before the final division; key indices
    stay absolute, so the causal mask is the same as for the whole row.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    j_start, j_end = (0, nk) if key_range is None else key_range
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    u = np.zeros((nq, v.shape[1]))
    rows = np.arange(nq)
    for j0 in range(j_start, j_end, block_n):
        j1 = min(j0 + block_n, j_end)
        s = scale * (q @ k[j0:j1].T)
        if causal:
            s[np.arange(j0, j1)[None, :] > rows[:, None]] = -np.inf
        m_new = np.maximum(m, s.max(axis=1))
        alpha = _rescale_factor(m, m_new) if rescale else np.where(np.isfinite(m), 1.0, 0.0)
        ref = np.where(np.isfinite(m_new), m_new, 0.0)
        p = np.exp(s - ref[:, None])
        l = alpha * l + p.sum(axis=1)
        u = alpha[:, None] * u + p @ v[j0:j1]
        m = m_new
    return m, l, u


def forward_blocked(q, k, v, scale: float, causal: bool, block_n: int, rescale: bool = True):
    """Online-softmax forward over key blocks of width ``block_n``. Returns (O, LSE)."""
    m, l, u = online_state(q, k, v, scale, causal, block_n, rescale=rescale)
    return u / l[:, None], m + np.log(l)


def forward_blocked_split(scores_row, values, splits, rescale: bool = True) -> float:
    """One query row given its scores directly, with explicit block boundaries.

    ``splits`` lists the block sizes in order (e.g. [2, 1]). Used for the pages'
    scalar worked examples, where scores are given already scaled.
    """
    s_all = np.asarray(scores_row, dtype=np.float64)
    v_all = np.asarray(values, dtype=np.float64)
    assert sum(splits) == s_all.size
    m, l, u = -np.inf, 0.0, 0.0
    pos = 0
    for n in splits:
        s = s_all[pos:pos + n]
        vv = v_all[pos:pos + n]
        pos += n
        m_new = max(m, float(s.max()))
        if rescale:
            alpha = 0.0 if m == -np.inf else float(np.exp(m - m_new))
        else:
            alpha = 0.0 if m == -np.inf else 1.0
        p = np.exp(s - m_new)
        l = alpha * l + float(p.sum())
        u = alpha * u + float(p @ vv)
        m = m_new
    return u / l


def merge_partials(parts):
    """Merge per-split partial states (m, l, u) of the same rows into (O, LSE).

    The page ("FlashAttentionを1から", section "その後の版と、推論での事情") notes that the
    same three update equations combine partial results computed over disjoint key
    ranges; each part is (m (n,), l (n,), u (n, dv)) with u unnormalised.
    """
    m = np.max(np.stack([p[0] for p in parts]), axis=0)
    l = np.zeros_like(m)
    u = np.zeros_like(parts[0][2])
    for mp, lp, up in parts:
        a = _rescale_factor(mp, m)
        l = l + a * lp
        u = u + a[:, None] * up
    return u / l[:, None], m + np.log(l)
