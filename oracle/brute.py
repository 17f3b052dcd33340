"""Brute-force checker for the oracle: the full T x T score matrix through library routines.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (same import rule as ``oracle/attention.py``).

It materialises every score, masks disallowed keys with -inf, and hands the rows to
``scipy.special.softmax`` / ``scipy.special.logsumexp``, so its softmax shares no arithmetic with
``attention.rows_forward``.  Causal window as read from the "Jan29" post's ``window_size`` keyword
(list of the largest improvements, item 1): key j is visible to query i iff j <= i and i - j < w.
"""
from __future__ import annotations

import numpy as np
from scipy.special import logsumexp, softmax


def mask(T: int, w: int) -> np.ndarray:
    """Allowed-set mask built by explicit loops (independent of ``attention.allowed``)."""
    m = np.zeros((T, T), dtype=bool)
    for i in range(T):
        for j in range(T):
            m[i, j] = (j <= i) and (i - j < w)
    return m


def fwd(q, k, v, w: int):
    """One head: q, k, v [T, D] -> O [T, D], LSE [T], P [T, T]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, D = q.shape
    scores = np.einsum("id,jd->ij", q, k) / np.sqrt(D)
    scores = np.where(mask(T, w), scores, -np.inf)
    p = softmax(scores, axis=1)
    lse = logsumexp(scores, axis=1)
    return p @ v, lse, p


def doc_mask(cu_seqlens, w: int) -> np.ndarray:
    """Allowed-set mask over packed documents, by explicit loops: query i sees key j iff both lie
    in the same document, j <= i and i - j < w."""
    cu = [int(x) for x in cu_seqlens]
    total = cu[-1]
    doc = np.empty(total, dtype=np.int64)
    for s in range(len(cu) - 1):
        for t in range(cu[s], cu[s + 1]):
            doc[t] = s
    m = np.zeros((total, total), dtype=bool)
    for i in range(total):
        for j in range(total):
            m[i, j] = (doc[i] == doc[j]) and (j <= i) and (i - j < w)
    return m


def fwd_masked(q, k, v, m):
    """One head over an explicit mask: q, k, v [N, D], m [N, N] -> O [N, D], LSE [N]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    scores = np.einsum("id,jd->ij", q, k) / np.sqrt(q.shape[1])
    scores = np.where(m, scores, -np.inf)
    return softmax(scores, axis=1) @ v, logsumexp(scores, axis=1)
