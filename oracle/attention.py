"""fp64 CPU oracle for exact softmax causal self-attention with an optional sliding window.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in ``oracle/``.  The HIP library and
its Python binding never import it, and this package imports nothing from them.

What is computed, and where it comes from
-----------------------------------------
* The attention kernel of the model, with a ``window_size`` keyword that lets layers alternate
  between short and long attention patterns: "nanochat: GPT-2-grade LLM for <<$100" post
  (web3.cnoyu.life, the "Jan29" entry), list of the largest improvements, item 1 (Flash Attention 3
  kernels).
* The KV-cache Engine with its two inference phases, prefill and decode: walkthrough "A fully
  hand-made copy of ChatGPT for $100 and 8,000 lines of code" (followin.io), section "Pretraining",
  closing paragraph; and the nanochat launch post (web3.ouchyi.army), feature list.
* Packed documents: training rows hold several documents separated by the beginning-of-sequence
  token (same walkthrough, section "Midtraining").  ``forward_varlen`` / ``backward_varlen`` take
  packed sequences in which each document attends only to itself.
* QK-norm: the model's RMS norms carry no trainable parameters (same walkthrough, section
  "Pretraining", the paragraph on the optimisers).  ``forward_qknorm`` / ``backward_qknorm``
  normalise each q and k row, r = 1 / sqrt(mean x^2 + eps), before the attention; by default the
  normalised rows are rounded to bf16 (they are stored activations), and the norm's backward uses
  its exact Jacobian at the raw rows.

The pages print no formula.  The definition below is textbook scaled dot-product attention; the
readings of what the pages leave open are:

* window ``w`` counts keys including the query itself: query ``i`` sees keys ``j`` with
  ``0 <= j <= i`` and ``i - j < w``; any ``w >= T`` is full causal attention;
* softmax scale ``1/sqrt(D)``; ``LSE`` is the natural-log row log-sum-exp;
* decode: the cache length ``L`` already counts the new token, whose position is ``L - 1``;
* the backward assumes no gradient flows into ``LSE``.

Everything is float64.  Inputs are the exact values the GPU receives (bf16 or fp32), upcast.

Pins (``tests/test_oracle.py``, all CPU): brute-force full-matrix softmax through
``scipy.special`` (``oracle/brute.py``), a hand-derived worked example (``tests/golden/``),
central finite differences and fp64 ``torch.autograd`` of the brute-force graph for every
gradient, closed forms (``w = 1``; equal keys; ``T = 1``) and invariants (rows of P sum to 1,
P is exactly 0 off the allowed set, ``w >= T`` equals full causal, sum_j dK_j = 0,
sum_j dV_j = sum_i dO_i, sum_i q_i.dQ_i = sum_j k_j.dK_j, decode equals the matching forward row).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "allowed",
    "rows_forward",
    "head_forward",
    "head_backward",
    "forward",
    "backward",
    "prefill",
    "kv_append",
    "decode",
    "forward_varlen",
    "backward_varlen",
    "rmsnorm",
    "forward_qknorm",
    "backward_qknorm",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def allowed(qpos: np.ndarray, kpos: np.ndarray, w: int) -> np.ndarray:
    """Boolean [len(qpos), len(kpos)]: key j is visible to query i iff j <= i and i - j < w.

    The causal mask plus the per-layer window of the "Jan29" post's attention kernels
    (``window_size``); w counts the query's own key.
    """
    qpos = np.asarray(qpos, dtype=np.int64)[:, None]
    kpos = np.asarray(kpos, dtype=np.int64)[None, :]
    return (kpos <= qpos) & (qpos - kpos < w)


def rows_forward(qr, qpos, k, v, w: int, return_p: bool = False):
    """Attention output for selected query rows of one head.

    qr [R, D] are the queries at positions ``qpos`` [R]; k, v [L, D] are the keys/values at
    positions 0..L-1.  Returns O [R, D], LSE [R] (and P [R, L] if asked):
        s_ij = q_i.k_j / sqrt(D) on the allowed set, -inf elsewhere
        m_i = max_j s_ij,  l_i = sum_j exp(s_ij - m_i),  LSE_i = m_i + ln l_i
        P_ij = exp(s_ij - LSE_i),  O_i = sum_j P_ij v_j
    """
    qr, k, v = _f64(qr), _f64(k), _f64(v)
    D = qr.shape[1]
    mask = allowed(qpos, np.arange(k.shape[0]), w)
    s = (qr @ k.T) / math.sqrt(D)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])  # exp(-inf) is exactly 0 off the allowed set
    l = e.sum(axis=1)
    p = e / l[:, None]
    o = p @ v
    lse = m + np.log(l)
    if return_p:
        return o, lse, p
    return o, lse


def head_forward(q, k, v, w: int, return_p: bool = False):
    """Forward of one (batch, head): q, k, v [T, D] -> O [T, D], LSE [T] (P [T, T])."""
    T = q.shape[0]
    return rows_forward(q, np.arange(T), k, v, w, return_p=return_p)


def head_backward(q, k, v, do, w: int):
    """Gradients of one (batch, head) for upstream dO [T, D] (no gradient into LSE).

        dV_j = sum_i P_ij dO_i
        dP_ij = dO_i.v_j,   Delta_i = dO_i.O_i  (= sum_j P_ij dP_ij)
        dS_ij = P_ij (dP_ij - Delta_i)
        dQ_i = (1/sqrt(D)) sum_j dS_ij k_j,   dK_j = (1/sqrt(D)) sum_i dS_ij q_i
    Returns dQ, dK, dV [T, D] and Delta [T].
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    D = q.shape[1]
    o, _, p = head_forward(q, k, v, w, return_p=True)
    dv = p.T @ do
    dp = do @ v.T
    delta = (do * o).sum(axis=1)
    ds = p * (dp - delta[:, None])
    dq = (ds @ k) / math.sqrt(D)
    dk = (ds.T @ q) / math.sqrt(D)
    return dq, dk, dv, delta


def _workers(n_items: int, threads: int | None) -> int:
    if threads is None:
        threads = len(os.sched_getaffinity(0))
    return max(1, min(threads, n_items))


def _map_heads(fn, items, threads):
    """Run fn over (b, h) items, in a thread pool whose BLAS calls are single-threaded."""
    n = _workers(len(items), threads)
    if n == 1:
        return [fn(it) for it in items]
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover - threadpoolctl is installed in this image
        threadpool_limits = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1, user_api="blas"):
            with ThreadPoolExecutor(n) as ex:
                return list(ex.map(fn, items))
    with ThreadPoolExecutor(n) as ex:
        return list(ex.map(fn, items))


def _eff_window(window, T: int) -> int:
    w = T if window is None else int(window)
    if w < 1:
        raise ValueError("window must be >= 1")
    return min(w, max(T, 1))


def forward(q, k, v, window=None, heads=None, threads=None):
    """Forward over [B, T, H, D] tensors.  Returns O [B, T, H, D] and LSE [B, H, T] (float64).

    ``heads``: optional list of (b, h) to compute; other entries are NaN.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, D = q.shape
    w = _eff_window(window, T)
    o = np.full((B, T, H, D), np.nan)
    lse = np.full((B, H, T), np.nan)
    items = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]

    def one(bh):
        b, h = bh
        return head_forward(q[b, :, h], k[b, :, h], v[b, :, h], w)

    for (b, h), (ob, lb) in zip(items, _map_heads(one, items, threads)):
        o[b, :, h] = ob
        lse[b, h] = lb
    return o, lse


def backward(q, k, v, do, window=None, heads=None, threads=None):
    """Backward over [B, T, H, D] tensors.  Returns dQ, dK, dV [B, T, H, D] (float64)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, T, H, D = q.shape
    w = _eff_window(window, T)
    dq = np.full((B, T, H, D), np.nan)
    dk = np.full((B, T, H, D), np.nan)
    dv = np.full((B, T, H, D), np.nan)
    items = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]

    def one(bh):
        b, h = bh
        return head_backward(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], w)

    for (b, h), (gq, gk, gv, _) in zip(items, _map_heads(one, items, threads)):
        dq[b, :, h] = gq
        dk[b, :, h] = gk
        dv[b, :, h] = gv
    return dq, dk, dv


def prefill(q, kcache, vcache, lens, window=None, threads=None):
    """Engine prefill (the walkthrough's "Pretraining" section, Engine paragraph).

    q [B, Tq, H, D] are the prompt queries at positions 0..Tq-1; the prompt keys/values already
    sit in cache rows 0..L_b-1 of kcache/vcache [B, Lcap, H, D].  Prompt b is the causal
    (windowed) forward with T = L_b.  Rows t >= L_b are undefined and returned as NaN.
    Returns O [B, Tq, H, D], LSE [B, H, Tq].
    """
    q, kcache, vcache = _f64(q), _f64(kcache), _f64(vcache)
    B, Tq, H, D = q.shape
    lens = np.asarray(lens, dtype=np.int64)
    o = np.full((B, Tq, H, D), np.nan)
    lse = np.full((B, H, Tq), np.nan)
    items = [(b, h) for b in range(B) for h in range(H) if lens[b] > 0]

    def one(bh):
        b, h = bh
        L = int(min(lens[b], Tq))
        w = _eff_window(window, L)
        return head_forward(q[b, :L, h], kcache[b, :L, h], vcache[b, :L, h], w)

    for (b, h), (ob, lb) in zip(items, _map_heads(one, items, threads)):
        L = ob.shape[0]
        o[b, :L, h] = ob
        lse[b, h, :L] = lb
    return o, lse


def kv_append(kcache, vcache, knew, vnew, pos):
    """Write one new token's key/value per sequence at cache row pos[b] (Engine KV cache).

    kcache/vcache [B, Lcap, H, D]; knew/vnew [B, H, D].  Returns updated copies.
    """
    kc = np.array(kcache, copy=True)
    vc = np.array(vcache, copy=True)
    for b, p in enumerate(np.asarray(pos, dtype=np.int64)):
        kc[b, p] = knew[b]
        vc[b, p] = vnew[b]
    return kc, vc


def decode(q, kcache, vcache, lens, window=None):
    """Engine decode step: one query per sequence against its cache.

    q [B, H, D]; kcache/vcache [B, Lcap, H, D]; lens [B] counts the cached tokens including the
    new one, so the query sits at position p = L - 1 and sees rows max(0, p - w + 1)..p.
    Returns O [B, H, D] and LSE [B, H]; a sequence with L = 0 gives O = 0 and LSE = -inf.
    Written per row, independently of ``rows_forward``.
    """
    q, kcache, vcache = _f64(q), _f64(kcache), _f64(vcache)
    B, H, D = q.shape
    Lcap = kcache.shape[1]
    o = np.zeros((B, H, D))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        L = int(min(max(int(lens[b]), 0), Lcap))
        if L == 0:
            continue
        p = L - 1
        w = L if window is None else int(window)
        j0 = max(0, p - w + 1)
        for h in range(H):
            kk = kcache[b, j0 : p + 1, h]
            vv = vcache[b, j0 : p + 1, h]
            s = kk @ q[b, h] / math.sqrt(D)
            m = s.max()
            e = np.exp(s - m)
            l = e.sum()
            o[b, h] = (e @ vv) / l
            lse[b, h] = m + math.log(l)
    return o, lse


def _segments(cu_seqlens):
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    return [(cu[s], cu[s + 1]) for s in range(len(cu) - 1)]


def forward_varlen(q, k, v, cu_seqlens, window=None, threads=None):
    """Packed sequences (documents): q, k, v [total, H, D]; sequence s is rows
    cu_seqlens[s] .. cu_seqlens[s + 1] - 1 and attends only to itself, causally, with the window
    counted from its own first row.  Returns O [total, H, D] and LSE [H, total] (float64)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    total, H, D = q.shape
    segs = _segments(cu_seqlens)
    o = np.full((total, H, D), np.nan)
    lse = np.full((H, total), np.nan)
    items = [(a, e, h) for a, e in segs if e > a for h in range(H)]

    def one(item):
        a, e, h = item
        return head_forward(q[a:e, h], k[a:e, h], v[a:e, h], _eff_window(window, e - a))

    for (a, e, h), (oh, lh) in zip(items, _map_heads(one, items, threads)):
        o[a:e, h] = oh
        lse[h, a:e] = lh
    return o, lse


def backward_varlen(q, k, v, do, cu_seqlens, window=None, threads=None):
    """Backward of ``forward_varlen``: dQ, dK, dV [total, H, D] (float64)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    total, H, D = q.shape
    segs = _segments(cu_seqlens)
    dq = np.full((total, H, D), np.nan)
    dk = np.full((total, H, D), np.nan)
    dv = np.full((total, H, D), np.nan)
    items = [(a, e, h) for a, e in segs if e > a for h in range(H)]

    def one(item):
        a, e, h = item
        return head_backward(q[a:e, h], k[a:e, h], v[a:e, h], do[a:e, h],
                             _eff_window(window, e - a))

    for (a, e, h), (gq, gk, gv, _) in zip(items, _map_heads(one, items, threads)):
        dq[a:e, h] = gq
        dk[a:e, h] = gk
        dv[a:e, h] = gv
    return dq, dk, dv



def rmsnorm(x, eps):
    """Parameter-free RMS norm over the last axis: returns (x * r, r), r = 1 / sqrt(mean x^2 + eps)."""
    x = _f64(x)
    r = 1.0 / np.sqrt((x * x).mean(axis=-1) + eps)
    return x * r[..., None], r


def _bf16(x):
    import torch  # rounding to bf16 (round to nearest even) through the library cast

    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def forward_qknorm(q, k, v, window=None, eps=1e-6, round_bf16=True, threads=None, heads=None):
    """Attention over RMS-normalised q, k ([B, T, H, D]).  Returns O, LSE and the normalised rows
    (qn, kn, as the attention saw them); ``heads`` as in ``forward``."""
    qn, _ = rmsnorm(q, eps)
    kn, _ = rmsnorm(k, eps)
    if round_bf16:
        qn, kn = _bf16(qn), _bf16(kn)
    o, lse = forward(qn, kn, v, window, heads=heads, threads=threads)
    return o, lse, qn, kn


def _rmsnorm_backward(x, g, eps):
    # y = x r, r = (mean x^2 + eps)^(-1/2):  dx = r (g - y (g . y) / D)
    y, r = rmsnorm(x, eps)
    D = y.shape[-1]
    return r[..., None] * (g - y * ((g * y).sum(axis=-1) / D)[..., None])


def backward_qknorm(q, k, v, do, window=None, eps=1e-6, round_bf16=True, threads=None,
                    heads=None):
    """Gradients of ``forward_qknorm``'s O with respect to the raw q, k and v; ``heads`` as in
    ``backward`` (other heads NaN)."""
    qn, _ = rmsnorm(q, eps)
    kn, _ = rmsnorm(k, eps)
    if round_bf16:
        qn, kn = _bf16(qn), _bf16(kn)
    gqn, gkn, gv = backward(qn, kn, v, do, window, heads=heads, threads=threads)
    return _rmsnorm_backward(q, gqn, eps), _rmsnorm_backward(k, gkn, eps), gv
