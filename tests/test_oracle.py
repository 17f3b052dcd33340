"""Pins for the fp64 oracle (CPU only).

The pages print no numeric attention example, so the oracle is pinned by what mathematics fixes:
a hand-derived worked example, brute force through library softmax, finite differences and fp64
autograd for the gradients, closed forms and invariants.  The planted-mistake tests at the end
show that plausible slips in the oracle (a window off by one, a wrong scale, a dropped Delta, a
transposed operand) are caught by these pins.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked.json")


def rnd(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------- worked example (hand-derived)
def test_handworked_forward():
    fx = json.load(open(GOLDEN))
    q, k, v = (np.array(fx[n], dtype=np.float64) for n in ("q", "k", "v"))
    for case in fx["cases"]:
        o, lse = A.head_forward(q, k, v, case["window"])
        np.testing.assert_allclose(o, np.array(case["O"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse, np.array(case["LSE"]), rtol=0, atol=1e-14)


def test_handworked_backward():
    fx = json.load(open(GOLDEN))
    q, k, v = (np.array(fx[n], dtype=np.float64) for n in ("q", "k", "v"))
    bw = fx["backward"]
    dq, dk, dv, delta = A.head_backward(q, k, v, np.array(bw["dO"], dtype=np.float64), bw["window"])
    np.testing.assert_allclose(dq, np.array(bw["dQ"]), atol=1e-14)
    np.testing.assert_allclose(dk, np.array(bw["dK"]), atol=1e-14)
    np.testing.assert_allclose(dv, np.array(bw["dV"]), atol=1e-14)
    assert abs(delta[3] - 2.0) < 1e-14


# ---------------------------------------------------------------- brute force (library softmax)
@pytest.mark.parametrize("T", [1, 2, 5, 17, 33])
@pytest.mark.parametrize("D", [4, 8])
def test_forward_matches_brute(T, D):
    rng = np.random.default_rng(100 * T + D)
    q, k, v = rnd(rng, T, D), rnd(rng, T, D), rnd(rng, T, D)
    for w in sorted({1, 2, 3, max(1, T - 1), T, T + 5}):
        o, lse, p = A.head_forward(q, k, v, w, return_p=True)
        ob, lb, pb = brute.fwd(q, k, v, w)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)
        np.testing.assert_allclose(p, pb, rtol=0, atol=1e-12)


def test_tiny_fp32_workload_matches_brute():
    """The tiny fp32 workload (B1 H2 T128 D64, full causal, seed 0) against brute force."""
    import workloads as W

    q, k, v = W.attn_inputs(W.TINY_F32)
    q, k, v = (t.double().numpy() for t in (q, k, v))
    o, lse = A.forward(q, k, v, W.TINY_F32.window, threads=1)
    for h in range(2):
        ob, lb, _ = brute.fwd(q[0, :, h], k[0, :, h], v[0, :, h], 128)
        np.testing.assert_allclose(o[0, :, h], ob, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], lb, atol=1e-12)


# ---------------------------------------------------------------- gradients
def _loss(q, k, v, g, w):
    o, _ = A.head_forward(q, k, v, w)
    return float((g * o).sum())


@pytest.mark.parametrize("T,w", [(1, 1), (5, 2), (9, 4), (16, 16), (16, 5), (12, 1)])
def test_gradients_finite_difference(T, w):
    rng = np.random.default_rng(T * 7 + w)
    D = 4
    q, k, v, g = (rnd(rng, T, D) for _ in range(4))
    dq, dk, dv, _ = A.head_backward(q, k, v, g, w)
    eps = 1e-6
    for x, grad in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, g, w)
            x[idx] = old - eps
            lm = _loss(q, k, v, g, w)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        den = max(np.linalg.norm(num), 1e-30)
        assert np.linalg.norm(num - grad) / den <= 1e-6 or np.abs(num - grad).max() < 1e-9


@pytest.mark.parametrize("T,w,D", [(7, 3, 8), (20, 20, 8), (33, 6, 16), (40, 1, 4)])
def test_gradients_torch_autograd(T, w, D):
    """fp64 autograd through the brute-force graph (masked_fill + torch.softmax)."""
    rng = np.random.default_rng(T + 1000 * w)
    q, k, v, g = (rnd(rng, T, D) for _ in range(4))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = (tq @ tk.T) / math.sqrt(D)
    m = torch.tensor(brute.mask(T, w))
    s = s.masked_fill(~m, float("-inf"))
    o = torch.softmax(s, dim=1) @ tv
    o.backward(torch.tensor(g))
    dq, dk, dv, _ = A.head_backward(q, k, v, g, w)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-10)


# ---------------------------------------------------------------- closed forms
def test_window_one_is_identity():
    rng = np.random.default_rng(5)
    T, D = 11, 8
    q, k, v, g = (rnd(rng, T, D) for _ in range(4))
    o, lse, p = A.head_forward(q, k, v, 1, return_p=True)
    np.testing.assert_array_equal(p, np.eye(T))
    np.testing.assert_allclose(o, v, atol=1e-15)
    np.testing.assert_allclose(lse, (q * k).sum(1) / math.sqrt(D), atol=1e-13)
    dq, dk, dv, _ = A.head_backward(q, k, v, g, 1)
    np.testing.assert_allclose(dq, 0, atol=1e-15)
    np.testing.assert_allclose(dk, 0, atol=1e-15)
    np.testing.assert_allclose(dv, g, atol=1e-15)


@pytest.mark.parametrize("w", [1, 3, 8, 100])
def test_equal_keys_give_window_mean(w):
    rng = np.random.default_rng(w)
    T, D = 13, 8
    q, v = rnd(rng, T, D), rnd(rng, T, D)
    c = rnd(rng, D)
    k = np.tile(c, (T, 1))
    o, lse = A.head_forward(q, k, v, w)
    for i in range(T):
        j0 = max(0, i - w + 1)
        np.testing.assert_allclose(o[i], v[j0 : i + 1].mean(0), atol=1e-13)
        np.testing.assert_allclose(lse[i], q[i] @ c / math.sqrt(D) + math.log(i - j0 + 1),
                                   atol=1e-13)


def test_zero_query_and_single_token():
    rng = np.random.default_rng(9)
    T, D = 9, 4
    k, v = rnd(rng, T, D), rnd(rng, T, D)
    o, _ = A.head_forward(np.zeros((T, D)), k, v, 4)
    for i in range(T):
        np.testing.assert_allclose(o[i], v[max(0, i - 3) : i + 1].mean(0), atol=1e-14)
    q1 = rnd(rng, 1, D)
    o1, lse1 = A.head_forward(q1, k[:1], v[:1], 7)
    np.testing.assert_allclose(o1, v[:1], atol=1e-15)
    np.testing.assert_allclose(lse1, q1[0] @ k[0] / 2.0, atol=1e-15)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("w", [1, 4, 16, 40])
def test_probability_invariants(w):
    rng = np.random.default_rng(77 + w)
    T, D = 40, 8
    q, k, v = rnd(rng, T, D, scale=3), rnd(rng, T, D, scale=3), rnd(rng, T, D)
    _, _, p = A.head_forward(q, k, v, w, return_p=True)
    np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-14)
    ii, jj = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
    off = (jj > ii) | (ii - jj >= w)
    assert np.all(p[off] == 0.0)
    assert np.all(p[~off] > 0.0)


def test_window_at_least_T_is_full_causal():
    rng = np.random.default_rng(3)
    T, D = 25, 8
    q, k, v, g = (rnd(rng, T, D) for _ in range(4))
    base = A.head_forward(q, k, v, T)
    for w in (T, T + 1, 10 * T):
        o, lse = A.head_forward(q, k, v, w)
        assert np.array_equal(o, base[0]) and np.array_equal(lse, base[1])
    gb = A.head_backward(q, k, v, g, T)
    ga = A.head_backward(q, k, v, g, 2 ** 31 - 1)
    for x, y in zip(ga, gb):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("w", [1, 5, 30])
def test_gradient_invariants(w):
    rng = np.random.default_rng(11 * w)
    T, D = 30, 8
    q, k, v, g = (rnd(rng, T, D) for _ in range(4))
    dq, dk, dv, _ = A.head_backward(q, k, v, g, w)
    np.testing.assert_allclose(dk.sum(0), 0.0, atol=1e-12)  # shift invariance of each row
    np.testing.assert_allclose(dv.sum(0), g.sum(0), atol=1e-12)  # rows of P sum to 1
    assert abs((q * dq).sum() - (k * dk).sum()) < 1e-11  # s_ij is bilinear in q_i, k_j


# ---------------------------------------------------------------- Engine: prefill, append, decode
def _cache_from(rng, B, Lcap, H, D, lens):
    kc = np.zeros((B, Lcap, H, D))
    vc = np.zeros((B, Lcap, H, D))
    for b in range(B):
        kc[b, : lens[b]] = rnd(rng, lens[b], H, D)
        vc[b, : lens[b]] = rnd(rng, lens[b], H, D)
    return kc, vc


@pytest.mark.parametrize("window", [None, 1, 3, 8])
def test_decode_equals_forward_last_row(window):
    rng = np.random.default_rng(21)
    B, Lcap, H, D = 3, 24, 2, 8
    lens = np.array([1, 9, 24])
    kc, vc = _cache_from(rng, B, Lcap, H, D, lens)
    qall = rnd(rng, B, Lcap, H, D)
    qd = np.stack([qall[b, lens[b] - 1] for b in range(B)])
    o, lse = A.decode(qd, kc, vc, lens, window)
    for b in range(B):
        L = lens[b]
        w = L if window is None else window
        for h in range(H):
            of, lf = A.head_forward(qall[b, :L, h], kc[b, :L, h], vc[b, :L, h], w)
            np.testing.assert_allclose(o[b, h], of[-1], atol=1e-13)
            np.testing.assert_allclose(lse[b, h], lf[-1], atol=1e-13)


def test_windowed_decode_equals_full_decode_on_slice():
    rng = np.random.default_rng(22)
    B, Lcap, H, D, w = 2, 30, 2, 8, 5
    lens = np.array([17, 30])
    kc, vc = _cache_from(rng, B, Lcap, H, D, lens)
    q = rnd(rng, B, H, D)
    o, lse = A.decode(q, kc, vc, lens, w)
    for b in range(B):
        L = lens[b]
        ks = np.zeros_like(kc[b : b + 1])
        vs = np.zeros_like(vc[b : b + 1])
        ks[0, :w] = kc[b, L - w : L]
        vs[0, :w] = vc[b, L - w : L]
        of, lf = A.decode(q[b : b + 1], ks, vs, np.array([w]), None)
        np.testing.assert_allclose(o[b], of[0], atol=1e-14)
        np.testing.assert_allclose(lse[b], lf[0], atol=1e-14)


def test_decode_zero_length():
    q = np.ones((1, 1, 4))
    kc = np.ones((1, 4, 1, 4))
    o, lse = A.decode(q, kc, kc, np.array([0]), None)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_prefill_is_per_prompt_forward_and_window_noop():
    rng = np.random.default_rng(23)
    B, Lcap, H, D = 3, 20, 2, 8
    lens = np.array([4, 13, 20])
    kc, vc = _cache_from(rng, B, Lcap, H, D, lens)
    q = rnd(rng, B, 20, H, D)
    o, lse = A.prefill(q, kc, vc, lens, None, threads=1)
    o_w, lse_w = A.prefill(q, kc, vc, lens, 20, threads=1)  # every L_b <= w: same as full causal
    for b in range(B):
        L = lens[b]
        ob, lb, _ = brute.fwd(q[b, :L, 0], kc[b, :L, 0], vc[b, :L, 0], L)
        np.testing.assert_allclose(o[b, :L, 0], ob, atol=1e-12)
        np.testing.assert_allclose(lse[b, 0, :L], lb, atol=1e-12)
        assert np.all(np.isnan(o[b, L:]))
    np.testing.assert_array_equal(o_w, o)
    np.testing.assert_array_equal(lse_w, lse)


def test_append_then_decode_matches_forward():
    rng = np.random.default_rng(24)
    B, Lcap, H, D = 2, 10, 1, 4
    lens = np.array([3, 6])
    kc, vc = _cache_from(rng, B, Lcap, H, D, lens)
    kn, vn, qn = rnd(rng, B, H, D), rnd(rng, B, H, D), rnd(rng, B, H, D)
    kc2, vc2 = A.kv_append(kc, vc, kn, vn, lens)
    for b in range(B):
        assert np.array_equal(kc2[b, lens[b]], kn[b]) and np.array_equal(vc2[b, lens[b]], vn[b])
        rest = np.ones(Lcap, dtype=bool)
        rest[lens[b]] = False
        assert np.array_equal(kc2[b, rest], kc[b, rest])
    o, _ = A.decode(qn, kc2, vc2, lens + 1, None)
    for b in range(B):
        L = lens[b] + 1
        ob, _, _ = brute.fwd(np.vstack([np.zeros((L - 1, D)), qn[b]]), kc2[b, :L, 0], vc2[b, :L, 0], L)
        np.testing.assert_allclose(o[b, 0], ob[-1], atol=1e-13)


def test_batched_forward_backward_match_heads():
    rng = np.random.default_rng(31)
    B, T, H, D, w = 2, 19, 3, 8, 6
    q, k, v, g = (rnd(rng, B, T, H, D) for _ in range(4))
    o, lse = A.forward(q, k, v, w, threads=4)
    dq, dk, dv = A.backward(q, k, v, g, w, threads=4)
    for b in range(B):
        for h in range(H):
            ob, lb, _ = brute.fwd(q[b, :, h], k[b, :, h], v[b, :, h], w)
            np.testing.assert_allclose(o[b, :, h], ob, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], lb, atol=1e-12)
            gq, gk, gv, _ = A.head_backward(q[b, :, h], k[b, :, h], v[b, :, h], g[b, :, h], w)
            assert np.array_equal(dq[b, :, h], gq) and np.array_equal(dk[b, :, h], gk)
            assert np.array_equal(dv[b, :, h], gv)


# ---------------------------------------------------------------- planted mistakes (CPU, oracle only)
def _pins_pass():
    """A compact subset of the pins above; returns False as soon as one fails."""
    fx = json.load(open(GOLDEN))
    q, k, v = (np.array(fx[n], dtype=np.float64) for n in ("q", "k", "v"))
    try:
        for case in fx["cases"]:
            o, lse = A.head_forward(q, k, v, case["window"])
            if not (np.allclose(o, case["O"], atol=1e-12) and np.allclose(lse, case["LSE"], atol=1e-12)):
                return False
        bw = fx["backward"]
        dq, dk, dv, _ = A.head_backward(q, k, v, np.array(bw["dO"], float), bw["window"])
        if not (np.allclose(dq, bw["dQ"], atol=1e-12) and np.allclose(dk, bw["dK"], atol=1e-12)
                and np.allclose(dv, bw["dV"], atol=1e-12)):
            return False
        rng = np.random.default_rng(0)
        T, D = 9, 4
        qq, kk, vv, gg = (rnd(rng, T, D) for _ in range(4))
        for w in (2, 9):
            o, lse, _ = A.head_forward(qq, kk, vv, w, return_p=True)
            ob, lb, _ = brute.fwd(qq, kk, vv, w)
            if not (np.allclose(o, ob, atol=1e-12) and np.allclose(lse, lb, atol=1e-12)):
                return False
            dq, dk, dv, _ = A.head_backward(qq, kk, vv, gg, w)
            if not (np.allclose(dk.sum(0), 0, atol=1e-12) and np.allclose(dv.sum(0), gg.sum(0))):
                return False
            if abs((qq * dq).sum() - (kk * dk).sum()) > 1e-10:
                return False
    except Exception:
        return False
    return True


def test_unmutated_oracle_passes_pin_subset():
    assert _pins_pass()


def _mut_allowed(qpos, kpos, w):  # window off by one (i - j <= w)
    qpos = np.asarray(qpos)[:, None]
    kpos = np.asarray(kpos)[None, :]
    return (kpos <= qpos) & (qpos - kpos <= w)


def _mut_noncausal(qpos, kpos, w):  # forgets the causal half
    qpos = np.asarray(qpos)[:, None]
    kpos = np.asarray(kpos)[None, :]
    return np.abs(qpos - kpos) < w


def _mut_backward_drop_delta(q, k, v, do, w):
    o, _, p = A.head_forward(q, k, v, w, return_p=True)
    ds = p * (do @ v.T)
    D = q.shape[1]
    return ds @ k / math.sqrt(D), ds.T @ q / math.sqrt(D), p.T @ do, (do * o).sum(1)


def _mut_backward_transposed(q, k, v, do, w):
    o, _, p = A.head_forward(q, k, v, w, return_p=True)
    dp = do @ v.T
    ds = p * (dp - (do * o).sum(1)[:, None])
    D = q.shape[1]
    return ds @ k / math.sqrt(D), ds.T @ q / math.sqrt(D), p @ do, (do * o).sum(1)


def _mut_backward_sign(q, k, v, do, w):
    o, _, p = A.head_forward(q, k, v, w, return_p=True)
    ds = p * (do @ v.T + (do * o).sum(1)[:, None])
    D = q.shape[1]
    return ds @ k / math.sqrt(D), ds.T @ q / math.sqrt(D), p.T @ do, (do * o).sum(1)


_orig_rows_forward = A.rows_forward


def _mut_scale(qr, qpos, k, v, w, return_p=False):  # 1/D instead of 1/sqrt(D)
    D = np.asarray(qr).shape[1]
    return _orig_rows_forward(np.asarray(qr) / math.sqrt(D), qpos, k, v, w, return_p)


@pytest.mark.parametrize("target,mutant", [
    ("allowed", _mut_allowed),
    ("allowed", _mut_noncausal),
    ("head_backward", _mut_backward_drop_delta),
    ("head_backward", _mut_backward_transposed),
    ("head_backward", _mut_backward_sign),
    ("rows_forward", _mut_scale),
])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(A, target, mutant)
    assert not _pins_pass()


# ---------------------------------------------------------------- packed documents (varlen)
# Training rows hold several documents separated by the beginning-of-sequence token (walkthrough,
# section "Midtraining"); each packed document attends only to itself.
VARLEN_CU = [0, 1, 9, 9, 26, 40]  # lengths 1, 8, 0 (empty), 17, 14


@pytest.mark.parametrize("w", [1, 3, 8, 100])
def test_varlen_forward_matches_brute_document_mask(w):
    rng = np.random.default_rng(50 + w)
    total, H, D = VARLEN_CU[-1], 2, 8
    q, k, v = (rng.standard_normal((total, H, D)) for _ in range(3))
    o, lse = A.forward_varlen(q, k, v, VARLEN_CU, w)
    m = brute.doc_mask(VARLEN_CU, w)
    for h in range(H):
        ob, lb = brute.fwd_masked(q[:, h], k[:, h], v[:, h], m)
        np.testing.assert_allclose(o[:, h], ob, atol=1e-12)
        np.testing.assert_allclose(lse[h], lb, atol=1e-12)


@pytest.mark.parametrize("w", [2, 100])
def test_varlen_backward_matches_autograd_of_document_mask(w):
    rng = np.random.default_rng(60 + w)
    total, H, D = VARLEN_CU[-1], 2, 8
    q, k, v, g = (rng.standard_normal((total, H, D)) for _ in range(4))
    dq, dk, dv = A.backward_varlen(q, k, v, g, VARLEN_CU, w)
    m = torch.tensor(brute.doc_mask(VARLEN_CU, w))
    for h in range(H):
        tq, tk, tv = (torch.tensor(x[:, h], requires_grad=True) for x in (q, k, v))
        s = ((tq @ tk.T) / math.sqrt(D)).masked_fill(~m, float("-inf"))
        (torch.softmax(s, dim=1) @ tv).backward(torch.tensor(g[:, h]))
        np.testing.assert_allclose(dq[:, h], tq.grad.numpy(), atol=1e-10)
        np.testing.assert_allclose(dk[:, h], tk.grad.numpy(), atol=1e-10)
        np.testing.assert_allclose(dv[:, h], tv.grad.numpy(), atol=1e-10)


def test_varlen_documents_are_isolated():
    """Changing one document's tokens leaves every other document's outputs unchanged, and a
    boundary moved by one row changes them (the pin sees the boundary)."""
    rng = np.random.default_rng(70)
    total, H, D = VARLEN_CU[-1], 1, 8
    q, k, v = (rng.standard_normal((total, H, D)) for _ in range(3))
    o1, _ = A.forward_varlen(q, k, v, VARLEN_CU)
    k2 = k.copy()
    k2[9:26] += rng.standard_normal((17, H, D))
    o2, _ = A.forward_varlen(q, k2, v, VARLEN_CU)
    assert np.array_equal(o1[:9], o2[:9]) and np.array_equal(o1[26:], o2[26:])
    assert not np.allclose(o1[9:26], o2[9:26])
    shifted = [0, 1, 10, 10, 26, 40]
    o3, _ = A.forward_varlen(q, k, v, shifted)
    m = brute.doc_mask(VARLEN_CU, total)
    ob, _ = brute.fwd_masked(q[:, 0], k[:, 0], v[:, 0], m)
    assert np.abs(o3[:, 0] - ob).max() > 1e-3


def test_varlen_one_sequence_is_the_dense_forward():
    rng = np.random.default_rng(80)
    T, H, D = 23, 2, 8
    q, k, v, g = (rng.standard_normal((T, H, D)) for _ in range(4))
    o, lse = A.forward_varlen(q, k, v, [0, T], 5)
    od, lsed = A.forward(q[None], k[None], v[None], 5)
    np.testing.assert_allclose(o, od[0], atol=1e-13)
    np.testing.assert_allclose(lse, lsed[0], atol=1e-13)


# ---------------------------------------------------------------- QK-norm
def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(90)
    x = rng.standard_normal((3, 5, 2, 16))
    y, r = A.rmsnorm(x, 0.0)
    np.testing.assert_allclose((y * y).mean(-1), 1.0, atol=1e-13)  # unit RMS
    y2, _ = A.rmsnorm(7.5 * x, 0.0)
    np.testing.assert_allclose(y2, y, atol=1e-13)  # scale invariance
    np.testing.assert_allclose(r, 1 / np.sqrt((x * x).mean(-1)), rtol=1e-14)
    tr = torch.nn.functional.rms_norm(torch.tensor(x), (16,), eps=1e-3).numpy()
    np.testing.assert_allclose(A.rmsnorm(x, 1e-3)[0], tr, atol=1e-13)  # the library routine


@pytest.mark.parametrize("w", [3, 100])
def test_qknorm_forward_and_backward_match_autograd(w):
    """fp64 autograd through torch's rms_norm and the masked softmax attention."""
    rng = np.random.default_rng(91 + w)
    B, T, H, D, eps = 1, 19, 2, 8, 1e-3
    q, k, v, g = (rng.standard_normal((B, T, H, D)) * s for s in (3.0, 0.5, 1.0, 1.0))
    o, lse, _, _ = A.forward_qknorm(q, k, v, w, eps, round_bf16=False)
    dq, dk, dv = A.backward_qknorm(q, k, v, g, w, eps, round_bf16=False)
    m = torch.tensor(brute.mask(T, w))
    for h in range(H):
        tq, tk, tv = (torch.tensor(x[0, :, h], requires_grad=True) for x in (q, k, v))
        nq = torch.nn.functional.rms_norm(tq, (D,), eps=eps)
        nk = torch.nn.functional.rms_norm(tk, (D,), eps=eps)
        s = ((nq @ nk.T) / math.sqrt(D)).masked_fill(~m, float("-inf"))
        to = torch.softmax(s, dim=1) @ tv
        np.testing.assert_allclose(o[0, :, h], to.detach().numpy(), atol=1e-12)
        to.backward(torch.tensor(g[0, :, h]))
        np.testing.assert_allclose(dq[0, :, h], tq.grad.numpy(), atol=1e-10)
        np.testing.assert_allclose(dk[0, :, h], tk.grad.numpy(), atol=1e-10)
        np.testing.assert_allclose(dv[0, :, h], tv.grad.numpy(), atol=1e-10)


def test_qknorm_gradient_is_orthogonal_to_the_row():
    """The norm is scale invariant (eps = 0), so dq . q = 0 and dk . k = 0 for every row."""
    rng = np.random.default_rng(93)
    q, k, v, g = (rng.standard_normal((1, 12, 1, 8)) for _ in range(4))
    dq, dk, _ = A.backward_qknorm(q, k, v, g, None, 0.0, round_bf16=False)
    assert np.abs((dq * q).sum(-1)).max() < 1e-12
    assert np.abs((dk * k).sum(-1)).max() < 1e-12


@pytest.mark.parametrize("w", [3, 100])
def test_qknorm_rounded_rows_match_straight_through_autograd(w):
    """round_bf16=True (the setting the GPU tests use): fp64 autograd through torch's rms_norm, a
    bf16 cast of the normalised rows with a straight-through gradient (the cast's value, identity
    derivative), and the masked softmax attention.  Inputs are far from unit RMS so the norm and the
    rounding both matter."""
    rng = np.random.default_rng(95 + w)
    B, T, H, D, eps = 1, 21, 2, 16, 1e-6
    q, k, v, g = (rng.standard_normal((B, T, H, D)) * s for s in (3.0, 0.5, 1.0, 1.0))
    o, lse, qn, kn = A.forward_qknorm(q, k, v, w, eps, round_bf16=True)
    dq, dk, dv = A.backward_qknorm(q, k, v, g, w, eps, round_bf16=True)
    m = torch.tensor(brute.mask(T, w))

    def st_bf16(x):  # value of the bf16 cast, gradient of the identity
        return x + (x.to(torch.bfloat16).to(torch.float64) - x).detach()

    for h in range(H):
        tq, tk, tv = (torch.tensor(x[0, :, h], requires_grad=True) for x in (q, k, v))
        nq = st_bf16(torch.nn.functional.rms_norm(tq, (D,), eps=eps))
        nk = st_bf16(torch.nn.functional.rms_norm(tk, (D,), eps=eps))
        # the rows the attention saw are exactly bf16 values
        np.testing.assert_array_equal(qn[0, :, h], nq.detach().numpy())
        np.testing.assert_array_equal(kn[0, :, h], nk.detach().numpy())
        s = ((nq @ nk.T) / math.sqrt(D)).masked_fill(~m, float("-inf"))
        to = torch.softmax(s, dim=1) @ tv
        np.testing.assert_allclose(o[0, :, h], to.detach().numpy(), atol=1e-12)
        np.testing.assert_allclose(lse[0, h], torch.logsumexp(s, dim=1).detach().numpy(),
                                   atol=1e-12)
        to.backward(torch.tensor(g[0, :, h]))
        np.testing.assert_allclose(dq[0, :, h], tq.grad.numpy(), atol=1e-10)
        np.testing.assert_allclose(dk[0, :, h], tk.grad.numpy(), atol=1e-10)
        np.testing.assert_allclose(dv[0, :, h], tv.grad.numpy(), atol=1e-10)
    # rounding changes the result: the unrounded oracle differs by far more than the tolerance above
    o_u, _, _, _ = A.forward_qknorm(q, k, v, w, eps, round_bf16=False)
    assert np.abs(o_u - o).max() > 1e-6
