"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle on the same seeded inputs.

Bars (bf16 in, fp32 accumulate): O max-abs <= 1e-2 over valid elements, except where storing the
exact value in the output format alone can miss it by more (a bf16 output with |O| >= 4, whose
half ulp is 2^-6 > 1e-2): there one bf16 ulp of the exact value (see o_bar); dQ, dK, dV relative
Frobenius error <= 2e-2 each, over the whole tensor; LSE max-abs <= 1e-3 (reported bar).  The
full-size workloads (the d20 layer, the four d26 layers, the packed-document d20 rows, the QK-norm
d20 layer) compare every head against the oracle run on the whole tensor.
"""
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as ref

pytestmark = pytest.mark.gpu

O_TOL = 1e-2
G_TOL = 2e-2
LSE_TOL = 1e-3


@pytest.fixture(scope="module")
def sw():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_sliding_window_attn_amd as m

    m.load()
    return m


DEV = "cuda"


def f64(t):
    return t.detach().double().cpu().numpy()


def o_bar(o_r, fp32=False):
    """Per-element bar on O: 1e-2, or for bf16 outputs with |O| >= 4 one bf16 ulp of the exact
    value.  A bf16 value near |O| in [4, 8) is only representable to 2^-5, so the nearest one can
    sit 2^-6 > 1e-2 from the exact result: there the bar is the format's own resolution."""
    if fp32:
        return np.full(np.shape(o_r), O_TOL)
    a = np.abs(o_r)
    ulp = np.exp2(np.floor(np.log2(np.maximum(a, 1e-300))) - 7)
    return np.where(a < 4.0, O_TOL, ulp)


def o_excess(o, o_r, fp32=False):
    """max |o - o_r| / bar over valid (finite-reference) elements; the check is <= 1."""
    o, o_r = np.asarray(o, np.float64), np.asarray(o_r, np.float64)
    m = np.isfinite(o_r)
    if not m.any():
        return 0.0
    return float((np.abs(o[m] - o_r[m]) / o_bar(o_r[m], fp32)).max())


def assert_o(o, o_r, tag="", fp32=False):
    x = o_excess(o, o_r, fp32)
    e = float(np.abs(np.asarray(o, np.float64) - np.asarray(o_r, np.float64))[np.isfinite(o_r)].max()) \
        if np.isfinite(o_r).any() else 0.0
    assert x <= 1.0, f"{tag} O error {x:.3f} x its bar (max-abs {e:.4g})"


def rel_fro(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def check_fwd(o, lse, o_r, lse_r, heads=None, tag=""):
    fp32 = o.dtype == torch.float32
    o, lse = f64(o), f64(lse) if lse is not None else None
    if heads is not None:
        for b, h in heads:
            assert_o(o[b, :, h], o_r[b, :, h], f"{tag} head {(b, h)}", fp32)
            if lse is not None:
                el = np.abs(lse[b, h] - lse_r[b, h]).max()
                assert el <= LSE_TOL, f"{tag} LSE max-abs {el} at head {(b, h)}"
        return
    assert_o(o, o_r, tag, fp32)
    if lse is not None:
        el = np.abs(lse - lse_r).max()
        assert el <= LSE_TOL, f"{tag} LSE max-abs {el}"


def zero_grad_bounds(Q, K, V, DO):
    """Rounding residue allowed where the exact dQ and dK vanish (window 1: P = I, O = V, so
    dS_ii = P_ii (dO_i . v_i - dO_i . O_i) = 0 exactly).  The kernels form the two dot products
    in fp32 in different orders; each is a sum of D rounded terms, whose rounding errors behave as
    a random walk of about sqrt(D) unit roundoffs u = 2^-24 times the sum of |terms|.  The bound
    allows 8 such steps on each side, then the gradient's factors: dQ_i = dS_ii k_i / sqrt(D),
    dK_i = dS_ii q_i / sqrt(D)."""
    D = Q.shape[-1]
    u = 2.0 ** -24
    dot_abs = np.abs(DO * V).sum(-1)  # [B, T, H]
    ds = 2 * 8 * math.sqrt(D) * u * dot_abs
    b_dq = float((ds * np.abs(K).max(-1)).max()) / math.sqrt(D)
    b_dk = float((ds * np.abs(Q).max(-1)).max()) / math.sqrt(D)
    return b_dq, b_dk


def check_grads(gs, rs, heads=None, tag="", zero_bounds=None):
    for i, (name, g, r) in enumerate(zip(("dQ", "dK", "dV"), gs, rs)):
        g = f64(g)
        if heads is not None:
            g = np.stack([g[b, :, h] for b, h in heads])
            r = np.stack([r[b, :, h] for b, h in heads])
        if not np.any(r):
            # closed-form zero gradient (window 1 gives dQ = dK = 0 exactly): relative error is
            # undefined, so bound the rounding residue absolutely instead
            assert zero_bounds is not None, f"{tag} {name}: exact zero needs a residue bound"
            e = float(np.abs(g).max())
            assert e <= zero_bounds[i], f"{tag} {name} should be 0, max-abs {e} > {zero_bounds[i]}"
            continue
        e = rel_fro(g, r)
        assert e <= G_TOL, f"{tag} {name} rel-Frobenius {e}"


def run_fwd_bwd(sw, q, k, v, do, window):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o, lse = sw.attn_fwd(qd, kd, vd, window=window)
    grads = None
    if do is not None:
        grads = sw.attn_bwd(qd, kd, vd, o, lse, do.to(DEV), window=window)
    torch.cuda.synchronize()
    return o, lse, grads


def test_single_hip_runtime(sw):
    maps = open("/proc/self/maps").read()
    libs = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(libs) == 1, libs


# --------------------------------------------------------------------------- the five workloads
def test_tiny_fp32_forward(sw):
    q, k, v = W.attn_inputs(W.TINY_F32)
    o, lse, _ = run_fwd_bwd(sw, q, k, v, None, W.TINY_F32.window)
    o_r, lse_r = ref.forward(f64(q), f64(k), f64(v), W.TINY_F32.window)
    check_fwd(o, lse, o_r, lse_r, tag="tiny-fp32")
    assert np.abs(f64(o) - o_r).max() < 1e-4  # fp32 end to end


def test_small_bf16_window128(sw):
    c = W.SMALL_W128
    q, k, v, do = W.attn_inputs(c)
    o, lse, g = run_fwd_bwd(sw, q, k, v, do, c.window)
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    o_r, lse_r = ref.forward(Q, K, V, c.window)
    check_fwd(o, lse, o_r, lse_r, tag=c.name)
    check_grads(g, ref.backward(Q, K, V, DO, c.window), tag=c.name)


@pytest.mark.slow
def test_d20_layer_every_head(sw):
    """The d20 layer in the bench's launch configuration, every head against the oracle: O and
    LSE max-abs over all elements, dQ / dK / dV relative Frobenius over the whole tensors."""
    c = W.D20_LAYER
    q, k, v, do = W.attn_inputs(c)
    o, lse, g = run_fwd_bwd(sw, q, k, v, do, c.window)
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    o_r, lse_r = ref.forward(Q, K, V, c.window)
    check_fwd(o, lse, o_r, lse_r, tag=c.name)
    del o_r, lse_r
    check_grads(g, ref.backward(Q, K, V, DO, c.window), tag=c.name)


@pytest.mark.slow
@pytest.mark.parametrize("layer", [0, 1, 2, 3])
def test_d26_alternating_layer(sw, layer):
    """Each layer of the d26 stack (windows 512, full, 512, full), every head."""
    window = W.D26_WINDOWS[layer]
    q, k, v, do = W.d26_layer_inputs(layer)
    o, lse, g = run_fwd_bwd(sw, q, k, v, do, window)
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    o_r, lse_r = ref.forward(Q, K, V, window)
    check_fwd(o, lse, o_r, lse_r, tag=f"d26 layer {layer}")
    del o_r, lse_r
    check_grads(g, ref.backward(Q, K, V, DO, window), tag=f"d26 layer {layer}")


@pytest.mark.slow
@pytest.mark.parametrize("layer", [0, 1])
def test_d30_engine_prefill_and_decode(sw, layer):
    E = W.D30_ENGINE
    window = E.window(layer)
    lens = W.engine_lens(E)
    Tq = int(lens.max())
    qp, kp, vp = W.engine_prefill_packed(layer, lens, E)
    q = W.pad_prompts(qp, lens, Tq)
    kc = W.pad_prompts(kp, lens, E.Lcap)
    vc = W.pad_prompts(vp, lens, E.Lcap)
    qd, kcd, vcd, lensd = q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV)
    sentinel = torch.full_like(qd, 7.0)
    o, lse = sw.attn_prefill(qd, kcd, vcd, lensd, o=sentinel.clone(), window=window,
                             want_lse=True)
    torch.cuda.synchronize()
    o_r, lse_r = ref.prefill(f64(q), f64(kc), f64(vc), lens.numpy(), window)
    of, lf = f64(o), f64(lse)
    for b in range(E.B):
        L = int(lens[b])
        assert_o(of[b, :L], o_r[b, :L], f"prefill b={b}")
        assert np.abs(lf[b, :, :L] - lse_r[b, :, :L]).max() <= LSE_TOL
        assert np.all(of[b, L:] == 7.0), "rows past the prompt must stay untouched"
    # decode steps: append, then attend with lens + 1
    kc_ref, vc_ref = f64(kc), f64(vc)
    kc_bf, vc_bf = kc.clone(), vc.clone()
    kcs, vcs = kcd.clone(), vcd.clone()  # the same steps through attn_decode_step
    cur = lens.clone()
    ws = torch.empty(sw.attn_decode_workspace_bytes(E.B, E.H, E.Lcap, E.D), device=DEV,
                     dtype=torch.uint8)
    worst = 0.0
    for s in range(E.steps):
        qn, kn, vn = W.engine_decode_step(s, layer, E)
        pos = cur.to(DEV)
        sw.attn_kv_append(kcd, vcd, kn.to(DEV), vn.to(DEV), pos)
        od, lsed = sw.attn_decode(qn.to(DEV), kcd, vcd, (cur + 1).to(DEV), window=window, ws=ws,
                                  want_lse=True)
        os_, lses = sw.attn_decode_step(qn.to(DEV), kn.to(DEV), vn.to(DEV), kcs, vcs, pos,
                                        window=window, ws=ws, want_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(os_, od) and torch.equal(lses, lsed), f"decode step {s}"

        for b in range(E.B):
            kc_ref[b, int(cur[b])] = f64(kn[b])
            vc_ref[b, int(cur[b])] = f64(vn[b])
            kc_bf[b, int(cur[b])] = kn[b]
            vc_bf[b, int(cur[b])] = vn[b]
        od_r, lse_dr = ref.decode(f64(qn), kc_ref, vc_ref, (cur + 1).numpy(), window)
        e = o_excess(f64(od), od_r)
        worst = max(worst, e)
        assert e <= 1.0, f"decode step {s}: O error {e:.3f} x its bar"
        assert np.abs(f64(lsed) - lse_dr).max() <= LSE_TOL
        cur += 1
    # the device cache holds exactly what the reference appended
    assert torch.equal(kcd.cpu(), kc_bf) and torch.equal(vcd.cpu(), vc_bf)
    assert torch.equal(kcs, kcd) and torch.equal(vcs, vcd)


# --------------------------------------------------------------------------- edge sweep
EDGE_T = [1, 17, 63, 64, 65, 127, 128, 129, 300, 1000]


def edge_windows(T):
    return sorted({1, 2, 63, 64, 65, 127, 128, max(1, T - 1), T, T + 5, 2 ** 31 - 1})


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", EDGE_T)
def test_edge_sweep_bf16(sw, T, D):
    q, k, v, do = W.random_attn(1, T, 2, D, seed=1000 + T + D)
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    for w in edge_windows(T):
        o, lse = sw.attn_fwd(qd, kd, vd, window=w)
        g = sw.attn_bwd(qd, kd, vd, o, lse, dod, window=w)
        torch.cuda.synchronize()
        o_r, lse_r = ref.forward(Q, K, V, w, threads=1)
        check_fwd(o, lse, o_r, lse_r, tag=f"T={T} D={D} w={w}")
        check_grads(g, ref.backward(Q, K, V, DO, w, threads=1), tag=f"T={T} D={D} w={w}",
                    zero_bounds=zero_grad_bounds(Q, K, V, DO) + (0.0,))


@pytest.mark.parametrize("T,w,D", [(1, 1, 64), (65, 7, 64), (129, 129, 128), (300, 64, 128),
                                   (257, 2 ** 31 - 1, 64)])
def test_edge_sweep_fp32(sw, T, w, D):
    q, k, v = W.random_attn(2, T, 3, D, seed=2000 + T, dtype=torch.float32, with_do=False)
    o, lse, _ = run_fwd_bwd(sw, q, k, v, None, w)
    o_r, lse_r = ref.forward(f64(q), f64(k), f64(v), w, threads=1)
    check_fwd(o, lse, o_r, lse_r, tag=f"fp32 T={T} w={w} D={D}")
    assert np.abs(f64(o) - o_r).max() < 1e-4


@pytest.mark.slow
@pytest.mark.parametrize("H,window", [(16, None), (4, 1024)])
def test_long_sequence_every_element(sw, H, window):
    """T = 8192, four times the training workloads' length, every element against the oracle.
    H = 16 under the full causal mask fills one round of tile pairs exactly (the paired forward
    and dQ pass, 64 key tiles per dK/dV pair); H = 4 with window 1024 takes single tiles with
    window-edge and diagonal masking far from the sequence start."""
    q, k, v, do = W.random_attn(1, 8192, H, 128, seed=91 + H)
    o, lse, g = run_fwd_bwd(sw, q, k, v, do, window)
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    o_r, lse_r = ref.forward(Q, K, V, window)
    tag = f"B1 H{H} T8192 w{window}"
    check_fwd(o, lse, o_r, lse_r, tag=tag)
    del o_r, lse_r
    check_grads(g, ref.backward(Q, K, V, DO, window), tag=tag)


@pytest.mark.slow
def test_long_sequence_d64_tile_pairs(sw):
    """D = 64 at T = 4096 with 32 heads: 512 tile pairs, one whole round, so the paired forward,
    dQ and dK/dV launches run with the 64-wide fragments and swizzle; every element against the
    oracle."""
    q, k, v, do = W.random_attn(1, 4096, 32, 64, seed=97)
    o, lse, g = run_fwd_bwd(sw, q, k, v, do, None)
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    o_r, lse_r = ref.forward(Q, K, V, None)
    check_fwd(o, lse, o_r, lse_r, tag="B1 H32 T4096 D64")
    del o_r, lse_r
    check_grads(g, ref.backward(Q, K, V, DO, None), tag="B1 H32 T4096 D64")


@pytest.mark.slow
def test_engine_prefill_window_bites(sw):
    """The Engine's 64 ragged prompts (layer 1's inputs) with a window of 256, shorter than most
    prompts, so the window-edge tiles of the ragged prefill are exercised at full size (the
    Engine's own window, 1024, never cuts a prompt of at most 1024 tokens); every prompt row."""
    E = W.D30_ENGINE
    window = 256
    lens = W.engine_lens(E)
    Tq = int(lens.max())
    qp, kp, vp = W.engine_prefill_packed(1, lens, E)
    q = W.pad_prompts(qp, lens, Tq)
    kc = W.pad_prompts(kp, lens, E.Lcap)
    vc = W.pad_prompts(vp, lens, E.Lcap)
    qd, kcd, vcd, lensd = q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV)
    o, lse = sw.attn_prefill(qd, kcd, vcd, lensd, o=torch.full_like(qd, 7.0), window=window,
                             want_lse=True)
    torch.cuda.synchronize()
    o_r, lse_r = ref.prefill(f64(q), f64(kc), f64(vc), lens.numpy(), window)
    of, lf = f64(o), f64(lse)
    assert int((lens > window).sum()) > E.B // 2
    for b in range(E.B):
        L = int(lens[b])
        assert_o(of[b, :L], o_r[b, :L], f"prefill w256 b={b}")
        assert np.abs(lf[b, :, :L] - lse_r[b, :, :L]).max() <= LSE_TOL
        assert np.all(of[b, L:] == 7.0), "rows past the prompt must stay untouched"


def test_multi_batch_head_strides(sw):
    """B, H > 1 with a ragged tail: every (b, h) slice is addressed correctly."""
    q, k, v, do = W.random_attn(3, 150, 5, 128, seed=42)
    o, lse, g = run_fwd_bwd(sw, q, k, v, do, 40)
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    o_r, lse_r = ref.forward(Q, K, V, 40)
    check_fwd(o, lse, o_r, lse_r, tag="B3 H5 T150")
    check_grads(g, ref.backward(Q, K, V, DO, 40), tag="B3 H5 T150")


@pytest.mark.parametrize("D", [64, 128])
def test_single_head_rows_touch(sw, D):
    """H = 1: consecutive tokens' rows touch (row stride D), so a tile's valid rows end exactly where
    the DMA's byte range ends; ragged tails (T = 150, 65) must read as masked, not as the next
    sequence's rows."""
    for B, T, w in ((2, 150, 2 ** 31 - 1), (3, 65, 37)):
        q, k, v, do = W.random_attn(B, T, 1, D, seed=3000 + T + D)
        o, lse, g = run_fwd_bwd(sw, q, k, v, do, w)
        Q, K, V, DO = (f64(t) for t in (q, k, v, do))
        o_r, lse_r = ref.forward(Q, K, V, w, threads=1)
        check_fwd(o, lse, o_r, lse_r, tag=f"H1 B{B} T{T} D{D} w{w}")
        check_grads(g, ref.backward(Q, K, V, DO, w, threads=1), tag=f"H1 B{B} T{T} D{D} w{w}")


@pytest.mark.parametrize("D", [64, 128])
def test_wide_launch_ragged(sw, D):
    """Enough (sequence, head) pairs for the 4-wave forward and dQ launches (small launches take one
    wave per workgroup, which the edge sweep covers), at ragged lengths and windows."""
    for T, w in ((150, 2 ** 31 - 1), (65, 37), (300, 129)):
        q, k, v, do = W.random_attn(4, T, 64, D, seed=4000 + T + D)
        o, lse, g = run_fwd_bwd(sw, q, k, v, do, w)
        Q, K, V, DO = (f64(t) for t in (q, k, v, do))
        o_r, lse_r = ref.forward(Q, K, V, w)
        check_fwd(o, lse, o_r, lse_r, tag=f"B4 H64 T{T} D{D} w{w}")
        check_grads(g, ref.backward(Q, K, V, DO, w), tag=f"B4 H64 T{T} D{D} w{w}")


# --------------------------------------------------------------------------- Engine edge cases
# Decode cases: (B, H, Lcap, cache lengths, windows, launches).  Few or many (sequence, head)
# pairs over short caches take the one-launch schedule; few pairs that may each see more than 2048
# rows take split-K across workgroups plus the merge kernel (the windows keep more than 2048 rows
# visible there).
DECODE_CASES = {
    "one-launch-few": (8, 3, 200, [0, 1, 63, 64, 65, 128, 199, 200], (None, 1, 2, 64, 65, 100, 10 ** 6), 1),
    "one-launch-many": (64, 8, 200, [0, 1, 63, 64, 65, 128, 199, 200], (None, 1, 2, 64, 65, 100, 10 ** 6), 1),
    "split-merge": (8, 3, 2112, [0, 1, 65, 2047, 2048, 2049, 2111, 2112], (None, 2049, 2100, 10 ** 6), 2),
}


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("case", list(DECODE_CASES))
def test_decode_edge_lengths(sw, D, case):
    B, H, Lcap, edge, windows, launches = DECODE_CASES[case]
    lens = torch.tensor([edge[b % len(edge)] for b in range(B)], dtype=torch.int32)
    g = torch.Generator().manual_seed(5 + D)
    kc = torch.randn(B, Lcap, H, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Lcap, H, D, generator=g).to(torch.bfloat16)
    q = torch.randn(B, H, D, generator=g).to(torch.bfloat16)
    kcd, vcd = kc.to(DEV), vc.to(DEV)
    for window in windows:
        assert sw.attn_decode_launches(B, H, Lcap, D, window) == launches, (case, window)
        o, lse = sw.attn_decode(q.to(DEV), kcd, vcd, lens.to(DEV), window=window, want_lse=True)
        torch.cuda.synchronize()
        o_r, lse_r = ref.decode(f64(q), f64(kc), f64(vc), lens.numpy(), window)
        assert_o(f64(o), o_r, f"window {window}")
        lf = f64(lse)
        zero = (lens == 0).numpy()
        assert np.all(f64(o)[zero] == 0) and np.all(np.isneginf(lf[zero]))
        assert np.abs(lf[~zero] - lse_r[~zero]).max() <= LSE_TOL


def test_prefill_ragged_and_window_noop(sw):
    B, H, D, Lcap = 5, 2, 128, 160
    lens = torch.tensor([1, 64, 65, 130, 0], dtype=torch.int32)
    Tq = 130
    g = torch.Generator().manual_seed(77)
    q = torch.randn(B, Tq, H, D, generator=g).to(torch.bfloat16)
    kc = torch.randn(B, Lcap, H, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Lcap, H, D, generator=g).to(torch.bfloat16)
    qd, kcd, vcd, ld = q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV)
    for window in (None, 3, 64, 130):
        o, lse = sw.attn_prefill(qd, kcd, vcd, ld, o=torch.full_like(qd, -3.0), window=window,
                                 want_lse=True)
        torch.cuda.synchronize()
        o_r, lse_r = ref.prefill(f64(q), f64(kc), f64(vc), lens.numpy(), window, threads=1)
        of = f64(o)
        for b in range(B):
            L = int(lens[b])
            if L:
                assert_o(of[b, :L], o_r[b, :L], f"window {window} b {b}")
                assert np.abs(f64(lse)[b, :, :L] - lse_r[b, :, :L]).max() <= LSE_TOL
            assert np.all(of[b, L:] == -3.0)
    # every prompt is <= 130 keys: window 130 equals full causal bit for bit
    o_full, _ = sw.attn_prefill(qd, kcd, vcd, ld, window=None)
    o_w, _ = sw.attn_prefill(qd, kcd, vcd, ld, window=130)
    for b in range(B):
        L = int(lens[b])
        assert torch.equal(o_full[b, :L], o_w[b, :L])


def test_append_skips_out_of_range_rows(sw):
    B, H, D, Lcap = 3, 2, 64, 10
    kc = torch.zeros(B, Lcap, H, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    kn = torch.ones(B, H, D, dtype=torch.bfloat16, device=DEV)
    pos = torch.tensor([0, 10, -1], dtype=torch.int32, device=DEV)
    sw.attn_kv_append(kc, vc, kn, kn * 2, pos)
    torch.cuda.synchronize()
    assert torch.all(kc[0, 0] == 1) and torch.all(vc[0, 0] == 2)
    assert kc[0, 1:].abs().sum() == 0 and kc[1:].abs().sum() == 0


# --------------------------------------------------------------------------- invariants
def test_determinism_and_full_window_bitwise(sw):
    q, k, v, do = W.random_attn(2, 333, 3, 128, seed=9)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    outs = []
    for _ in range(3):
        o, lse = sw.attn_fwd(qd, kd, vd, window=100)
        outs.append((o, lse) + sw.attn_bwd(qd, kd, vd, o, lse, dod, window=100))
    torch.cuda.synchronize()
    for rep in outs[1:]:
        for a, b in zip(outs[0], rep):
            assert torch.equal(a, b)
    full = sw.attn_fwd(qd, kd, vd, window=None)
    eq = sw.attn_fwd(qd, kd, vd, window=333)
    big = sw.attn_fwd(qd, kd, vd, window=10 ** 9)
    assert torch.equal(full[0], eq[0]) and torch.equal(full[0], big[0])
    assert torch.equal(full[1], eq[1])
    gf = sw.attn_bwd(qd, kd, vd, full[0], full[1], dod, window=None)
    ge = sw.attn_bwd(qd, kd, vd, eq[0], eq[1], dod, window=333)
    for a, b in zip(gf, ge):
        assert torch.equal(a, b)


def test_decode_long_cache_split_merge(sw):
    """Few sequences over a 16384-row cache: up to 256 chunks per (sequence, head) meet in the
    merge kernel (four chunks in flight per thread, plus the remainder), against the oracle."""
    B, H, D, Lcap = 2, 3, 128, 16384
    g = torch.Generator().manual_seed(140)
    kc = torch.randn(B, Lcap, H, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Lcap, H, D, generator=g).to(torch.bfloat16)
    q = torch.randn(B, H, D, generator=g).to(torch.bfloat16)
    lens = torch.tensor([Lcap, 9001], dtype=torch.int32)
    kcd, vcd = kc.to(DEV), vc.to(DEV)
    for window in (None, 5000):
        assert sw.attn_decode_launches(B, H, Lcap, D, window) == 2
        o, lse = sw.attn_decode(q.to(DEV), kcd, vcd, lens.to(DEV), window=window, want_lse=True)
        torch.cuda.synchronize()
        o_r, lse_r = ref.decode(f64(q), f64(kc), f64(vc), lens.numpy(), window)
        assert_o(f64(o), o_r, f"window {window}")
        assert np.abs(f64(lse) - lse_r).max() <= LSE_TOL, f"window {window}"


@pytest.mark.slow
def test_decode_largest_cache(sw):
    """The largest cache the split schedule accepts, Lcap = 65535 x 64 rows: the split kernel's
    grid takes all 65535 chunks of the (sequence, head) on its y dimension and the merge kernel
    combines all of them.  Every row visible, then a window of 3,000,000 rows; against the
    oracle (inputs drawn on the device, the oracle given the same bf16 values)."""
    B, H, D = 1, 1, 128
    Lcap = 65535 * 64
    g = torch.Generator(device=DEV).manual_seed(150)
    kcd = torch.randn((B, Lcap, H, D), device=DEV, generator=g).to(torch.bfloat16)
    vcd = torch.randn((B, Lcap, H, D), device=DEV, generator=g).to(torch.bfloat16)
    qd = torch.randn((B, H, D), device=DEV, generator=g).to(torch.bfloat16)
    lens = torch.tensor([Lcap], dtype=torch.int32)
    K, V, Q = f64(kcd), f64(vcd), f64(qd)
    for window in (None, 3_000_000):
        assert sw.attn_decode_launches(B, H, Lcap, D, window) == 2
        o, lse = sw.attn_decode(qd, kcd, vcd, lens.to(DEV), window=window, want_lse=True)
        torch.cuda.synchronize()
        o_r, lse_r = ref.decode(Q, K, V, lens.numpy(), window)
        assert_o(f64(o), o_r, f"Lcap {Lcap} window {window}")
        assert np.abs(f64(lse) - lse_r).max() <= LSE_TOL, f"Lcap {Lcap} window {window}"


def test_decode_deterministic_and_schedule_independent(sw):
    """Decode repeats bit for bit, and its two schedules agree: the same 4 sequences decoded
    within a batch of 64 (one workgroup per (sequence, head)) and alone (32 pairs over caches of
    more than 2048 rows: 64-key chunks across workgroups, then a merge kernel)."""
    B, H, D, Lcap, Bs = 64, 8, 128, 2176, 4
    g = torch.Generator().manual_seed(130)
    lens = torch.randint(1, Lcap + 1, (B,), generator=g, dtype=torch.int32)
    lens[:2] = torch.tensor([Lcap, 2049], dtype=torch.int32)
    gd = torch.Generator(device=DEV).manual_seed(130)
    kc, vc = (torch.randn(B, Lcap, H, D, generator=gd, device=DEV).to(torch.bfloat16)
              for _ in range(2))
    q = torch.randn(B, H, D, generator=gd, device=DEV).to(torch.bfloat16)
    ld = lens.to(DEV)
    for window in (None, 2100):
        assert sw.attn_decode_launches(B, H, Lcap, D, window) == 1
        assert sw.attn_decode_launches(Bs, H, Lcap, D, window) == 2
        runs = [sw.attn_decode(q, kc, vc, ld, window=window, want_lse=True) for _ in range(3)]
        small = sw.attn_decode(q[:Bs].contiguous(), kc[:Bs].contiguous(), vc[:Bs].contiguous(),
                               ld[:Bs].contiguous(), window=window, want_lse=True)
        torch.cuda.synchronize()
        for o, l in runs[1:]:
            assert torch.equal(o, runs[0][0]) and torch.equal(l, runs[0][1])
        o, l = runs[0]
        assert (o[:Bs].float() - small[0].float()).abs().max().item() <= 2 ** -7 * o.abs().max().item()
        assert (l[:Bs] - small[1]).abs().max().item() <= 1e-4


def test_split_passes_equal_attn_bwd(sw):
    q, k, v, do = W.random_attn(2, 200, 3, 128, seed=14)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = sw.attn_fwd(qd, kd, vd, window=70)
    g = sw.attn_bwd(qd, kd, vd, o, lse, dod, window=70)
    ws = torch.empty(sw.attn_bwd_workspace_bytes(2, 3, 200, 128), device=DEV, dtype=torch.uint8)
    dq = sw.attn_bwd_dq(qd, kd, vd, o, lse, dod, ws, window=70)
    dk, dv = sw.attn_bwd_dkdv(qd, kd, vd, lse, dod, ws, window=70)
    torch.cuda.synchronize()
    for a, b in zip(g, (dq, dk, dv)):
        assert torch.equal(a, b)


def test_gradient_sum_invariants(sw):
    q, k, v, do = W.random_attn(1, 256, 2, 128, seed=10)
    o, lse, (dq, dk, dv) = run_fwd_bwd(sw, q, k, v, do, 50)
    dk64, dv64, do64 = f64(dk), f64(dv), f64(do)
    scale = np.abs(dk64).sum(1).max()
    assert np.abs(dk64.sum(1)).max() <= 2e-2 * scale
    assert np.abs(dv64.sum(1) - do64.sum(1)).max() <= 2e-2 * np.abs(do64).sum(1).max()
    # sum_i q_i . dQ_i = sum_j k_j . dK_j (both equal sum_ij dS_ij q_i . k_j / sqrt(D)), per head
    q64, k64, dq64 = f64(q), f64(k), f64(dq)
    lhs = (q64 * dq64).sum(axis=(1, 3))
    rhs = (k64 * dk64).sum(axis=(1, 3))
    assert np.abs(lhs - rhs).max() <= 2e-2 * np.abs(q64 * dq64).sum(axis=(1, 3)).max()


def test_decode_matches_prefill_last_row(sw):
    B, H, D, Lcap = 4, 3, 128, 256
    lens = torch.tensor([1, 70, 129, 256], dtype=torch.int32)
    g = torch.Generator().manual_seed(11)
    q = torch.randn(B, 256, H, D, generator=g).to(torch.bfloat16)
    kc = torch.randn(B, Lcap, H, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Lcap, H, D, generator=g).to(torch.bfloat16)
    qd, kcd, vcd, ld = q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV)
    for window in (None, 17):
        o, _ = sw.attn_prefill(qd, kcd, vcd, ld, window=window)
        qlast = torch.stack([qd[b, int(lens[b]) - 1] for b in range(B)])
        od, _ = sw.attn_decode(qlast.contiguous(), kcd, vcd, ld, window=window)
        torch.cuda.synchronize()
        for b in range(B):
            a = f64(o[b, int(lens[b]) - 1])
            assert_o(f64(od[b]), a, f"decode vs prefill row, b {b}")


def test_autograd_wrapper_and_kvcache(sw):
    q, k, v, do = W.random_attn(1, 96, 2, 64, seed=12)
    qd, kd, vd = (t.to(DEV).requires_grad_() for t in (q, k, v))
    o = sw.attention(qd, kd, vd, window=32)
    o.backward(do.to(DEV))
    g_r = ref.backward(f64(q), f64(k), f64(v), f64(do), 32)
    check_grads((qd.grad, kd.grad, vd.grad), g_r, tag="autograd")

    cache = sw.KVCache(2, 2, 64, 2, 64, windows=[None, 8])
    lens = torch.tensor([3, 10], dtype=torch.int32, device=DEV)
    g = torch.Generator().manual_seed(13)
    qp, kp, vp = (torch.randn(2, 10, 2, 64, generator=g).to(torch.bfloat16).to(DEV)
                  for _ in range(3))
    for layer in range(2):
        cache.prefill(layer, qp, kp, vp, lens)
    qn, kn, vn = (torch.randn(2, 2, 64, generator=g).to(torch.bfloat16).to(DEV) for _ in range(3))
    od = cache.decode(1, qn, kn, vn)
    torch.cuda.synchronize()
    kc, vc = f64(cache.k[1]), f64(cache.v[1])
    od_r, _ = ref.decode(f64(qn), kc, vc, np.array([4, 11]), 8)
    assert_o(f64(od), od_r, "kvcache decode")


# ------------------------------------------------------------------ decode step (append + decode)
STEP_CASES = {  # (B, H, Lcap, positions, windows, launches)
    "one-launch-few": (8, 3, 200, [0, 1, 63, 64, 65, 128, 199, -1, 200], (None, 1, 2, 64, 65, 100), 1),
    "one-launch-many": (64, 8, 200, [0, 1, 63, 64, 65, 128, 199, -1, 200], (None, 1, 2, 64, 65, 100), 1),
    "split-merge": (8, 3, 2112, [0, 1, 2047, 2048, 2110, 2111, -1, 2112], (None, 2049, 2100), 2),
}


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("case", list(STEP_CASES))
def test_decode_step_equals_append_then_decode(sw, D, case):
    """attn_decode_step(pos) is attn_kv_append(pos) then attn_decode(lens = pos + 1), bit for bit,
    and matches the oracle; a pos outside [0, Lcap) writes nothing and gives o = 0, lse = -inf."""
    B, H, Lcap, edge, windows, launches = STEP_CASES[case]
    pos = torch.tensor([edge[b % len(edge)] for b in range(B)], dtype=torch.int32)
    valid = ((pos >= 0) & (pos < Lcap)).numpy()
    g = torch.Generator().manual_seed(21 + D)
    kc = torch.randn(B, Lcap, H, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Lcap, H, D, generator=g).to(torch.bfloat16)
    q, kn, vn = (torch.randn(B, H, D, generator=g).to(torch.bfloat16) for _ in range(3))
    qd, knd, vnd, posd = q.to(DEV), kn.to(DEV), vn.to(DEV), pos.to(DEV)
    lens_after = torch.where(pos >= 0, pos + 1, torch.zeros_like(pos)).to(DEV)
    kc_r, vc_r = f64(kc), f64(vc)
    vb = np.nonzero(valid)[0]  # the oracle's append covers in-range rows only
    kc_r[vb], vc_r[vb] = ref.kv_append(kc_r[vb], vc_r[vb], f64(kn)[vb], f64(vn)[vb],
                                       pos.numpy()[vb])
    for window in windows:
        assert sw.attn_decode_launches(B, H, Lcap, D, window) == launches, (case, window)
        k1, v1 = kc.to(DEV), vc.to(DEV)
        o1, lse1 = sw.attn_decode_step(qd, knd, vnd, k1, v1, posd, window=window, want_lse=True)
        k2, v2 = kc.to(DEV), vc.to(DEV)
        sw.attn_kv_append(k2, v2, knd, vnd, posd)
        o2, lse2 = sw.attn_decode(qd, k2, v2, lens_after, window=window, want_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(k1, k2) and torch.equal(v1, v2), f"cache after the step, window {window}"
        assert torch.equal(o1[valid], o2[valid]) and torch.equal(lse1[valid], lse2[valid]), window
        assert torch.all(o1[~valid] == 0) and torch.all(torch.isneginf(lse1[~valid]))
        o_r, lse_r = ref.decode(f64(q), kc_r, vc_r, np.where(valid, pos.numpy() + 1, 0), window)
        assert_o(f64(o1), o_r, f"window {window}")
        assert np.abs(f64(lse1)[valid] - lse_r[valid]).max() <= LSE_TOL


@pytest.mark.parametrize("B,H,Lcap,windows", [(4, 2, 96, [None, 5, 40]), (64, 8, 96, [None, 5, 40]),
                                               (4, 2, 2100, [None, 5, 2049])])
def test_decode_step_graph_replays_match_eager(sw, B, H, Lcap, windows):
    """A captured decode step over every layer, replayed token after token with unrelated eager
    work and synchronisations in between, equals the same steps run eagerly, bit for bit.  With
    Lcap = 2100 the layers with more than 2048 visible rows capture the two-launch schedule."""
    n_layer, D = 3, 128
    launches = [sw.attn_decode_launches(B, H, Lcap, D, w) for w in windows]
    assert launches == ([2, 1, 2] if Lcap > 2048 else [1, 1, 1])
    g = torch.Generator().manual_seed(31 + B)
    lens0 = torch.randint(1, 60, (B,), generator=g, dtype=torch.int32)
    Tq = int(lens0.max())
    caches = [sw.KVCache(n_layer, B, Lcap, H, D, windows=windows) for _ in range(2)]
    prompt = [[torch.randn(B, Tq, H, D, generator=g).to(torch.bfloat16).to(DEV) for _ in range(3)]
              for _ in range(n_layer)]
    for c in caches:
        for layer in range(n_layer):
            c.prefill(layer, *prompt[layer], lens0.to(DEV))
    eager, graphed = caches
    step_graph = sw.DecodeStepGraph(graphed)
    junk = torch.randn(512, 512, device=DEV)
    for s in range(4):
        ins = [torch.randn(n_layer, B, H, D, generator=g).to(torch.bfloat16).to(DEV)
               for _ in range(3)]
        o_e = torch.stack([eager.decode(layer, ins[0][layer], ins[1][layer], ins[2][layer])
                           for layer in range(n_layer)])
        eager.step()
        step_graph.q.copy_(ins[0])
        step_graph.k_new.copy_(ins[1])
        step_graph.v_new.copy_(ins[2])
        o_g = step_graph.replay()
        junk = (junk @ junk).tanh_()  # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {s}"
        assert torch.equal(graphed.lens, eager.lens)
        assert torch.equal(graphed.k, eager.k) and torch.equal(graphed.v, eager.v), f"replay {s}"
        # the eager path itself against the oracle, last layer
        lens_now = f64(eager.lens).astype(np.int64)
        o_r, _ = ref.decode(f64(ins[0][-1]), f64(eager.k[-1]), f64(eager.v[-1]), lens_now,
                            windows[-1])
        assert_o(f64(o_e[-1]), o_r, f"replay {s}")


# ------------------------------------------------------------- packed documents (varlen)
def _packed(lengths, H, D, seed):
    g = torch.Generator().manual_seed(seed)
    total = int(sum(lengths))
    cu = torch.tensor([0] + [int(x) for x in np.cumsum(lengths)], dtype=torch.int32)
    q, k, v, do = (torch.randn(total, H, D, generator=g).to(torch.bfloat16) for _ in range(4))
    return cu, q, k, v, do


@pytest.mark.parametrize("D", [64, 128])
def test_varlen_matches_oracle(sw, D):
    """Packed documents of assorted lengths (tile edges, a single token, an empty one) against the
    oracle, forward and backward, for several windows."""
    lengths = [129, 1, 64, 0, 300, 31, 65, 128, 33, 200]
    H = 3
    cu, q, k, v, do = _packed(lengths, H, D, 90 + D)
    qd, kd, vd, dod, cud = (t.to(DEV) for t in (q, k, v, do, cu))
    for window in (None, 1, 17, 64, 100):
        o, lse = sw.attn_fwd_varlen(qd, kd, vd, cud, max(lengths), window=window)
        g = sw.attn_bwd_varlen(qd, kd, vd, o, lse, dod, cud, max(lengths), window=window)
        torch.cuda.synchronize()
        o_r, lse_r = ref.forward_varlen(f64(q), f64(k), f64(v), cu.numpy(), window)
        assert_o(f64(o), o_r, f"window {window}")
        assert np.abs(f64(lse) - lse_r).max() <= LSE_TOL, f"window {window}"
        g_r = ref.backward_varlen(f64(q), f64(k), f64(v), f64(do), cu.numpy(), window)
        check_grads(g, g_r, tag=f"varlen D{D} window {window}",
                    zero_bounds=zero_grad_bounds(f64(q), f64(k), f64(v), f64(do)) + (0.0,))


@pytest.mark.slow
def test_varlen_long_document(sw):
    """A packed buffer whose longest document is 16384 tokens, eight times the bench's row length,
    beside short ones: the launch is sized by that document (128 query tiles of 128) and the
    dK/dV job plan has 128 levels; forward and backward against the oracle, full and windowed."""
    lengths = [3000, 16384, 5, 1, 700]
    H = 2
    cu, q, k, v, do = _packed(lengths, H, 128, 160)
    qd, kd, vd, dod, cud = (t.to(DEV) for t in (q, k, v, do, cu))
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    for window in (None, 2048):
        o, lse = sw.attn_fwd_varlen(qd, kd, vd, cud, max(lengths), window=window)
        g = sw.attn_bwd_varlen(qd, kd, vd, o, lse, dod, cud, max(lengths), window=window)
        torch.cuda.synchronize()
        o_r, lse_r = ref.forward_varlen(Q, K, V, cu.numpy(), window)
        assert_o(f64(o), o_r, f"long document, window {window}")
        assert np.abs(f64(lse) - lse_r).max() <= LSE_TOL, f"long document, window {window}"
        del o_r, lse_r
        g_r = ref.backward_varlen(Q, K, V, DO, cu.numpy(), window)
        check_grads(g, g_r, tag=f"long document, window {window}")


def test_varlen_is_each_document_alone_bit_for_bit(sw):
    """Each packed document gives exactly what the dense entry points give for it alone."""
    lengths = [70, 1, 129, 256, 0, 33]
    H, D = 2, 128
    cu, q, k, v, do = _packed(lengths, H, D, 95)
    qd, kd, vd, dod, cud = (t.to(DEV) for t in (q, k, v, do, cu))
    for window in (None, 40):
        o, lse = sw.attn_fwd_varlen(qd, kd, vd, cud, max(lengths), window=window)
        dq, dk, dv = sw.attn_bwd_varlen(qd, kd, vd, o, lse, dod, cud, max(lengths), window=window)
        for a, e in zip(cu[:-1].tolist(), cu[1:].tolist()):
            if e == a:
                continue
            sl = slice(a, e)
            one = [t[sl].unsqueeze(0).contiguous() for t in (qd, kd, vd, dod)]
            od, lsed = sw.attn_fwd(one[0], one[1], one[2], window=window)
            gd = sw.attn_bwd(one[0], one[1], one[2], od, lsed, one[3], window=window)
            torch.cuda.synchronize()
            assert torch.equal(o[sl], od[0]) and torch.equal(lse[:, sl], lsed[0]), (window, a)
            for x, y in zip((dq, dk, dv), gd):
                assert torch.equal(x[sl], y[0]), (window, a)


@pytest.mark.parametrize("case", ["queue", "full_plan", "fallback"])
def test_varlen_many_documents(sw, case):
    """Many packed documents. queue: 600 documents of 0-300 tokens (about 1200 dK/dV jobs per
    head, far more than workgroups, handed out by the pass's job queue); full_plan: 6000
    documents of 0-3 tokens, a job plan of 6002 of its 6144 entries; fallback: 6200 such
    documents, too many for the plan, so the dK/dV pass runs one workgroup per unit.  Forward
    and backward against the oracle, and a second run equal bit for bit."""
    rng = np.random.default_rng({"queue": 131, "full_plan": 134, "fallback": 132}[case])
    if case == "queue":
        lengths, H, windows = rng.integers(0, 301, 600).tolist(), 2, (None, 50)
    else:
        n = 6000 if case == "full_plan" else 6200
        lengths, H, windows = rng.integers(0, 4, n).tolist(), 1, (None,)
    D = 64
    cu, q, k, v, do = _packed(lengths, H, D, 133)
    qd, kd, vd, dod, cud = (t.to(DEV) for t in (q, k, v, do, cu))
    ms = max(lengths)
    for window in windows:
        o, lse = sw.attn_fwd_varlen(qd, kd, vd, cud, ms, window=window)
        g = sw.attn_bwd_varlen(qd, kd, vd, o, lse, dod, cud, ms, window=window)
        g2 = sw.attn_bwd_varlen(qd, kd, vd, o, lse, dod, cud, ms, window=window)
        torch.cuda.synchronize()
        for a, b in zip(g, g2):
            assert torch.equal(a, b), f"{case} window {window}: second run differs"
        o_r, lse_r = ref.forward_varlen(f64(q), f64(k), f64(v), cu.numpy(), window)
        assert_o(f64(o), o_r, f"{case} window {window}")
        assert np.abs(f64(lse) - lse_r).max() <= LSE_TOL, f"{case} window {window}"
        g_r = ref.backward_varlen(f64(q), f64(k), f64(v), f64(do), cu.numpy(), window)
        check_grads(g, g_r, tag=f"varlen {case} window {window}",
                    zero_bounds=zero_grad_bounds(f64(q), f64(k), f64(v), f64(do)) + (0.0,))


def test_varlen_autograd_and_rows_past_max_seqlen(sw):
    lengths = [40, 90, 7]
    H, D = 2, 64
    cu, q, k, v, do = _packed(lengths, H, D, 97)
    cud = cu.to(DEV)
    qd, kd, vd = (t.to(DEV).requires_grad_() for t in (q, k, v))
    o = sw.attention_varlen(qd, kd, vd, cud, max(lengths), window=25)
    o.backward(do.to(DEV))
    g_r = ref.backward_varlen(f64(q), f64(k), f64(v), f64(do), cu.numpy(), 25)
    check_grads((qd.grad, kd.grad, vd.grad), g_r, tag="varlen autograd")
    # max_seqlen below the longest document: its rows past max_seqlen are left untouched, the
    # rows before it (which see only earlier keys) are exact
    o2 = torch.full_like(qd, 7.0, requires_grad=False)
    sw.attn_fwd_varlen(qd.detach(), kd.detach(), vd.detach(), cud, 64, o=o2, window=25,
                       want_lse=False)
    torch.cuda.synchronize()
    o_r, _ = ref.forward_varlen(f64(q), f64(k), f64(v), cu.numpy(), 25)
    a = int(cu[1])
    assert torch.all(o2[a + 64:a + 90] == 7.0)
    assert_o(f64(o2[a:a + 64]), o_r[a:a + 64], "rows before max_seqlen")
    assert_o(f64(o2[:a]), o_r[:a], "first document")


# ------------------------------------------------------------------------------ QK-norm
@pytest.mark.parametrize("D", [64, 128])
def test_qknorm_matches_oracle(sw, D):
    """Attention over RMS-normalised q, k against the oracle (normalised rows rounded to bf16, as
    stored); q and k are drawn far from unit RMS so that the norm matters."""
    B, T, H, eps = 2, 300, 3, 1e-6
    g = torch.Generator().manual_seed(110 + D)
    q = (3.0 * torch.randn(B, T, H, D, generator=g)).to(torch.bfloat16)
    k = (0.5 * torch.randn(B, T, H, D, generator=g)).to(torch.bfloat16)
    v, do = (torch.randn(B, T, H, D, generator=g).to(torch.bfloat16) for _ in range(2))
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    for window in (None, 50):
        o, lse, qn, kn, rq, rk = sw.attn_fwd_qknorm(qd, kd, vd, window=window, eps=eps)
        g3 = sw.attn_bwd_qknorm(qn, kn, vd, o, lse, dod, rq, rk, window=window)
        torch.cuda.synchronize()
        o_r, lse_r, qn_r, kn_r = ref.forward_qknorm(f64(q), f64(k), f64(v), window, eps)
        # normalised rows: within one bf16 rounding step of the oracle's (fp32 vs fp64 scale)
        for a, b in ((qn, qn_r), (kn, kn_r)):
            assert np.abs(f64(a) - b).max() <= 2 ** -7 * np.abs(b).max()
        _, r_q = ref.rmsnorm(f64(q), eps)
        assert np.abs(f64(rq) - r_q.transpose(0, 2, 1)).max() <= 1e-5 * np.abs(r_q).max()
        assert_o(f64(o), o_r, f"window {window}")
        assert np.abs(f64(lse) - lse_r).max() <= LSE_TOL, f"window {window}"
        g_r = ref.backward_qknorm(f64(q), f64(k), f64(v), f64(do), window, eps)
        check_grads(g3, g_r, tag=f"qknorm D{D} window {window}")


def test_qknorm_fused_epilogue_equals_unfused_composition(sw):
    """The norm's backward inside the passes' epilogues equals the plain composition: attn_bwd on
    the normalised rows, then dx = r (g - y (g . y) / D) in float32 on the device."""
    B, T, H, D = 1, 200, 2, 128
    g = torch.Generator().manual_seed(120)
    q, k, v, do = (torch.randn(B, T, H, D, generator=g).mul(s).to(torch.bfloat16).to(DEV)
                   for s in (2.0, 0.7, 1.0, 1.0))
    o, lse, qn, kn, rq, rk = sw.attn_fwd_qknorm(q, k, v, window=64)
    dq, dk, dv = sw.attn_bwd_qknorm(qn, kn, v, o, lse, do, rq, rk, window=64)
    gq, gk, gv = sw.attn_bwd(qn, kn, v, o, lse, do, window=64)

    def through(gr, y, r):
        gr, y = gr.float(), y.float()
        rr = r.permute(0, 2, 1).unsqueeze(-1)  # [B, T, H, 1]
        return rr * (gr - y * (gr * y).sum(-1, keepdim=True) / D)

    for fused, unfused in ((dq, through(gq, qn, rq)), (dk, through(gk, kn, rk)), (dv, gv.float())):
        e = rel_fro(f64(fused), f64(unfused))
        assert e <= 1e-2, e


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("shape", [(2, 333, 3), (4, 600, 16)])  # one-wave and 4-wave launches
def test_qknorm_prologue_matches_norm_pass(sw, D, shape):
    """q is normalised inside the forward's prologue and k by the separate pass: on equal rows the
    two give bit-identical normalised rows and r, and O / LSE are bit for bit those of the plain
    forward over the rows the call wrote."""
    B, T, H = shape
    g = torch.Generator().manual_seed(130 + D + T)
    x = (1.7 * torch.randn(B, T, H, D, generator=g)).to(torch.bfloat16).to(DEV)
    v = torch.randn(B, T, H, D, generator=g).to(torch.bfloat16).to(DEV)
    for window in (None, 77):
        o, lse, qn, kn, rq, rk = sw.attn_fwd_qknorm(x, x, v, window=window, eps=1e-5)
        o2, lse2 = sw.attn_fwd(qn, kn, v, window=window)
        torch.cuda.synchronize()
        assert torch.equal(qn, kn), f"window {window}"
        assert torch.equal(rq, rk), f"window {window}"
        assert torch.equal(o, o2), f"window {window}"
        assert torch.equal(lse, lse2), f"window {window}"


def test_qknorm_autograd_wrapper(sw):
    q, k, v, do = W.random_attn(1, 96, 2, 64, seed=121)
    qd, kd, vd = (t.to(DEV).requires_grad_() for t in (q, k, v))
    o = sw.attention_qknorm(qd, kd, vd, window=40, eps=1e-5)
    o.backward(do.to(DEV))
    g_r = ref.backward_qknorm(f64(q), f64(k), f64(v), f64(do), 40, 1e-5)
    check_grads((qd.grad, kd.grad, vd.grad), g_r, tag="qknorm autograd")


# ------------------------------------------------- full-size NEXT workloads, every head
@pytest.mark.slow
def test_d20_packed_documents_every_head(sw):
    """The bench's packed-document d20 rows (same q, k, v, dO as the d20 layer), forward and
    backward in the bench's launch configuration, every document and head against the oracle:
    O and LSE max-abs over all rows, dQ / dK / dV relative Frobenius over the whole tensors."""
    c = W.D20_LAYER
    q, k, v, do = W.attn_inputs(c)
    B, T, H, D = q.shape
    cu = W.d20_packed_cu(B, T)
    lens = (cu[1:] - cu[:-1]).tolist()
    ms = max(lens)
    qp, kp, vp, dop = (t.reshape(B * T, H, D) for t in (q, k, v, do))
    qd, kd, vd, dod = (t.to(DEV) for t in (qp, kp, vp, dop))
    o, lse = sw.attn_fwd_varlen(qd, kd, vd, cu.to(DEV), ms, window=c.window)
    g = sw.attn_bwd_varlen(qd, kd, vd, o, lse, dod, cu.to(DEV), ms, window=c.window)
    torch.cuda.synchronize()
    Q, K, V, DO = (f64(t) for t in (qp, kp, vp, dop))
    o_r, lse_r = ref.forward_varlen(Q, K, V, cu.numpy(), c.window)
    assert_o(f64(o), o_r, "packed d20")
    el = float(np.abs(f64(lse) - lse_r).max())
    assert el <= LSE_TOL, f"packed d20 LSE max-abs {el}"
    del o_r, lse_r
    check_grads(g, ref.backward_varlen(Q, K, V, DO, cu.numpy(), c.window), tag="packed d20")


@pytest.mark.slow
def test_d20_qknorm_every_head(sw):
    """QK-norm on the d20 layer in the bench's configuration, every head against the oracle."""
    c = W.D20_LAYER
    q, k, v, do = W.attn_inputs(c)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse, qn, kn, rq, rk = sw.attn_fwd_qknorm(qd, kd, vd, window=c.window)
    g = sw.attn_bwd_qknorm(qn, kn, vd, o, lse, dod, rq, rk, window=c.window)
    torch.cuda.synchronize()
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    o_r, lse_r, _, _ = ref.forward_qknorm(Q, K, V, c.window)
    check_fwd(o, lse, o_r, lse_r, tag="d20 qknorm")
    del o_r, lse_r
    check_grads(g, ref.backward_qknorm(Q, K, V, DO, c.window), tag="d20 qknorm")


@pytest.mark.slow
def test_d26_window_layer_qknorm_every_head(sw):
    """QK-norm on the d26 window-512 layer (B 16, T 2048, H 13), q and k drawn far from unit RMS so
    that the norm matters: the QK-norm forward and dQ pass as single tiles and the dK/dV pass one
    workgroup per key tile, every head against the oracle."""
    window = W.D26_WINDOWS[0]
    q, k, v, do = W.d26_layer_inputs(0)
    q = (3.0 * q.float()).to(torch.bfloat16)
    k = (0.5 * k.float()).to(torch.bfloat16)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse, qn, kn, rq, rk = sw.attn_fwd_qknorm(qd, kd, vd, window=window)
    g = sw.attn_bwd_qknorm(qn, kn, vd, o, lse, dod, rq, rk, window=window)
    torch.cuda.synchronize()
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    o_r, lse_r, _, _ = ref.forward_qknorm(Q, K, V, window)
    check_fwd(o, lse, o_r, lse_r, tag="d26 w512 qknorm")
    del o_r, lse_r
    check_grads(g, ref.backward_qknorm(Q, K, V, DO, window), tag="d26 w512 qknorm")


@pytest.mark.slow
def test_full_size_runs_repeat_bit_for_bit(sw):
    """Deterministic at full size: the d20 layer (tile pairs, the persistent dK/dV grid), a d26
    window-512 layer (single tiles) and the packed d20 rows (the dK/dV job queue, whose hand-out
    to workgroups varies from run to run) give the same bits on a second run, forward and
    backward."""
    c = W.D20_LAYER
    q, k, v, do = (t.to(DEV) for t in W.attn_inputs(c))
    B, T, H, D = q.shape
    q6, k6, v6, do6 = (t.to(DEV) for t in W.d26_layer_inputs(0))
    cu = W.d20_packed_cu(B, T).to(DEV)
    ms = int((cu[1:] - cu[:-1]).max())
    qv, kv, vv, dov = (t.view(B * T, H, D) for t in (q, k, v, do))

    def runs():
        o, lse = sw.attn_fwd(q, k, v, window=c.window)
        g = sw.attn_bwd(q, k, v, o, lse, do, window=c.window)
        o6, lse6 = sw.attn_fwd(q6, k6, v6, window=W.D26_WINDOWS[0])
        g6 = sw.attn_bwd(q6, k6, v6, o6, lse6, do6, window=W.D26_WINDOWS[0])
        ov, lsev = sw.attn_fwd_varlen(qv, kv, vv, cu, ms)
        gv = sw.attn_bwd_varlen(qv, kv, vv, ov, lsev, dov, cu, ms)
        torch.cuda.synchronize()
        return [o, lse, *g, o6, lse6, *g6, ov, lsev, *gv]

    first, second = runs(), runs()
    names = ["o", "lse", "dq", "dk", "dv"]
    for i, (a, b) in enumerate(zip(first, second)):
        tag = ["d20", "d26 w512", "packed"][i // 5] + " " + names[i % 5]
        assert torch.equal(a, b), f"{tag} differs between two runs"
