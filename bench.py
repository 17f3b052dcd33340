#!/usr/bin/env python3
"""Benchmark of the windowed causal attention hot path on one MI355X.

One step is one pass over every part of the path, on synthetic data of the pages' shapes:
  * the d20 training layer (B=32, T=2048, H=10, D=128, bf16, full causal): forward, dQ pass,
    dK/dV pass;
  * one Engine decode step of the d30-style model (30 layers, B=64, H=15, D=128, cache 2048,
    prompts U[32,1024], window 1024 on odd layers): every layer's KV append, then every
    layer's decode (split-K inside each workgroup at this batch), the 30 decodes between one
    pair of events;
  * one Engine prefill layer (the same prompts, layer step % 30).
Every part is bracketed by HIP events on the stream the kernels run on.

The headline ``value`` is the d20 fwd+bwd rate in TFLOP/s counting unmasked FLOPs only (4D per
visible (query, key) pair forward, 10D backward).  ``decode`` reports algorithmic HBM GB/s (every
visible cache row read once, plus q and o), next to a plain streaming read of the same byte count
(the rate this GPU sustains at that size), and ``decode.step_graph`` the same decode step for all
30 layers as one replay of a captured HIP graph (attn_decode_step: append and decode in one launch
per layer); ``decode.small_batch`` the first 8 sequences alone, and ``decode.long_context`` 2
sequences over 16384 cached rows, where the decode takes its two-kernel schedule (split-K partials
across workgroups, then the merge kernel); ``prefill`` TFLOP/s; ``varlen`` the d20 rows re-read as packed documents that attend
only to themselves (attn_fwd_varlen / attn_bwd_varlen); ``qknorm`` the d20 layer with RMS-normalised
q and k (attn_fwd_qknorm / attn_bwd_qknorm); ``d26`` the alternating-window d26 layers (window
512 and full causal, B=16, H=13); ``small_configs`` the tiny fp32 forward and the small bf16
fwd + bwd (launch-latency bound).  ``roofline`` describes the
longest-running MFMA kernel; ``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
d20 workload on the host cores.  One JSON line goes to stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd+bwd TFLOP/s (unmasked FLOPs) & % bf16 MFMA peak; decode HBM GB/s"
PEAK_MFMA_BF16 = 2500.0  # TFLOP/s, MI355X dense bf16 (published)
PEAK_HBM = 8000.0        # GB/s, MI355X HBM3E (published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pairs(T: int, w) -> int:
    """Visible (query, key) pairs of one causal head with window w (None = full)."""
    w = T if w is None else min(int(w), T)
    return w * (w + 1) // 2 + (T - w) * w


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "causal_sliding_window_attn_amd", "csrc", "*"))):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def stream_read_gbs(bufs, nbytes: int, reps: int = 3) -> float:
    """GB/s of a plain streaming read of nbytes per call (libswattn_probe.so), one call per
    buffer in turn so that no call finds its bytes in the last-level cache."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "causal_sliding_window_attn_amd", "libswattn_probe.so"))
    lib.swattn_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_void_p]
    lib.swattn_stream_read.restype = ctypes.c_int
    blocks = 1024
    out = torch.empty(blocks * 256, dtype=torch.int32, device=bufs[0].device)
    st = torch.cuda.current_stream()
    nbytes = nbytes // 16 * 16

    def run():
        for b in bufs:
            assert b.numel() * b.element_size() >= nbytes
            rc = lib.swattn_stream_read(b.data_ptr(), nbytes, out.data_ptr(), blocks,
                                        ctypes.c_void_p(st.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"swattn_stream_read failed ({rc})")

    run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / (reps * len(bufs))
    return nbytes / t / 1e9


def cpu_baseline(case, q, k, v, do, n_heads: int):
    """The fp64 oracle, as it stands, on n_heads (b, h) heads of the d20 layer, fwd + bwd."""
    import torch

    from oracle import attention as ref

    B, H = case.B, case.H
    n_heads = min(n_heads, B * H)
    if n_heads == B * H:  # the whole layer
        heads = [(b, h) for b in range(B) for h in range(H)]
    else:  # a spread of distinct heads
        heads = sorted({((i * 13) % B, (i * 7) % H) for i in range(4 * n_heads)})[:n_heads]
    pick = lambda t: torch.stack([t[b, :, h] for b, h in heads])[:, :, None, :].double().numpy()  # noqa: E731
    Q, K, V, DO = pick(q), pick(k), pick(v), pick(do)
    threads = min(16, len(os.sched_getaffinity(0)))
    t0 = time.perf_counter()
    ref.forward(Q, K, V, case.window, threads=threads)
    ref.backward(Q, K, V, DO, case.window, threads=threads)
    dt = time.perf_counter() - t0
    flops = 14 * case.D * pairs(case.T, case.window) * len(heads)
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"fp64 oracle fwd+bwd on {len(heads)} of the {B * H} (b,h) heads of the d20 "
                  f"layer (T={case.T}, D={case.D}, full causal), same seeded inputs; {dt:.2f} s "
                  f"wall on {threads} threads",
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-heads", type=int, default=320)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-ref", action="store_true",
                    help="skip the streaming-read reference of the decode roofline")
    ap.add_argument("--no-step-graph", action="store_true",
                    help="skip the graph-replayed whole-model decode step measurement")
    ap.add_argument("--no-qknorm", action="store_true",
                    help="skip the QK-norm (normalised q, k) fwd+bwd measurement")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the packed-document (varlen) fwd+bwd measurement")
    ap.add_argument("--no-d26", action="store_true",
                    help="skip the d26 alternating-window layers (w = 512 and full) measurement")
    ap.add_argument("--no-small-configs", action="store_true",
                    help="skip the tiny fp32 and small bf16 configuration measurements")
    ap.add_argument("--no-small-batch", action="store_true",
                    help="skip the small-batch decode measurement")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the long-context decode (split-K across workgroups + merge kernel) "
                         "measurement")
    ap.add_argument("--calib-copy-mib", type=int, default=1024,
                    help="after the timed region, one plain device copy of this size (the "
                         "reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single GPU: this attention path is data parallel over "
              "(batch, head) with no exchange between GPUs, and only the one-GPU figure is "
              "measured here (run with --gpus 1).", file=sys.stderr)
        return 2

    import torch

    import causal_sliding_window_attn_amd as sw
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sw.load()
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name}, {props.multi_processor_count} CUs")

    # ------------------------------------------------------------------ d20 training layer
    case = W.D20_LAYER
    log("drawing d20 inputs ...")
    q_c, k_c, v_c, do_c = W.attn_inputs(case)
    q, k, v, do = (t.to(dev) for t in (q_c, k_c, v_c, do_c))
    B, T, H, D = case.B, case.T, case.H, case.D
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_b = torch.empty(sw.attn_bwd_workspace_bytes(B, H, T, D), device=dev, dtype=torch.uint8)
    P20 = pairs(T, case.window) * B * H
    F_fwd = 4 * D * P20
    F_dq = 2 * D * P20
    F_dkdv = 8 * D * P20

    # ------------------------------------------------------------------ d30 Engine
    E = W.D30_ENGINE
    lens0 = W.engine_lens(E)
    Tq = int(lens0.max())
    log(f"allocating Engine caches: {E.n_layer} layers x 2 x {E.B}x{E.Lcap}x{E.H}x{E.D} bf16 ...")
    g = torch.Generator(device=dev).manual_seed(E.seed)
    eng = sw.KVCache(E.n_layer, E.B, E.Lcap, E.H, E.D, device=dev,
                     windows=[E.window(l) for l in range(E.n_layer)])
    for l in range(E.n_layer):
        eng.k[l].copy_(torch.randn((E.B, E.Lcap, E.H, E.D), device=dev, dtype=torch.bfloat16,
                                   generator=g))
    for l in range(E.n_layer):
        eng.v[l].copy_(torch.randn((E.B, E.Lcap, E.H, E.D), device=dev, dtype=torch.bfloat16,
                                   generator=g))
    kcache = [eng.k[l] for l in range(E.n_layer)]
    vcache = [eng.v[l] for l in range(E.n_layer)]
    qn = torch.randn((E.n_layer, E.B, E.H, E.D), device=dev, dtype=torch.bfloat16, generator=g)
    kn = torch.randn((E.n_layer, E.B, E.H, E.D), device=dev, dtype=torch.bfloat16, generator=g)
    vn = torch.randn((E.n_layer, E.B, E.H, E.D), device=dev, dtype=torch.bfloat16, generator=g)
    on = torch.empty((E.B, E.H, E.D), device=dev, dtype=torch.bfloat16)
    qp = torch.randn((E.B, Tq, E.H, E.D), device=dev, dtype=torch.bfloat16, generator=g)
    op = torch.empty_like(qp)
    steps_tab = torch.arange(E.steps, dtype=torch.int32)[:, None]
    pos_tab = (lens0[None, :] + steps_tab).to(dev).contiguous()        # append row of step s
    len_tab = (lens0[None, :] + steps_tab + 1).to(dev).contiguous()    # keys after the append
    lens0_d = lens0.to(dev)
    ws_d = torch.empty(sw.attn_decode_workspace_bytes(E.B, E.H, E.Lcap, E.D), device=dev,
                       dtype=torch.uint8)

    def decode_bytes(s: int, nb: int = E.B) -> int:
        tot = 0
        for l in range(E.n_layer):
            w = E.window(l)
            for b in range(nb):
                L = int(lens0[b]) + s + 1
                tot += E.H * (min(L, w) if w else L) * E.D * 2 * 2
            tot += 2 * nb * E.H * E.D * 2  # q read, o written
        return tot

    def prefill_flops(layer: int) -> int:
        w = E.window(layer)
        return 4 * E.D * E.H * sum(pairs(int(L), w) for L in lens0)

    # ------------------------------------------------------------------ timed loop
    n_total = args.warmup + args.steps
    Ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev = [[Ev() for _ in range(7)] for _ in range(n_total)]
    win = case.window

    def step(i: int):
        e = ev[i]
        s = i % E.steps
        e[0].record()
        sw.attn_fwd(q, k, v, o=o, lse=lse, window=win)
        e[1].record()
        sw.attn_bwd_dq(q, k, v, o, lse, do, ws_b, window=win, dq=dq)
        e[2].record()
        sw.attn_bwd_dkdv(q, k, v, lse, do, ws_b, window=win, dk=dk, dv=dv)
        e[3].record()
        # the Engine step: every layer's KV append, then every layer's decode back to back (the
        # layers' caches are distinct, so the order is free), so that the decode events bracket
        # the 30 decode launches and no event falls between two of them
        for l in range(E.n_layer):
            sw.attn_kv_append(kcache[l], vcache[l], kn[l], vn[l], pos_tab[s])
        e[4].record()
        for l in range(E.n_layer):
            sw.attn_decode(qn[l], kcache[l], vcache[l], len_tab[s], o=on, window=E.window(l),
                           ws=ws_d)
        e[5].record()
        pl = i % E.n_layer
        sw.attn_prefill(qp, kcache[pl], vcache[pl], lens0_d, o=op, window=E.window(pl))
        e[6].record()

    log(f"warmup {args.warmup} steps ...")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps ...")
    t0 = time.perf_counter()
    for i in range(args.warmup, n_total):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log("timed region done")

    K = args.steps
    timed = range(args.warmup, n_total)
    t_fwd = sum(ev[i][0].elapsed_time(ev[i][1]) for i in timed) / K * 1e-3
    t_dq = sum(ev[i][1].elapsed_time(ev[i][2]) for i in timed) / K * 1e-3
    t_dkdv = sum(ev[i][2].elapsed_time(ev[i][3]) for i in timed) / K * 1e-3
    t_app = sum(ev[i][3].elapsed_time(ev[i][4]) for i in timed) / K * 1e-3
    t_dec = sum(ev[i][4].elapsed_time(ev[i][5]) for i in timed) / K * 1e-3
    t_pre = sum(ev[i][5].elapsed_time(ev[i][6]) for i in timed) / K * 1e-3
    dec_bytes = sum(decode_bytes(i % E.steps) for i in timed) / K
    pre_flops = sum(prefill_flops(i % E.n_layer) for i in timed) / K
    t_fb = t_fwd + t_dq + t_dkdv
    value = (F_fwd + F_dq + F_dkdv) / t_fb / 1e12

    kernels = {
        "fwd_bf16_kernel": (F_fwd, t_fwd),
        "bwd_dq_kernel": (F_dq, t_dq),
        "bwd_dkdv_kernel": (F_dkdv, t_dkdv),
    }
    dom = max(kernels, key=lambda n: kernels[n][1])
    f_dom, t_dom = kernels[dom]
    achieved = f_dom / t_dom / 1e12
    traffic = None
    src_hash = kernel_source_hash()
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        ent = tr.get("kernels", {}).get(dom)
        if ent and tr.get("source_hash") == src_hash:
            traffic = ent["hbm_bytes_per_launch"]
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_MFMA_BF16, "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_BF16, 4),
                "traffic": traffic, "avg_launch_us": round(t_dom * 1e6, 2),
                "algorithmic_flops_per_launch": f_dom}

    # plain copy kernel of known size (rocprofv3 counter calibration); outside the timed region
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # packed documents in the same d20 rows (each document attends only to itself; the sequence
    # offsets come from workloads.d20_packed_cu): the same q, k, v, dO viewed as [B*T, H, D],
    # forward + backward timed with events, outside the timed region
    varlen = None
    if not args.no_varlen:
        log("packed-document d20 rows: forward + backward ...")
        cu_h = W.d20_packed_cu(B, T)
        lens_d = (cu_h[1:] - cu_h[:-1]).tolist()
        ms = max(lens_d)
        cu_d = cu_h.to(dev)
        qv, kv, vv, dov = (t.view(B * T, H, D) for t in (q, k, v, do))
        ov = torch.empty_like(qv)
        lsev = torch.empty((H, B * T), device=dev, dtype=torch.float32)
        gv = [torch.empty_like(qv) for _ in range(3)]
        wsv = torch.empty(sw.attn_bwd_workspace_bytes(1, H, B * T, D), device=dev,
                          dtype=torch.uint8)
        reps = max(args.steps, 5)
        ev_v = [[Ev() for _ in range(3)] for _ in range(reps + 2)]
        for i in range(reps + 2):
            ev_v[i][0].record()
            sw.attn_fwd_varlen(qv, kv, vv, cu_d, ms, o=ov, lse=lsev, window=win)
            ev_v[i][1].record()
            sw.attn_bwd_varlen(qv, kv, vv, ov, lsev, dov, cu_d, ms, window=win, dq=gv[0], dk=gv[1],
                               dv=gv[2], ws=wsv)
            ev_v[i][2].record()
        torch.cuda.synchronize()
        tv_f = sum(e[0].elapsed_time(e[1]) for e in ev_v[2:]) / reps * 1e-3
        tv_b = sum(e[1].elapsed_time(e[2]) for e in ev_v[2:]) / reps * 1e-3
        pv = sum(pairs(L, win) for L in lens_d) * H
        varlen = {"TFLOP/s": round(14 * D * pv / (tv_f + tv_b) / 1e12, 2),
                  "fwd_ms": round(tv_f * 1e3, 4), "bwd_ms": round(tv_b * 1e3, 4),
                  "documents": len(lens_d), "max_seqlen": ms, "visible_pairs": pv,
                  "workload": "d20 rows B32 T2048 H10 D128 holding packed documents (log-normal "
                              "lengths, median 600, cut at row ends), same q, k, v, dO"}
        del ov, lsev, gv, wsv

    # QK-norm on the d20 layer: the same q, k, v, dO; forward = norm pass + attention on the
    # normalised rows, backward = both passes with the norm's backward in their epilogues
    qknorm = None
    if not args.no_qknorm:
        log("QK-norm d20 layer: forward + backward ...")
        reps = max(args.steps, 5)
        ev_q = [[Ev() for _ in range(3)] for _ in range(reps + 2)]
        gq = [torch.empty_like(q) for _ in range(3)]
        for i in range(reps + 2):
            ev_q[i][0].record()
            oq, lq, qn_, kn_, rq_, rk_ = sw.attn_fwd_qknorm(q, k, v, window=win)
            ev_q[i][1].record()
            sw.attn_bwd_qknorm(qn_, kn_, v, oq, lq, do, rq_, rk_, window=win, dq=gq[0], dk=gq[1],
                               dv=gq[2], ws=ws_b)
            ev_q[i][2].record()
        torch.cuda.synchronize()
        tq_f = sum(e[0].elapsed_time(e[1]) for e in ev_q[2:]) / reps * 1e-3
        tq_b = sum(e[1].elapsed_time(e[2]) for e in ev_q[2:]) / reps * 1e-3
        qknorm = {"TFLOP/s": round((F_fwd + F_dq + F_dkdv) / (tq_f + tq_b) / 1e12, 2),
                  "fwd_ms": round(tq_f * 1e3, 4), "bwd_ms": round(tq_b * 1e3, 4),
                  "note": "fwd includes the norm pass; FLOPs are the attention's only"}
        del gq, oq, lq, qn_, kn_, rq_, rk_

    # d26 alternating-window layers (B 16, T 2048, H 13, D 128; windows 512, full, 512, full):
    # layer 0 (w = 512) and layer 1 (full causal) of the same seeded stack, forward + backward,
    # timed with events outside the timed region.  Algorithmic bytes: every input read once, every
    # output written once.
    d26 = None
    if not args.no_d26:
        log("d26 layers (w = 512 and full): forward + backward ...")
        d26 = {}
        for layer in (0, 1):
            w26 = W.D26_WINDOWS[layer]
            q6, k6, v6, do6 = (t.to(dev) for t in W.d26_layer_inputs(layer))
            B6, T6, H6, D6 = q6.shape
            o6 = torch.empty_like(q6)
            lse6 = torch.empty((B6, H6, T6), device=dev, dtype=torch.float32)
            g6 = [torch.empty_like(q6) for _ in range(3)]
            ws6 = torch.empty(sw.attn_bwd_workspace_bytes(B6, H6, T6, D6), device=dev,
                              dtype=torch.uint8)
            reps = max(args.steps, 5)
            ev6 = [[Ev() for _ in range(3)] for _ in range(reps + 2)]
            for i in range(reps + 2):
                ev6[i][0].record()
                sw.attn_fwd(q6, k6, v6, o=o6, lse=lse6, window=w26)
                ev6[i][1].record()
                sw.attn_bwd(q6, k6, v6, o6, lse6, do6, window=w26, dq=g6[0], dk=g6[1], dv=g6[2],
                            ws=ws6)
                ev6[i][2].record()
            torch.cuda.synchronize()
            t6f = sum(e[0].elapsed_time(e[1]) for e in ev6[2:]) / reps * 1e-3
            t6b = sum(e[1].elapsed_time(e[2]) for e in ev6[2:]) / reps * 1e-3
            P6 = pairs(T6, w26) * B6 * H6
            nb, nst = q6.numel() * 2, B6 * H6 * T6 * 4
            d26[f"layer{layer}"] = {
                "window": w26, "TFLOP/s": round(14 * D6 * P6 / (t6f + t6b) / 1e12, 2),
                "fwd_ms": round(t6f * 1e3, 4), "bwd_ms": round(t6b * 1e3, 4),
                "fwd_GB/s": round((4 * nb + nst) / t6f / 1e9, 1),
                "bwd_GB/s": round((8 * nb + nst) / t6b / 1e9, 1)}
            del q6, k6, v6, do6, o6, lse6, g6, ws6
        d26["workload"] = ("d26 stack B16 T2048 H13 D128, seed 3: layer 0 (window 512) and "
                           "layer 1 (full causal), fwd + bwd")

    # the whole 30-layer decode step (append + decode per layer, one launch each) captured in one
    # HIP graph and replayed per token; timed per replay with events, outside the timed region
    step_graph = None
    if not args.no_step_graph:
        log("decode step graph: capture and replay ...")
        sg = sw.DecodeStepGraph(eng)
        sg.q.copy_(qn)
        sg.k_new.copy_(kn)
        sg.v_new.copy_(vn)
        reps = max(args.steps, 5)
        ev_g = [(Ev(), Ev()) for _ in range(reps + 2)]
        for i in range(reps + 2):
            eng.lens.copy_(pos_tab[i % E.steps])
            ev_g[i][0].record()
            sg.replay()
            ev_g[i][1].record()
        torch.cuda.synchronize()
        t_g = sum(a.elapsed_time(b) for a, b in ev_g[2:]) / reps * 1e-3
        g_bytes = sum(decode_bytes(i % E.steps) for i in range(2, reps + 2)) / reps
        step_graph = {"us_per_layer_step": round(t_g / E.n_layer * 1e6, 2),
                      "GB/s": round(g_bytes / t_g / 1e9, 1),
                      "frac_of_hbm_peak": round(g_bytes / t_g / 1e9 / PEAK_HBM, 4),
                      "us_per_token_all_layers": round(t_g * 1e6, 1), "replays": reps}
        del sg

    # Short decode calls take less GPU time than the host needs to launch them, so the two figures
    # below time whole passes of calls queued behind ~1 ms of unrelated GPU work (a bf16 matmul):
    # by the time the first call runs, the host has queued them all.
    busy = torch.randn((8192, 8192), device=dev, dtype=torch.bfloat16)

    def queued_pass_time(calls, reps):
        evs = [(Ev(), Ev()) for _ in range(reps + 2)]
        for i in range(reps + 2):
            torch.matmul(busy, busy)
            evs[i][0].record()
            for c in calls:
                c(i)
            evs[i][1].record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs[2:]) / reps * 1e-3

    # the two small training configurations (fp32 tiny forward, B 1 T 128 H 2 D 64 full causal;
    # bf16 small fwd + bwd, B 2 T 512 H 4 D 128 window 128), 50 back-to-back calls per pass:
    # launch-latency bound, reported for completeness
    small_cfg = None
    if not args.no_small_configs:
        log("small configurations (tiny fp32 forward, small bf16 fwd + bwd) ...")
        small_cfg = {}
        tc = W.TINY_F32
        qt_, kt_, vt_ = (t.to(dev) for t in W.attn_inputs(tc)[:3])
        ot_ = torch.empty_like(qt_)
        lt_ = torch.empty((tc.B, tc.H, tc.T), device=dev, dtype=torch.float32)
        n_rep = 50
        t_t = queued_pass_time([lambda i: sw.attn_fwd(qt_, kt_, vt_, o=ot_, lse=lt_, window=tc.window)]
                               * n_rep, 5) / n_rep
        small_cfg["tiny_fp32_fwd"] = {"us_per_call": round(t_t * 1e6, 2),
                                      "TFLOP/s": round(4 * tc.D * pairs(tc.T, tc.window) * tc.B
                                                       * tc.H / t_t / 1e12, 4)}
        sc_ = W.SMALL_W128
        qs_, ks_, vs_, dos_ = (t.to(dev) for t in W.attn_inputs(sc_))
        os_ = torch.empty_like(qs_)
        ls_ = torch.empty((sc_.B, sc_.H, sc_.T), device=dev, dtype=torch.float32)
        gs_ = [torch.empty_like(qs_) for _ in range(3)]
        wss_ = torch.empty(sw.attn_bwd_workspace_bytes(sc_.B, sc_.H, sc_.T, sc_.D), device=dev,
                           dtype=torch.uint8)
        t_sf = queued_pass_time([lambda i: sw.attn_fwd(qs_, ks_, vs_, o=os_, lse=ls_,
                                                       window=sc_.window)] * n_rep, 5) / n_rep
        t_sb = queued_pass_time([lambda i: sw.attn_bwd(qs_, ks_, vs_, os_, ls_, dos_,
                                                       window=sc_.window, dq=gs_[0], dk=gs_[1],
                                                       dv=gs_[2], ws=wss_)] * n_rep, 5) / n_rep
        ps_ = pairs(sc_.T, sc_.window) * sc_.B * sc_.H
        small_cfg["small_bf16_w128"] = {"fwd_us": round(t_sf * 1e6, 2), "bwd_us": round(t_sb * 1e6, 2),
                                        "TFLOP/s": round(14 * sc_.D * ps_ / (t_sf + t_sb) / 1e12, 3)}

    # small-batch decode: the first 8 sequences of the same Engine caches, all 30 layers, outside
    # the timed region
    small = None
    if not args.no_small_batch:
        Bs = 8
        log(f"small-batch decode (first {Bs} sequences) ...")
        reps = max(args.steps, 5)
        on_s = on[:Bs]
        qs = [qn[l][:Bs] for l in range(E.n_layer)]
        ks = [kcache[l][:Bs] for l in range(E.n_layer)]
        vs = [vcache[l][:Bs] for l in range(E.n_layer)]
        lens_s = len_tab[0][:Bs]

        def small_call(l):
            return lambda i: sw.attn_decode(qs[l], ks[l], vs[l], lens_s, o=on_s,
                                            window=E.window(l), ws=ws_d)

        t_s = queued_pass_time([small_call(l) for l in range(E.n_layer)], reps)
        s_bytes = decode_bytes(0, Bs)
        small = {"B": Bs, "launches": sw.attn_decode_launches(Bs, E.H, E.Lcap, E.D),
                 "us_per_layer_step": round(t_s / E.n_layer * 1e6, 2),
                 "GB/s": round(s_bytes / t_s / 1e9, 1),
                 "frac_of_hbm_peak": round(s_bytes / t_s / 1e9 / PEAK_HBM, 4)}

    # long-context decode: 2 sequences x 15 heads, each attending to all of its 16384 cached rows,
    # four layers' caches in rotation (1 GB, beyond the last-level cache).  With 30 (sequence, head)
    # pairs each reading more than 2048 rows, the decode splits every pair's keys across
    # workgroups and merges the chunks in a second kernel; outside the timed region
    longctx = None
    if not args.no_long_context:
        Bl, Ll, nll = 2, 16384, 4
        log(f"long-context decode ({Bl} sequences x {Ll} rows) ...")
        gl = torch.Generator(device=dev).manual_seed(E.seed + 1)
        kl = [torch.randn((Bl, Ll, E.H, E.D), device=dev, dtype=torch.bfloat16, generator=gl)
              for _ in range(nll)]
        vl = [torch.randn((Bl, Ll, E.H, E.D), device=dev, dtype=torch.bfloat16, generator=gl)
              for _ in range(nll)]
        ql = torch.randn((Bl, E.H, E.D), device=dev, dtype=torch.bfloat16, generator=gl)
        ol = torch.empty_like(ql)
        lens_l = torch.full((Bl,), Ll, dtype=torch.int32, device=dev)
        ws_l = torch.empty(sw.attn_decode_workspace_bytes(Bl, E.H, Ll, E.D), device=dev,
                           dtype=torch.uint8)

        def long_call(l):
            return lambda i: sw.attn_decode(ql, kl[l], vl[l], lens_l, o=ol, ws=ws_l)

        t_l = queued_pass_time([long_call(l) for l in range(nll)], max(args.steps, 5)) / nll
        l_bytes = Bl * E.H * Ll * E.D * 2 * 2 + 2 * Bl * E.H * E.D * 2
        longctx = {"B": Bl, "H": E.H, "L": Ll, "launches": sw.attn_decode_launches(Bl, E.H, Ll, E.D),
                   "us_per_call": round(t_l * 1e6, 2), "GB/s": round(l_bytes / t_l / 1e9, 1),
                   "frac_of_hbm_peak": round(l_bytes / t_l / 1e9 / PEAK_HBM, 4)}
        del kl, vl, ql, ol, ws_l
    del busy

    # streaming-read reference: a plain read of the decode step's byte count, rotating over the
    # 30 layers' key caches (each larger than the last-level cache), outside the timed region
    stream_ref = None
    if not args.no_stream_ref:
        stream_ref = stream_read_gbs(kcache, int(dec_bytes / E.n_layer))

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_heads} heads ...")
        cpu = cpu_baseline(case, q_c, k_c, v_c, do_c, args.cpu_heads)

    dec_gbs = dec_bytes / t_dec / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "d20 training layer B32 T2048 H10 D128 bf16 full causal fwd+bwd; d30 "
                        "Engine B64 H15 D128 Lcap2048 prompts U[32,1024], 30 layers, window "
                        "1024 on odd layers: one decode step + one prefill layer per step",
            "B": B, "T": T, "H": H, "D": D, "window": None,
        },
        "frac_of_peak": round(value / PEAK_MFMA_BF16, 4),
        "fwd": {"TFLOP/s": round(F_fwd / t_fwd / 1e12, 2), "ms": round(t_fwd * 1e3, 4)},
        "bwd": {"TFLOP/s": round((F_dq + F_dkdv) / (t_dq + t_dkdv) / 1e12, 2),
                "ms_dq": round(t_dq * 1e3, 4), "ms_dkdv": round(t_dkdv * 1e3, 4)},
        "decode": {"GB/s": round(dec_gbs, 1), "frac_of_hbm_peak": round(dec_gbs / PEAK_HBM, 4),
                   "us_per_layer_step": round(t_dec / E.n_layer * 1e6, 2),
                   "append_us_per_layer": round(t_app / E.n_layer * 1e6, 2),
                   "bytes_per_layer_step": round(dec_bytes / E.n_layer),
                   "stream_read_ref_GB/s": stream_ref and round(stream_ref, 1),
                   "frac_of_stream_read_ref": stream_ref and round(dec_gbs / stream_ref, 4),
                   "step_graph": step_graph, "small_batch": small,
                   "long_context": longctx},
        "prefill": {"TFLOP/s": round(pre_flops / t_pre / 1e12, 2), "ms_per_layer": round(t_pre * 1e3, 4)},
        "d26": d26,
        "small_configs": small_cfg,
        "varlen": varlen,
        "qknorm": qknorm,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "device": props.name,
        "kernel_source_hash": src_hash,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
