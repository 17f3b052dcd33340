#!/usr/bin/env python3
"""Benchmark of the windowed causal attention hot path on one MI355X.

One step is one pass over every part of the path, on synthetic data of the pages' shapes:
  * the d20 training layer (B=32, T=2048, H=10, D=128, bf16, full causal): forward and backward
    (each backward entry point timed on its own);
  * one Engine decode step of the d30-style model (30 layers, B=64, H=15, D=128, cache 2048,
    prompts U[32,1024], window 1024 on odd layers): every layer's KV append, then every
    layer's decode, the 30 decodes between one pair of events;
  * one Engine prefill layer (the same prompts, layer step % 30).

Timing protocol: every part of a step is bracketed by HIP events on the stream the kernels run on,
and a 512 MiB scratch buffer is written, then another 512 MiB read, just before each part (outside
its events), so that no part finds its inputs in the 4 MB L2s or the 256 MB last-level cache, nor
pays for writing back lines the flush left dirty.  Each figure is the median over the
timed steps (the minimum and mean are reported next to it).  The GPU's clocks and power are sampled
with amd-smi after the timed region, while the d20 passes run back to back for a few seconds (one
amd-smi call takes longer than the timed region).

The headline ``value`` is the d20 fwd+bwd rate in TFLOP/s counting unmasked FLOPs only (4D per
visible (query, key) pair forward, 10D backward), from the median times.  ``decode`` reports
algorithmic HBM GB/s (every visible cache row read once, plus q and o), next to a plain streaming
read of the same byte count; ``decode.reading_b`` the same decode over cache lengths drawn
uniformly from 1..2048 (where the 1024 window bites); ``decode.step_graph`` the whole 30-layer
decode step as one HIP-graph replay; ``decode.small_batch`` and ``decode.long_context`` two more
batch shapes; ``prefill`` TFLOP/s; ``varlen`` the d20 rows as packed documents; ``qknorm`` the
d20 layer with RMS-normalised q and k; ``d26`` the alternating-window d26 layers; ``small_configs``
the tiny fp32 forward and the small bf16 fwd + bwd.  ``roofline`` describes the longest-running MFMA
kernel, ``roofline_decode`` the decode kernel; ``cpu_baseline`` times the fp64 oracle on the same
d20 inputs on the host cores.  One JSON line goes to stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd+bwd TFLOP/s (unmasked FLOPs) & % bf16 MFMA peak; decode HBM GB/s"
PEAK_MFMA_BF16 = 2500.0  # TFLOP/s, MI355X dense bf16 (published)
PEAK_HBM = 8000.0        # GB/s, MI355X HBM3E (published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
FLUSH_BYTES = 512 << 20  # > 256 MB last-level cache + 8 x 4 MB L2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pairs(T: int, w) -> int:
    """Visible (query, key) pairs of one causal head with window w (None = full)."""
    w = T if w is None else min(int(w), T)
    return w * (w + 1) // 2 + (T - w) * w


def kernel_source_hash() -> str:
    """Hash of the sources libswattn.so is built from (the HBM-traffic figures recorded in
    profiles/ stand for these sources only)."""
    from causal_sliding_window_attn_amd import build as bld

    h = hashlib.sha256()
    files = [os.path.join(bld.CSRC, s) for s in bld.SOURCES]
    files += [os.path.join(bld.CSRC, s) for s in bld.HEADERS]
    files.append(os.path.join(ROOT, "include", "swattn.h"))
    for f in sorted(files):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def stats_us(xs):
    """Median, minimum and mean of a list of seconds, in microseconds."""
    return {"median_us": round(statistics.median(xs) * 1e6, 2), "min_us": round(min(xs) * 1e6, 2),
            "mean_us": round(sum(xs) / len(xs) * 1e6, 2), "n": len(xs)}


# ------------------------------------------------------------------------------ clocks and power
class SmiSampler:
    """Samples the GPU's clocks and power with amd-smi in a background thread."""

    def __init__(self):
        self.samples, self.errors = [], []
        self._stop = threading.Event()
        self._t = None

    @staticmethod
    def _numbers(obj, path=""):
        if isinstance(obj, dict):
            for k, v in obj.items():
                yield from SmiSampler._numbers(v, f"{path}/{k}")
        elif isinstance(obj, list):
            for i, v in enumerate(obj):
                yield from SmiSampler._numbers(v, f"{path}/{i}")
        else:
            try:
                yield path.lower(), float(obj)
            except (TypeError, ValueError):
                pass

    def _once(self):
        try:
            r = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--power", "--json"],
                               capture_output=True, text=True, timeout=10)
            if r.returncode != 0:
                self.errors.append(r.stderr.strip()[-200:])
                return
            s = r.stdout[r.stdout.find("[") if r.stdout.lstrip().startswith("[") else
                         r.stdout.find("{"):]
            data = json.loads(s)
            # gpu_data/0/clock/gfx_<n>/clk/value (MHz, one per XCD) and
            # gpu_data/0/power/socket_power/value (W)
            gfx, power = [], []
            for path, val in self._numbers(data):
                if re.search(r"/clock/gfx_\d+/clk/value$", path):
                    gfx.append(val)
                elif re.search(r"/power/socket_power/value$", path):
                    power.append(val)
            self.samples.append({"gfx_mhz": max(gfx) if gfx else None,
                                 "power_w": max(power) if power else None})
        except Exception as e:  # noqa: BLE001 -- a missing tool must not stop the measurement
            self.errors.append(repr(e)[-200:])

    def _run(self):
        while not self._stop.is_set():
            self._once()
            self._stop.wait(0.05)

    def start(self):
        self._t = threading.Thread(target=self._run, daemon=True)
        self._t.start()

    def stop(self):
        self._stop.set()
        if self._t is not None:
            self._t.join(timeout=15)
        g = [s["gfx_mhz"] for s in self.samples if s["gfx_mhz"] is not None]
        p = [s["power_w"] for s in self.samples if s["power_w"] is not None]
        out = {"tool": "amd-smi metric -g 0 --clock --power --json", "samples": len(self.samples)}
        if g:
            out["gfx_clock_mhz"] = {"median": statistics.median(g), "min": min(g), "max": max(g)}
        if p:
            out["power_w"] = {"median": statistics.median(p), "min": min(p), "max": max(p)}
        if not self.samples and self.errors:
            out["error"] = self.errors[-1]
        return out


# ------------------------------------------------------------------------------ cpu baseline
def host_info():
    import numpy as np

    info = {"affinity_cpus": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count()}
    try:
        model = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                 if l.startswith("model name")]
        info["cpu_model"] = model[0] if model else None
    except OSError:
        info["cpu_model"] = None
    try:
        deps = np.show_config(mode="dicts").get("Build Dependencies", {})
        blas = deps.get("blas", {})
        info["numpy_blas"] = (f"{blas.get('name')} {blas.get('version')} "
                              f"({blas.get('openblas configuration', '').strip()})")
    except Exception as e:  # noqa: BLE001
        info["numpy_blas"] = f"unknown ({e!r})"
    return info


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
    host = host_info()
    threads = min(16, host["affinity_cpus"])
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
                  f"wall on {threads} worker threads (one single-threaded BLAS call each)",
        "host": host,
    }


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


def decode_pattern_gbs(kcs, vcs, lens_h, windows, H, D, reps: int = 3) -> dict:
    """GB/s of two plain reads (libswattn_probe.so) of exactly the cache rows a decode over these
    lengths reads, one layer's caches per call: in the decode's own order (per (sequence, head)
    256-byte pieces) and as whole rows (all heads of 32-row chunks)."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "causal_sliding_window_attn_amd", "libswattn_probe.so"))
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.swattn_decode_pattern_read.argtypes = [i, vp, vp, vp, vp, i, i, i, i, i, i, vp, vp]
    lib.swattn_decode_pattern_read.restype = ctypes.c_int
    dev = kcs[0].device
    B, Lcap = kcs[0].shape[0], kcs[0].shape[1]
    lens_d = lens_h.to(torch.int32).to(dev)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    plans, nbytes = [], 0
    for w in windows:
        vis = [min(int(L), w) for L in lens_h]
        nbytes += sum(vis) * H * D * 2 * 2
        cs = [0]
        for x in vis:
            cs.append(cs[-1] + (x + 31) // 32)
        plans.append((torch.tensor(cs, dtype=torch.int32, device=dev), cs[-1]))
    out = torch.empty(max(B * H, max(n for _, n in plans)) * 512, dtype=torch.int32, device=dev)
    res = {}
    for pat, name in ((0, "pieces"), (1, "rows")):
        def run():
            for l, w in enumerate(windows):
                cs_d, n = plans[l]
                rc = lib.swattn_decode_pattern_read(pat, kcs[l].data_ptr(), vcs[l].data_ptr(),
                                                    lens_d.data_ptr(), cs_d.data_ptr(), n, B, H,
                                                    Lcap, D, w, out.data_ptr(), st)
                if rc != 0:
                    raise RuntimeError(f"swattn_decode_pattern_read failed ({rc})")

        run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        res[f"{name}_GB/s"] = round(nbytes / (e0.elapsed_time(e1) * 1e-3 / reps) / 1e9, 1)
    res["cache_bytes_per_layer_step"] = nbytes // len(windows)
    res["note"] = ("plain nontemporal reads of the cache rows this decode reads, no arithmetic: "
                   "'pieces' in the decode's order (per sequence and head, four rows' 256-byte "
                   "pieces per load instruction), 'rows' as whole rows (all heads of 32-row "
                   "chunks, consecutive threads on consecutive bytes)")
    return res


def traffic_entry(key: str, src_hash: str):
    """HBM bytes per launch recorded in profiles/traffic.json for one (kernel, launch grid) entry,
    or None when absent or recorded for other kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    tr = json.load(open(TRAFFIC_FILE))
    if tr.get("source_hash") != src_hash:
        return None
    return tr.get("entries", {}).get(key)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-heads", type=int, default=320)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the 512 MiB cache flush before each timed part")
    ap.add_argument("--no-smi", action="store_true", help="do not sample clocks with amd-smi")
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
    ap.add_argument("--no-reading-b", action="store_true",
                    help="skip the decode over cache lengths U[1, 2048]")
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

    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    scratch_rd = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)  # read by a sum
    flush_n = [0]

    def flush():
        """Write 512 MiB, then read another 512 MiB, so that the next part starts with cold L2 and
        last-level caches holding no dirty lines (left dirty by the write alone, their write-back
        would be charged to the next part: measured ~45 us on the row-sized passes)."""
        if not args.no_flush:
            flush_n[0] += 1
            scratch.fill_(flush_n[0] & 0xFF)
            scratch_rd.sum()

    Ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed_parts(parts, reps, warm=2):
        """Runs the named parts `warm + reps` times, each preceded by a flush and bracketed by its
        own events; returns {name: [seconds per rep]} over the last reps."""
        evs = [[(Ev(), Ev()) for _ in parts] for _ in range(warm + reps)]
        for i in range(warm + reps):
            for j, (_, fn) in enumerate(parts):
                flush()
                evs[i][j][0].record()
                fn(i)
                evs[i][j][1].record()
        torch.cuda.synchronize()
        return {name: [evs[i][j][0].elapsed_time(evs[i][j][1]) * 1e-3
                       for i in range(warm, warm + reps)]
                for j, (name, _) in enumerate(parts)}

    med = statistics.median

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
    F_bwd = 10 * D * P20
    win = case.window

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

    def decode_bytes_for(lens_list, nb: int = E.B) -> int:
        tot = 0
        for l in range(E.n_layer):
            w = E.window(l)
            for b in range(nb):
                L = int(lens_list[b])
                tot += E.H * (min(L, w) if w else L) * E.D * 2 * 2
            tot += 2 * nb * E.H * E.D * 2  # q read, o written
        return tot

    def decode_bytes(s: int, nb: int = E.B) -> int:
        return decode_bytes_for([int(lens0[b]) + s + 1 for b in range(nb)], nb)

    def prefill_flops(layer: int) -> int:
        w = E.window(layer)
        return 4 * E.D * E.H * sum(pairs(int(L), w) for L in lens0)

    # ------------------------------------------------------------------ timed loop
    n_total = args.warmup + args.steps
    part_names = ["fwd", "bwd_dq", "bwd_dkdv", "append", "decode", "prefill"]
    ev = [[(Ev(), Ev()) for _ in part_names] for _ in range(n_total)]

    def step(i: int):
        e = ev[i]
        s = i % E.steps

        def part(j, fn):
            flush()
            e[j][0].record()
            fn()
            e[j][1].record()

        part(0, lambda: sw.attn_fwd(q, k, v, o=o, lse=lse, window=win))
        part(1, lambda: sw.attn_bwd_dq(q, k, v, o, lse, do, ws_b, window=win, dq=dq))
        part(2, lambda: sw.attn_bwd_dkdv(q, k, v, lse, do, ws_b, window=win, dk=dk, dv=dv))

        # the Engine step: every layer's KV append, then every layer's decode back to back (the
        # layers' caches are distinct, so the order is free), so that the decode events bracket
        # the 30 decode launches and no event falls between two of them
        def appends():
            for l in range(E.n_layer):
                sw.attn_kv_append(kcache[l], vcache[l], kn[l], vn[l], pos_tab[s])

        def decodes():
            for l in range(E.n_layer):
                sw.attn_decode(qn[l], kcache[l], vcache[l], len_tab[s], o=on, window=E.window(l),
                               ws=ws_d)

        part(3, appends)
        part(4, decodes)
        pl = i % E.n_layer
        part(5, lambda: sw.attn_prefill(qp, kcache[pl], vcache[pl], lens0_d, o=op,
                                        window=E.window(pl)))

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

    # clocks and power under the same load: amd-smi reports the current clock, and one call takes
    # longer than the timed region, so the d20 layer's passes run back to back for a few seconds
    # while it samples (outside the timed region)
    clocks = None
    if not args.no_smi:
        log("sampling clocks and power under load ...")
        smi = SmiSampler()
        smi.start()
        t_end = time.perf_counter() + 4.0
        while time.perf_counter() < t_end:
            for _ in range(20):
                sw.attn_fwd(q, k, v, o=o, lse=lse, window=win)
                sw.attn_bwd(q, k, v, o, lse, do, window=win, dq=dq, dk=dk, dv=dv, ws=ws_b)
            torch.cuda.synchronize()
        clocks = smi.stop()
        clocks["load"] = "d20 layer fwd + bwd back to back"

    K = args.steps
    timed = list(range(args.warmup, n_total))
    per = {name: [ev[i][j][0].elapsed_time(ev[i][j][1]) * 1e-3 for i in timed]
           for j, name in enumerate(part_names)}
    t_fwd, t_dq, t_dkdv = med(per["fwd"]), med(per["bwd_dq"]), med(per["bwd_dkdv"])
    t_app, t_dec, t_pre = med(per["append"]), med(per["decode"]), med(per["prefill"])
    dec_bytes_s = [decode_bytes(i % E.steps) for i in timed]
    dec_gbs_s = [b / t / 1e9 for b, t in zip(dec_bytes_s, per["decode"])]
    dec_bytes = sum(dec_bytes_s) / K
    pre_flops_s = [prefill_flops(i % E.n_layer) for i in timed]
    pre_tf_s = [f / t / 1e12 for f, t in zip(pre_flops_s, per["prefill"])]
    t_fb = t_fwd + t_dq + t_dkdv
    value = (F_fwd + F_bwd) / t_fb / 1e12
    fb_min = min(a + b + c for a, b, c in zip(per["fwd"], per["bwd_dq"], per["bwd_dkdv"]))
    src_hash = kernel_source_hash()

    # the longest-running MFMA kernel of the d20 layer, with the FLOPs the algorithm credits it
    # (each backward entry point launches one kernel on this workload)
    F_dq_credit, F_dkdv_credit = 2 * D * P20, 8 * D * P20
    kernels = {
        "fwd_bf16_kernel": ("d20 forward", F_fwd, t_fwd),
        "bwd_dq_kernel": ("d20 dQ pass", F_dq_credit, t_dq),
        "bwd_dkdv_chain_kernel": ("d20 dK/dV pass", F_dkdv_credit, t_dkdv),
    }
    dom = max(kernels, key=lambda n: kernels[n][2])
    dom_label, f_dom, t_dom = kernels[dom]
    achieved = f_dom / t_dom / 1e12
    tr_dom = traffic_entry(dom_label, src_hash)
    roofline = {"bound": "mfma", "kernel": dom, "workload": dom_label,
                "achieved": round(achieved, 2), "peak": PEAK_MFMA_BF16, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_MFMA_BF16, 4),
                "traffic": tr_dom and tr_dom["hbm_bytes_per_launch"],
                "traffic_grid": tr_dom and tr_dom["grid"],
                "avg_launch_us": round(t_dom * 1e6, 2),
                "algorithmic_flops_per_launch": f_dom,
                "algorithmic_flops_per_pair": f_dom // P20, "pairs_per_launch": P20}
    dec_achieved = dec_bytes / E.n_layer / (t_dec / E.n_layer) / 1e9
    tr_dec = traffic_entry("d30 decode", src_hash)
    roofline_decode = {"bound": "hbm", "kernel": "decode_fused_kernel", "workload": "d30 decode",
                       "achieved": round(dec_achieved, 1), "peak": PEAK_HBM, "unit": "GB/s",
                       "frac": round(dec_achieved / PEAK_HBM, 4),
                       "traffic": tr_dec and tr_dec["hbm_bytes_per_launch"],
                       "traffic_grid": tr_dec and tr_dec["grid"],
                       "avg_launch_us": round(t_dec / E.n_layer * 1e6, 2),
                       "algorithmic_bytes_per_launch": round(dec_bytes / E.n_layer)}

    # plain copy kernel of known size (rocprofv3 counter calibration); outside the timed region
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    reps = max(args.steps, 5)

    # packed documents in the same d20 rows (each document attends only to itself; the sequence
    # offsets come from workloads.d20_packed_cu): the same q, k, v, dO viewed as [B*T, H, D]
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
        tv = timed_parts([
            ("fwd", lambda i: sw.attn_fwd_varlen(qv, kv, vv, cu_d, ms, o=ov, lse=lsev, window=win)),
            ("bwd", lambda i: sw.attn_bwd_varlen(qv, kv, vv, ov, lsev, dov, cu_d, ms, window=win,
                                                 dq=gv[0], dk=gv[1], dv=gv[2], ws=wsv))], reps)
        tv_f, tv_b = med(tv["fwd"]), med(tv["bwd"])
        pv = sum(pairs(L, win) for L in lens_d) * H
        varlen = {"TFLOP/s": round(14 * D * pv / (tv_f + tv_b) / 1e12, 2),
                  "fwd_ms": round(tv_f * 1e3, 4), "bwd_ms": round(tv_b * 1e3, 4),
                  "documents": len(lens_d), "max_seqlen": ms, "visible_pairs": pv,
                  "workload": "d20 rows B32 T2048 H10 D128 holding packed documents (log-normal "
                              "lengths, median 600, cut at row ends), same q, k, v, dO"}
        del ov, lsev, gv, wsv

    # QK-norm on the d20 layer: the same q, k, v, dO; forward = norm + attention on the
    # normalised rows, backward = both passes with the norm's backward in their epilogues
    qknorm = None
    if not args.no_qknorm:
        log("QK-norm d20 layer: forward + backward ...")
        gq = [torch.empty_like(q) for _ in range(3)]
        fq = {}

        def qk_fwd(i):
            fq["r"] = sw.attn_fwd_qknorm(q, k, v, window=win)

        def qk_bwd(i):
            oq, lq, qn_, kn_, rq_, rk_ = fq["r"]
            sw.attn_bwd_qknorm(qn_, kn_, v, oq, lq, do, rq_, rk_, window=win, dq=gq[0], dk=gq[1],
                               dv=gq[2], ws=ws_b)

        tq = timed_parts([("fwd", qk_fwd), ("bwd", qk_bwd)], reps)
        tq_f, tq_b = med(tq["fwd"]), med(tq["bwd"])
        qknorm = {"TFLOP/s": round((F_fwd + F_bwd) / (tq_f + tq_b) / 1e12, 2),
                  "fwd_ms": round(tq_f * 1e3, 4), "bwd_ms": round(tq_b * 1e3, 4),
                  "overhead_vs_plain_ms": round((tq_f + tq_b - t_fb) * 1e3, 4),
                  "note": "fwd includes the norm of q and k; FLOPs are the attention's only"}
        del gq, fq

    # d26 alternating-window layers (B 16, T 2048, H 13, D 128; windows 512, full, 512, full):
    # layer 0 (w = 512) and layer 1 (full causal) of the same seeded stack, forward + backward.
    # Algorithmic bytes: every input read once, every output written once.
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
            t6 = timed_parts([
                ("fwd", lambda i: sw.attn_fwd(q6, k6, v6, o=o6, lse=lse6, window=w26)),
                ("bwd", lambda i: sw.attn_bwd(q6, k6, v6, o6, lse6, do6, window=w26, dq=g6[0],
                                              dk=g6[1], dv=g6[2], ws=ws6))], reps)
            t6f, t6b = med(t6["fwd"]), med(t6["bwd"])
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
    # HIP graph and replayed per token
    step_graph = None
    if not args.no_step_graph:
        log("decode step graph: capture and replay ...")
        sg = sw.DecodeStepGraph(eng)
        sg.q.copy_(qn)
        sg.k_new.copy_(kn)
        sg.v_new.copy_(vn)
        lmax0 = int(lens0.max())
        tg = timed_parts([("replay", lambda i: (
            eng.set_lens(pos_tab[i % E.steps], max_len=lmax0 + i % E.steps), sg.replay()))], reps)
        t_g = med(tg["replay"])
        g_bytes = sum(decode_bytes(i % E.steps) for i in range(2, reps + 2)) / reps
        step_graph = {"us_per_layer_step": round(t_g / E.n_layer * 1e6, 2),
                      "GB/s": round(g_bytes / t_g / 1e9, 1),
                      "frac_of_hbm_peak": round(g_bytes / t_g / 1e9 / PEAK_HBM, 4),
                      "us_per_token_all_layers": round(t_g * 1e6, 1), "replays": reps,
                      "note": "includes the lens reset copy before each replay"}
        del sg

    # decode over cache lengths drawn uniformly from 1..2048 (the 1024 window of the odd layers
    # then limits most rows), same caches and queries, all 30 layers
    reading_b = None
    if not args.no_reading_b:
        log("decode over cache lengths U[1, 2048] ...")
        gb = torch.Generator("cpu").manual_seed(E.seed + 2)
        lens_b = torch.randint(1, E.Lcap + 1, (E.B,), generator=gb, dtype=torch.int32)
        lens_bd = lens_b.to(dev)

        def decodes_b(i):
            for l in range(E.n_layer):
                sw.attn_decode(qn[l], kcache[l], vcache[l], lens_bd, o=on, window=E.window(l),
                               ws=ws_d)

        tb = timed_parts([("decode", decodes_b)], reps)
        t_b = med(tb["decode"])
        b_bytes = decode_bytes_for(lens_b.tolist())
        reading_b = {"us_per_layer_step": round(t_b / E.n_layer * 1e6, 2),
                     "GB/s": round(b_bytes / t_b / 1e9, 1),
                     "frac_of_hbm_peak": round(b_bytes / t_b / 1e9 / PEAK_HBM, 4),
                     "bytes_per_layer_step": round(b_bytes / E.n_layer),
                     "lens": "U[1, 2048], seed 6, the Engine's 64 sequences"}

    # Short calls take less GPU time than the host needs to launch them, so the figures below time
    # whole passes of calls queued behind ~1 ms of unrelated GPU work (a bf16 matmul): by the time
    # the first call runs, the host has queued them all.
    busy = torch.randn((8192, 8192), device=dev, dtype=torch.bfloat16)

    def queued_pass_times(calls, n):
        evs = [(Ev(), Ev()) for _ in range(n + 2)]
        for i in range(n + 2):
            flush()
            torch.matmul(busy, busy)
            evs[i][0].record()
            for c in calls:
                c(i)
            evs[i][1].record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e-3 for a, b in evs[2:]]

    small_cfg = None
    if not args.no_small_configs:
        log("small configurations (tiny fp32 forward, small bf16 fwd + bwd) ...")
        small_cfg = {}
        tc = W.TINY_F32
        qt_, kt_, vt_ = (t.to(dev) for t in W.attn_inputs(tc)[:3])
        ot_ = torch.empty_like(qt_)
        lt_ = torch.empty((tc.B, tc.H, tc.T), device=dev, dtype=torch.float32)
        n_rep = 50
        t_t = med(queued_pass_times(
            [lambda i: sw.attn_fwd(qt_, kt_, vt_, o=ot_, lse=lt_, window=tc.window)] * n_rep,
            5)) / n_rep
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
        t_sf = med(queued_pass_times([lambda i: sw.attn_fwd(qs_, ks_, vs_, o=os_, lse=ls_,
                                                            window=sc_.window)] * n_rep, 5)) / n_rep
        t_sb = med(queued_pass_times([lambda i: sw.attn_bwd(qs_, ks_, vs_, os_, ls_, dos_,
                                                            window=sc_.window, dq=gs_[0], dk=gs_[1],
                                                            dv=gs_[2], ws=wss_)] * n_rep, 5)) / n_rep
        ps_ = pairs(sc_.T, sc_.window) * sc_.B * sc_.H
        small_cfg["small_bf16_w128"] = {"fwd_us": round(t_sf * 1e6, 2), "bwd_us": round(t_sb * 1e6, 2),
                                        "TFLOP/s": round(14 * sc_.D * ps_ / (t_sf + t_sb) / 1e12, 3)}

    small = None
    if not args.no_small_batch:
        Bs = 8
        log(f"small-batch decode (first {Bs} sequences) ...")
        on_s = on[:Bs]
        qs = [qn[l][:Bs] for l in range(E.n_layer)]
        ks = [kcache[l][:Bs] for l in range(E.n_layer)]
        vs = [vcache[l][:Bs] for l in range(E.n_layer)]
        lens_s = len_tab[0][:Bs]

        def small_call(l):
            return lambda i: sw.attn_decode(qs[l], ks[l], vs[l], lens_s, o=on_s,
                                            window=E.window(l), ws=ws_d)

        t_s = med(queued_pass_times([small_call(l) for l in range(E.n_layer)], reps))
        s_bytes = decode_bytes(0, Bs)
        small = {"B": Bs, "launches": sw.attn_decode_launches(Bs, E.H, E.Lcap, E.D),
                 "us_per_layer_step": round(t_s / E.n_layer * 1e6, 2),
                 "GB/s": round(s_bytes / t_s / 1e9, 1),
                 "frac_of_hbm_peak": round(s_bytes / t_s / 1e9 / PEAK_HBM, 4)}

    # long-context decode: 2 sequences x 15 heads, each attending to all of its 16384 cached rows,
    # four layers' caches in rotation; the decode splits every pair's keys across workgroups and
    # merges the chunks in a second kernel
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

        t_l = med(queued_pass_times([long_call(l) for l in range(nll)], reps)) / nll
        l_bytes = Bl * E.H * Ll * E.D * 2 * 2 + 2 * Bl * E.H * E.D * 2
        longctx = {"B": Bl, "H": E.H, "L": Ll, "launches": sw.attn_decode_launches(Bl, E.H, Ll, E.D),
                   "us_per_call": round(t_l * 1e6, 2), "GB/s": round(l_bytes / t_l / 1e9, 1),
                   "frac_of_hbm_peak": round(l_bytes / t_l / 1e9 / PEAK_HBM, 4)}
        del kl, vl, ql, ol, ws_l
    del busy

    # streaming-read reference: a plain read of the decode step's byte count, rotating over the
    # 30 layers' key caches (each larger than the last-level cache)
    stream_ref = pattern_ref = None
    if not args.no_stream_ref:
        stream_ref = stream_read_gbs(kcache, int(dec_bytes / E.n_layer))
        # the decode step timed above: lens0 + 1 rows per sequence
        pattern_ref = decode_pattern_gbs(kcache, vcache, lens0 + 1,
                                         [E.window(l) or E.Lcap for l in range(E.n_layer)],
                                         E.H, E.D)

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
        "timing": ("median over the timed steps of HIP-event intervals per part, each part "
                   "preceded by a 512 MiB scratch write and a 512 MiB read" if not args.no_flush else
                   "median over the timed steps of HIP-event intervals per part, no flush"),
        "frac_of_peak": round(value / PEAK_MFMA_BF16, 4),
        "value_from_min": round((F_fwd + F_bwd) / fb_min / 1e12, 3),
        "fwd": {"TFLOP/s": round(F_fwd / t_fwd / 1e12, 2), "ms": round(t_fwd * 1e3, 4),
                **stats_us(per["fwd"])},
        "bwd": {"TFLOP/s": round(F_bwd / (t_dq + t_dkdv) / 1e12, 2),
                "ms_dq": round(t_dq * 1e3, 4), "ms_dkdv": round(t_dkdv * 1e3, 4),
                "dq": stats_us(per["bwd_dq"]), "dkdv": stats_us(per["bwd_dkdv"])},
        "decode": {"GB/s": round(dec_gbs, 1), "frac_of_hbm_peak": round(dec_gbs / PEAK_HBM, 4),
                   "GB/s_min_max": [round(min(dec_gbs_s), 1), round(max(dec_gbs_s), 1)],
                   "us_per_layer_step": round(t_dec / E.n_layer * 1e6, 2),
                   "append_us_per_layer": round(t_app / E.n_layer * 1e6, 2),
                   "bytes_per_layer_step": round(dec_bytes / E.n_layer),
                   "stream_read_ref_GB/s": stream_ref and round(stream_ref, 1),
                   "frac_of_stream_read_ref": stream_ref and round(dec_gbs / stream_ref, 4),
                   "pattern_ref": pattern_ref,
                   "reading_b": reading_b, "step_graph": step_graph, "small_batch": small,
                   "long_context": longctx},
        "prefill": {"TFLOP/s": round(med(pre_tf_s), 2), "ms_per_layer": round(t_pre * 1e3, 4)},
        "d26": d26,
        "small_configs": small_cfg,
        "varlen": varlen,
        "qknorm": qknorm,
        "roofline": roofline,
        "roofline_decode": roofline_decode,
        "cpu_baseline": cpu,
        "clocks": clocks,
        "device": props.name,
        "kernel_source_hash": src_hash,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
