#!/usr/bin/env python3
"""Throughput of the sparse-MoE decode layer on one MI355X.

A step is one decode layer (router GEMV, top-k + softmax, gate/up with SiLU
gating, down projection, weighted combine with the shared expert, residual
add) on one batch of the chosen workload, through the C ABI of
libmoe_decode.so.  Default workload: the K3-shaped batch-1 layer (hidden 7168,
896 routed experts, top-16, expert FFN 2048, one shared expert of FFN 2048).

Measurement
-----------
* Several independent weight sets (about 21 GB each) stay resident in HBM and
  16 distinct tokens are rotated over them, so consecutive steps stream
  different bytes and the 256 MB Infinity Cache cannot serve a step from the
  previous one.
* The K timed steps are captured into HIP graphs (one graph of all K steps
  when K <= 256, else graphs of 64) and replayed; a device synchronisation
  and HIP events on the stream the kernels run on bracket them.  p10/p50/p90
  come from the per-replay times.
* Before the timed replays the GPU is settled: after the W warmup steps and
  the graph's upload, the same graph is replayed (untimed) until SETTLE_S of
  back-to-back work has run.  Right after a capture or an idle spell the
  first ~10 ms of replays run up to ~12 % slower than the steady state (the
  GPU's clocks and power state adjust), which a short timed region would
  otherwise measure instead of the layer.  The JSON reports the settle work.
  One more untimed replay is enqueued right before the event that opens
  the timed region, with no synchronisation in between: after a
  synchronisation the stream is idle, so the opening event would fire at
  once and the timed region would also hold the host's submission of the
  graph and a cold start (measured: a single timed 20-step replay ran 0.2 to
  1.5 us per layer above the replays that followed it).
* Kernel pass: the same rotation through moe_decode_layer_timed, which
  launches the same kernels with HIP recording each kernel's own start and
  end; it gives the kernels per layer, their mean durations, the idle time
  between them, and the dominant kernel's duration for the roofline.
* A plain streaming read of 4 GiB gives this GPU's measured read ceiling as
  context for the 8 TB/s peak.
* The fp64 CPU oracle is timed on a bounded sample of the same workload
  (cpu_baseline leg; the oracle is test infrastructure and is used here only
  as that reported baseline).

Prints ONE JSON line on stdout; details go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published
METRIC = "µs per MoE decode layer (batch 1) and achieved HBM GB/s as fraction of peak"
ROT_TOKENS = 16                 # distinct batches in the rotation
ONE_GRAPH_MAX = 256             # up to this many steps are captured as one graph
GRAPH_STEPS = 64                # steps per graph beyond that
SETTLE_S = 0.15                 # untimed back-to-back replays before the timed ones
CALIB_BYTES = 1 << 30           # size of the counter-calibration copy
STREAM_BYTES = 4 << 30          # streaming-read ceiling buffer
PROFILES = os.path.join(ROOT, "profiles")
COUNTERS = {  # workload -> committed rocprofv3 counter summary
    "k3_batch1": os.path.join(PROFILES, "k2_gateup_k3_batch1_counters.txt"),
    "k3_batch64_zipf": os.path.join(PROFILES, "kb_gateup_kb_down_k3_batch64_counters.txt"),
}
T1_KERNELS = ["k1_router", "k2_gateup", "k3_down_combine"]
TB_KERNELS = ["kb_router", "kb_topk", "kb_group", "kb_gateup", "kb_down", "kb_combine"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def mx_bytes(rows: int, cols: int) -> int:
    """Bytes of one MXFP4 matrix: codes (4 bits/element) + one scale per 32."""
    return rows * cols // 2 + rows * cols // 32


def layer_bytes(w, touched=None) -> int:
    """Compulsory HBM bytes of one decode layer: x in, out, router rows, and
    every touched expert once (the k routed experts of each token; at batch
    T > 1 the distinct experts the batch selected) plus the shared expert;
    the residual is x."""
    expert = 2 * mx_bytes(w.F, w.H) + mx_bytes(w.H, w.F)
    shared = w.S * (2 * mx_bytes(w.Fs, w.H) + mx_bytes(w.H, w.Fs))
    gamma = 2 * w.H if w.L > 1 else 0
    n = w.T * w.k if touched is None else touched
    return w.T * (2 * w.H + 2 * w.H) + 2 * w.E * w.H + n * expert + shared + gamma


def gateup_bytes_in_layer(w, touched=None) -> int:
    """Compulsory bytes of the layer's gate/up kernel: gate and up matrices of
    every touched routed expert and of the shared expert, x in, the router
    logits in (batch 1: the selection runs in this kernel), and the gated
    activations out (two bf16 parts per element)."""
    n = w.T * w.k if touched is None else touched
    mats = n * 2 * mx_bytes(w.F, w.H) + w.S * 2 * mx_bytes(w.Fs, w.H)
    logits = 4 * w.E if w.T == 1 else 0
    acts = 2 * 2 * w.T * (w.k * w.F + w.S * w.Fs)
    return mats + 2 * w.T * w.H + logits + acts


def gateup_bytes_standalone(w) -> int:
    """The exported routed gate/up: k experts' gate and up matrices, x in,
    fp32 activations out."""
    return w.k * 2 * mx_bytes(w.F, w.H) + 2 * w.H + 4 * w.k * w.F


def measured_traffic(workload: str, kernel_key: str):
    """HBM bytes per launch of one kernel from the committed rocprofv3 counter
    summary, or None if there is none or it was taken on other kernel
    sources."""
    from sparse_moe_decode_gemv_amd import profiling as P
    path = COUNTERS.get(workload)
    if not path or not os.path.exists(path):
        return None
    vals, table = P.read_counter_summary(path)
    # A kernel's bytes depend on its own source file (and the shared headers):
    # the kb_* kernels on the batched file, the others on the one-token file.
    if kernel_key.startswith("kb_"):
        field, src = "batched_source_sha256_16", P.BATCHED_SRC
    else:
        field, src = "kernel_source_sha256_16", P.KERNEL_SRC
    if vals.get(field) != P.source_digest(src):
        return None
    return table.get(kernel_key)


def cpu_info():
    visible = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return visible, model


# ----------------------------------------------------------------- CPU leg
def cpu_baseline(w, router_hosts, toks, budget_s: float):
    """The fp64 oracle on a bounded sample of the same layer calls."""
    from concurrent.futures import ThreadPoolExecutor

    import moe_inputs as G
    import oracle as O
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                      # pragma: no cover
        threadpool_limits = None

    visible, model = cpu_info()
    # the host's CPU share for one GPU (the environment's thread setting), at
    # most what the process may run on
    share = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    cores = max(1, min(visible, share))
    pool = ThreadPoolExecutor(max_workers=cores)
    hx = G.HostExperts(w, 0)
    shared = hx.shared()
    done, spent = 0, 0.0
    lim = threadpool_limits(1) if threadpool_limits else None
    try:
        for x in toks:
            # input generation (expert bytes for this token) stays outside the clock
            sel = O.topk_select(O.router_logits(x, router_hosts[0]), w.k)[0]
            cache = {int(e): hx.routed(int(e)) for e in sel}
            t0 = time.perf_counter()
            O.moe_layer(x, router_hosts[0], w.k, lambda e: cache[e], shared,
                        residual_bits=x, pmap=pool.map)
            spent += time.perf_counter() - t0
            done += 1
            if spent >= budget_s:
                break
    finally:
        if lim is not None:
            lim.unregister()
        pool.shutdown()
    unit = "µs per layer" if w.T == 1 else "µs per token per layer"
    return {"value": round(spent / done * 1e6, 1), "unit": unit, "cores": cores,
            "kind": "oracle", "cores_visible": visible, "cpu_model": model,
            "sample": f"{done} single token(s) of {w.name} through one layer (weight set 0), "
                      f"fp64 numpy oracle on {cores} worker threads (the host's CPU share for "
                      f"one GPU; {visible} visible), BLAS limited to 1 thread per worker; "
                      f"expert bytes generated before the clock starts"}


# ------------------------------------------------------------------ GPU leg
def percentiles(v):
    import numpy as np
    q = np.percentile(np.asarray(v), [10, 50, 90])
    return {"p10": round(float(q[0]), 3), "p50": round(float(q[1]), 3), "p90": round(float(q[2]), 3)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="k3_batch1",
                    choices=["tiny", "k3_batch1", "k3_tp16_slice", "k3_stack8",
                             "k3_batch64_zipf", "k3_verify8"])
    ap.add_argument("--sets", type=int, default=4, help="resident weight sets rotated")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step directly (no graph), e.g. under counter profiling")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed steps (no kernel pass, stand-alone gate/up or "
                         "streaming read), e.g. under counter profiling")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): the decode layer is built and measured on a single MI355X; "
              f"multi-GPU sharding is not part of this library.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_inputs as G
    import sparse_moe_decode_gemv_amd as M

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (torch.cuda.is_available() is False)")
    M.lib()                                   # fails loudly if the library is not built
    torch.cuda.set_device(0)
    w = G.WORKLOADS[args.workload]
    stack = w.L > 1
    nsets = 1 if stack else max(1, args.sets)
    nlayers = w.L if stack else 1
    log(f"[bench] workload {w.name}: H={w.H} E={w.E} k={w.k} F={w.F} S={w.S} L={w.L}; "
        f"{nsets} weight set(s) x {nlayers} layer(s)")

    t0 = time.time()
    sets = [[G.DeviceLayer(w, s * nlayers + l) for l in range(nlayers)] for s in range(nsets)]
    torch.cuda.synchronize()
    log(f"[bench] weights resident in {time.time() - t0:.1f}s, "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")
    # A plain device copy of known size (1 GiB read + 1 GiB written), run once
    # so that HBM byte counters of a profiled run can be scaled against it.
    calib_src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst
    shape = M.make_shape(w.H, w.E, w.k, w.F, w.S, w.Fs)
    wts = [[M.make_weights(d.router, d.gate, d.up, d.down, d.s_gate, d.s_up, d.s_down)
            for d in s] for s in sets]
    T = w.T
    toks_host = [np.stack([G.token(w, ROT_TOKENS * b + d) for d in range(T)])
                 for b in range(ROT_TOKENS)]           # ROT_TOKENS batches of T tokens
    xs = torch.from_numpy(np.stack(toks_host).view(np.int16)).cuda()   # [R][T][H]
    outs = torch.empty_like(xs)
    hid = xs.clone()
    ws = torch.empty(M.workspace_size(shape, T), dtype=torch.uint8, device="cuda")
    M.workspace_init(ws)

    def step(i):
        s, t = i % nsets, i % ROT_TOKENS
        if stack:
            M.decode_stack(shape, wts[s], [d.gamma for d in sets[s]], w.eps, hid[t], T,
                           None, None, ws)
        else:
            M.decode_layer(shape, wts[s][0], xs[t], xs[t], outs[t], T, None, None, ws)

    touched = None
    if T > 1 and not stack:
        # distinct experts each (weight set, batch) selects, for the byte count
        idx = torch.empty((T, w.k), dtype=torch.int32, device="cuda")
        tw = torch.empty((T, w.k), dtype=torch.float32, device="cuda")
        counts = []
        for i in range(ROT_TOKENS):
            s_, t_ = i % nsets, i % ROT_TOKENS
            M.router_topk(shape, xs[t_], sets[s_][0].router, T, idx, tw, None, ws)
            counts.append(len(np.unique(idx.cpu().numpy())))
        touched = float(np.mean(counts))
        log(f"[bench] distinct experts per batch: mean {touched:.1f}, "
            f"min {min(counts)}, max {max(counts)}")

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- the timed steps
    K = args.steps
    per_rep, rep_steps, settle = [], 0, None
    if args.eager:
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(K):
            step(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        total_ms = ev0.elapsed_time(ev1)
    else:
        def capture(first, n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(first, first + n):
                    step(i)
            return g
        rep_steps = K if K <= ONE_GRAPH_MAX else GRAPH_STEPS
        full, rem = divmod(K, rep_steps)
        # rep_steps is a multiple of the rotation or covers K: every replay
        # walks the same rotation
        g_full = capture(0, rep_steps) if full else None
        g_rem = capture(0, rem) if rem else None
        for g in (g_full, g_rem):             # first replay uploads the graph: untimed
            if g is not None:
                g.replay()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(full + 2)]
        # settle (untimed): replays back to back until SETTLE_S has passed
        g_settle = g_full if g_full is not None else g_rem
        settle_steps, t_settle = 0, time.perf_counter()
        while time.perf_counter() - t_settle < SETTLE_S:
            for _ in range(4):
                g_settle.replay()
            settle_steps += 4 * (rep_steps if g_full is not None else rem)
            torch.cuda.synchronize()
        settle = {"steps": settle_steps, "seconds": round(time.perf_counter() - t_settle, 3)}
        # one more untimed replay right before the opening event, with no
        # synchronisation in between (see the module docstring)
        g_settle.replay()
        settle["lead_steps"] = rep_steps if g_full is not None else rem
        evs[0].record(stream)
        for r in range(full):
            g_full.replay()
            evs[r + 1].record(stream)
        if g_rem is not None:
            g_rem.replay()
        evs[-1].record(stream)
        torch.cuda.synchronize()
        total_ms = evs[0].elapsed_time(evs[-1])
        per_rep = [evs[r].elapsed_time(evs[r + 1]) * 1e3 / (rep_steps * nlayers) for r in range(full)]

    ms_per_step = total_ms / K
    us_layer = ms_per_step * 1e3 / nlayers
    lb = int(layer_bytes(w, touched))
    layer_gbps = lb / (us_layer * 1e-6) / 1e9
    log(f"[bench] {K} steps in {total_ms:.3f} ms: {us_layer:.2f} µs/layer, "
        f"{layer_gbps:.0f} GB/s algorithmic ({lb} B/layer), "
        f"{layer_gbps / PEAK_HBM_GBPS:.3f} of peak")

    # ---- spread over graph replays (extra untimed replays when the timed
    # region holds fewer than 8)
    spread = None
    if not args.eager:
        src = f"{len(per_rep)} timed replays of {rep_steps} steps"
        if len(per_rep) < 8 and g_full is not None:
            extra = [torch.cuda.Event(enable_timing=True) for _ in range(33)]
            torch.cuda.synchronize()
            g_full.replay()  # untimed lead, as for the timed replays
            extra[0].record(stream)
            for r in range(32):
                g_full.replay()
                extra[r + 1].record(stream)
            torch.cuda.synchronize()
            per_rep = per_rep + [extra[r].elapsed_time(extra[r + 1]) * 1e3 / (rep_steps * nlayers)
                                 for r in range(32)]
            src += " + 32 untimed replays of the same graph"
        if per_rep:
            spread = {"unit": "µs/layer", **percentiles(per_rep), "source": src}
            log(f"[bench] per-replay µs/layer p10 {spread['p10']} p50 {spread['p50']} "
                f"p90 {spread['p90']} ({src})")

    kernels = roofline = standalone = ceiling = warm = None
    if not args.no_extras:
        # ---- kernel pass: every kernel of a layer timed by HIP itself
        names = T1_KERNELS if T == 1 else TB_KERNELS
        nk_max = len(names)
        n_prof = min(64, max(16, K))
        # the stack's layers are the batch-1 layer's kernels (RMSNorm runs in
        # the router's prologue); they are timed as plain layers here
        evp = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(nk_max)] for _ in range(n_prof)]
        for row in evp:                       # create the events before handing them over
            for a, b in row:
                a.record(stream)
                b.record(stream)
        torch.cuda.synchronize()
        nks = []
        for i in range(n_prof):
            s, t = i % nsets, i % ROT_TOKENS
            lay = i % nlayers
            nks.append(M.decode_layer_timed(shape, wts[s][lay], xs[t], xs[t], outs[t], T, None,
                                            None, ws, evp[i]))
        torch.cuda.synchronize()
        assert len(set(nks)) == 1 and nks[0] == nk_max, nks
        dur = np.array([[a.elapsed_time(b) * 1e3 for a, b in row] for row in evp])
        gaps = np.array([[row[j][1].elapsed_time(row[j + 1][0]) * 1e3 for j in range(nk_max - 1)]
                         for row in evp])
        span = np.array([row[0][0].elapsed_time(row[-1][1]) * 1e3 for row in evp])
        kernels = {"per_layer": nk_max, "names": names,
                   "mean_us": {n: round(float(dur[:, j].mean()), 3) for j, n in enumerate(names)},
                   "idle_between_kernels_us": round(float(gaps.sum(axis=1).mean()), 3),
                   "gap_us": [round(float(g), 3) for g in gaps.mean(axis=0)],
                   "layer_span_us": round(float(span.mean()), 3),
                   "source": f"moe_decode_layer_timed over {n_prof} layers of the same rotation, "
                             f"eager; each kernel's start and end recorded by HIP (the eager "
                             f"launches leave gaps a graph does not have)"}
        if not stack:
            # in the graph: the timed µs per layer minus the kernels' own time
            kernels["graph_idle_us_per_layer"] = round(us_layer - float(dur.mean(axis=0).sum()), 3)
        log(f"[bench] kernels per layer {nk_max}: " +
            ", ".join(f"{n} {kernels['mean_us'][n]:.2f} µs" for n in names) +
            f"; idle between them {kernels['idle_between_kernels_us']:.2f} µs; "
            f"span {kernels['layer_span_us']:.2f} µs")

        # ---- roofline of the dominant kernel as it runs in the layer
        kname = "k2_gateup" if T == 1 else "kb_gateup"
        j = names.index(kname)
        kb = gateup_bytes_in_layer(w, touched)
        us_k = float(dur[:, j].mean())
        ach = kb / (us_k * 1e-6) / 1e9
        key = "k2_gateup (in layer)" if T == 1 else "kb_gateup"
        traffic = measured_traffic(w.name, key)
        roofline = {"bound": "hbm", "kernel": f"{kname} in the layer (gate/up + SiLU gating of "
                                              f"the selected and shared experts)",
                    "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": traffic,
                    "bytes_per_launch": kb, "us_per_launch": round(us_k, 3)}
        log(f"[bench] {kname} in the layer: {us_k:.2f} µs/launch, {ach:.0f} GB/s "
            f"({kb} B/launch), traffic {traffic}")

        # ---- the exported routed gate/up alone (batch 1)
        if T == 1 and not stack:
            idx = torch.empty((nsets, ROT_TOKENS, w.k), dtype=torch.int32, device="cuda")
            tw = torch.empty((nsets, ROT_TOKENS, w.k), dtype=torch.float32, device="cuda")
            for s in range(nsets):
                for t in range(ROT_TOKENS):
                    M.router_topk(shape, xs[t], sets[s][0].router, 1, idx[s, t:t + 1],
                                  tw[s, t:t + 1], None, ws)
            act = torch.empty((w.k, w.F), dtype=torch.float32, device="cuda")

            def gu(i):
                s, t = i % nsets, i % ROT_TOKENS
                M.expert_gateup(shape, wts[s][0], xs[t], idx[s, t:t + 1], 1, act, ws)

            for i in range(ROT_TOKENS):
                gu(i)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(ROT_TOKENS):
                    gu(i)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 8
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us_sa = e0.elapsed_time(e1) * 1e3 / (reps * ROT_TOKENS)
            kb_sa = gateup_bytes_standalone(w)
            standalone = {"kernel": "k2_gateup via moe_expert_gateup (16 routed experts given, "
                                    "no selection, no shared expert)",
                          "us_per_launch": round(us_sa, 3), "bytes_per_launch": kb_sa,
                          "achieved": round(kb_sa / (us_sa * 1e-6) / 1e9, 1),
                          "traffic": measured_traffic(w.name, "k2_gateup (stand-alone)")}
            log(f"[bench] routed gate/up alone: {us_sa:.2f} µs/launch, "
                f"{standalone['achieved']:.0f} GB/s")

        # ---- measured streaming-read ceiling
        buf = torch.empty(STREAM_BYTES, dtype=torch.uint8, device="cuda")
        sink = torch.empty(M.MOE_STREAM_SINK_WORDS, dtype=torch.int32, device="cuda")
        for _ in range(2):
            M.stream_read(buf, sink)
        reps = 8
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            M.stream_read(buf, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        gbps = STREAM_BYTES * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        ceiling = {"kernel": "stream_read_kernel (moe_stream_read, 16-byte nontemporal loads)",
                   "bytes": STREAM_BYTES, "achieved": round(gbps, 1), "unit": "GB/s",
                   "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
                   "layer_frac_of_ceiling": round(layer_gbps / gbps, 4)}
        del buf
        log(f"[bench] streaming read of {STREAM_BYTES >> 30} GiB: {gbps:.0f} GB/s "
            f"({gbps / PEAK_HBM_GBPS:.3f} of peak); layer at {layer_gbps / gbps:.3f} of it")

        # ---- warm number: one token and one weight set, the same call 16
        # times per graph (caches may keep weights between calls; context
        # only, the metric above rotates tokens and weight sets)
        if not args.eager:
            g_w = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_w):
                for _ in range(ROT_TOKENS):
                    step(0)
            for _ in range(3):
                g_w.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 8
            e0.record(stream)
            for _ in range(reps):
                g_w.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us_w = e0.elapsed_time(e1) * 1e3 / (reps * ROT_TOKENS * nlayers)
            warm = {"us_per_layer": round(us_w, 3),
                    "what": f"one token and one weight set, the same call {ROT_TOKENS} times per "
                            "graph (weights may stay cached between calls); context, not the metric"}
            del g_w
            log(f"[bench] warm, same token and weights: {us_w:.2f} µs/layer")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host ...")
        cpu = cpu_baseline(w, [d.router_host for d in sets[0]],
                           [b[0] for b in toks_host[:8]], args.cpu_seconds)
        log(f"[bench] oracle: {cpu['value']} {cpu['unit']} on {cpu['cores']} threads "
            f"({cpu['cpu_model']})")

    line = {
        "metric": METRIC, "value": round(us_layer, 3), "unit": "µs/layer",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "settle_untimed": settle,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4xbf16-fp32acc", "data": "synthetic",
        "config": {"workload": f"{w.name}: T={w.T} H={w.H} E={w.E} top-{w.k} F={w.F} "
                               f"shared={w.S}x{w.Fs} layers={nlayers}",
                   "global_batch": w.T, "weight_sets": nsets,
                   "timing": "eager" if args.eager else
                   f"hipGraph replays of {rep_steps} steps"},
        "layer_tokens_per_s": round(T * 1e6 / us_layer, 1),
        "us_per_token": round(ms_per_step * 1e3 / T, 3) if stack else None,
        "layer_hbm": {"bytes": lb, "achieved": round(layer_gbps, 1), "unit": "GB/s",
                      "frac": round(layer_gbps / PEAK_HBM_GBPS, 4)},
        "spread": spread,
        "kernels": kernels,
        "roofline": roofline,
        "gateup_standalone": standalone,
        "stream_read_ceiling": ceiling,
        "warm_same_inputs": warm,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line, ensure_ascii=False), flush=True)


if __name__ == "__main__":
    main()
