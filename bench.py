#!/usr/bin/env python3
"""Throughput of the sparse-MoE decode layer on one MI355X.

A step is one decode layer (router GEMV, top-k + softmax, gate/up with SiLU
gating, down projection, weighted combine with the shared expert, residual
add) on one token of the chosen workload, through the C ABI of
libmoe_decode.so.  Default workload: the K3-shaped batch-1 layer (hidden 7168,
896 routed experts, top-16, expert FFN 2048, one shared expert of FFN 2048).

Measurement
-----------
* Several independent weight sets (about 21 GB each) stay resident in HBM and
  16 distinct tokens are rotated over them, so consecutive steps stream
  different bytes and the 256 MB Infinity Cache cannot serve a step from the
  previous one.
* Steps are captured into HIP graphs of 16 layer calls and replayed; the K
  timed steps are bracketed by a device synchronisation and HIP events on
  the stream the kernels run on.
* The dominant kernel (routed gate/up) is also timed on its own, in graphs of
  16 launches over the same rotation, for the roofline figure.
* The fp64 CPU oracle is timed on a bounded sample of the same workload
  (cpu_baseline leg; the oracle is test infrastructure and is used here only
  as that reported baseline).

Prints ONE JSON line on stdout; details go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published
METRIC = "µs per MoE decode layer (batch 1) and achieved HBM GB/s as fraction of peak"
ROT_TOKENS = 16                 # distinct tokens in the rotation (= steps per graph)
CALIB_BYTES = 1 << 30           # size of the counter-calibration copy
COUNTERS = os.path.join(ROOT, "profiles", "k2_gateup_k3_batch1_counters.txt")
KERNEL_SRC = os.path.join(ROOT, "sparse_moe_decode_gemv_amd", "csrc", "moe_t1.hip")


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


def gateup_bytes(w) -> int:
    """Compulsory bytes of one routed gate/up launch: k experts' gate and up
    matrices, x in, fp32 activations out."""
    return w.k * 2 * mx_bytes(w.F, w.H) + 2 * w.H + 4 * w.k * w.F


def source_digest() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per gate/up launch from the committed rocprofv3 counter
    summary, or None if it is missing or was taken on another kernel source."""
    if not os.path.exists(COUNTERS):
        return None
    vals = {}
    with open(COUNTERS) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != source_digest():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


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

    cores = max(1, min(16, len(os.sched_getaffinity(0))))
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
    # one token per call: per layer at batch 1, per token and layer otherwise
    unit = "µs per layer" if w.T == 1 else "µs per token per layer"
    return {"value": round(spent / done * 1e6, 1), "unit": unit, "cores": cores,
            "kind": "oracle",
            "sample": f"{done} single token(s) of {w.name} through one layer (weight set 0), "
                      f"fp64 numpy oracle, {cores} worker threads, BLAS limited to 1 thread; "
                      f"expert bytes generated before the clock starts"}


# ------------------------------------------------------------------ GPU leg
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

    K = args.steps
    per_rep = []
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
        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    step(i)
            return g
        full, rem = divmod(K, ROT_TOKENS)
        g_full = capture(ROT_TOKENS) if full else None
        g_rem = capture(rem) if rem else None
        for g in (g_full, g_rem):             # first replay uploads the graph: untimed
            if g is not None:
                g.replay()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(full + 2)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for r in range(full):
            g_full.replay()
            evs[r + 1].record(stream)
        if g_rem is not None:
            g_rem.replay()
        evs[-1].record(stream)
        torch.cuda.synchronize()
        total_ms = evs[0].elapsed_time(evs[-1])
        per_rep = [evs[r].elapsed_time(evs[r + 1]) / ROT_TOKENS for r in range(full)]

    ms_per_step = total_ms / K
    us_layer = ms_per_step * 1e3 / nlayers
    lb = int(layer_bytes(w, touched))
    layer_gbps = lb / (us_layer * 1e-6) / 1e9
    log(f"[bench] {K} steps in {total_ms:.3f} ms: {us_layer:.2f} µs/layer, "
        f"{layer_gbps:.0f} GB/s algorithmic ({lb} B/layer), "
        f"{layer_gbps / PEAK_HBM_GBPS:.3f} of peak")
    if per_rep:
        q = np.percentile(np.array(per_rep) * 1e3 / nlayers, [10, 50, 90])
        log(f"[bench] per-graph µs/layer p10 {q[0]:.2f} p50 {q[1]:.2f} p90 {q[2]:.2f}")

    # ---- dominant kernel alone: routed gate/up over the same rotation
    roofline = None
    if not stack and T == 1:
        k = w.k
        idx = torch.empty((nsets, ROT_TOKENS, k), dtype=torch.int32, device="cuda")
        tw = torch.empty((nsets, ROT_TOKENS, k), dtype=torch.float32, device="cuda")
        for s in range(nsets):
            for t in range(ROT_TOKENS):
                M.router_topk(shape, xs[t], sets[s][0].router, 1, idx[s, t:t + 1],
                              tw[s, t:t + 1], None, ws)
        act = torch.empty((k, w.F), dtype=torch.float32, device="cuda")

        def gu(i):
            s, t = i % nsets, i % ROT_TOKENS
            M.expert_gateup(shape, wts[s][0], xs[t], idx[s, t:t + 1], 1, act, ws)

        for i in range(ROT_TOKENS):
            gu(i)
        n_launch = max(ROT_TOKENS, (K // ROT_TOKENS) * ROT_TOKENS)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if args.eager:
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(n_launch):
                gu(i)
            e1.record(stream)
        else:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(ROT_TOKENS):
                    gu(i)
            g.replay()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(n_launch // ROT_TOKENS):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        us_k2 = e0.elapsed_time(e1) * 1e3 / n_launch
        kb = gateup_bytes(w)
        ach = kb / (us_k2 * 1e-6) / 1e9
        # the counter summary covers the K3 batch-1 workload's gate/up launch only
        traffic = measured_traffic() if w.name == "k3_batch1" else None
        roofline = {"bound": "hbm", "kernel": "k2_gateup (routed gate/up + SiLU gating)",
                    "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": traffic,
                    "bytes_per_launch": kb, "us_per_launch": round(us_k2, 3)}
        log(f"[bench] gate/up kernel alone: {us_k2:.2f} µs/launch, {ach:.0f} GB/s "
            f"({kb} B/launch), traffic {traffic}")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host ...")
        cpu = cpu_baseline(w, [d.router_host for d in sets[0]],
                           [b[0] for b in toks_host[:8]], args.cpu_seconds)
        log(f"[bench] oracle: {cpu['value']} {cpu['unit']} on {cpu['cores']} threads")

    line = {
        "metric": METRIC, "value": round(us_layer, 3), "unit": "µs/layer",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4xbf16-fp32acc", "data": "synthetic",
        "config": {"workload": f"{w.name}: T={w.T} H={w.H} E={w.E} top-{w.k} F={w.F} "
                               f"shared={w.S}x{w.Fs} layers={nlayers}",
                   "global_batch": w.T, "weight_sets": nsets,
                   "timing": "eager" if args.eager else "hipGraph of 16 steps"},
        "layer_tokens_per_s": round(T * 1e6 / us_layer, 1),
        "layer_hbm": {"bytes": lb, "achieved": round(layer_gbps, 1), "unit": "GB/s",
                      "frac": round(layer_gbps / PEAK_HBM_GBPS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line, ensure_ascii=False), flush=True)


if __name__ == "__main__":
    main()
