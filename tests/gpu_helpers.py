"""Shared pieces of the GPU parity tests: device-resident workloads, the
library calls, and the comparison rules against the fp64 oracle."""
from __future__ import annotations

import functools
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import moe_inputs as G  # noqa: E402
import oracle as O  # noqa: E402
import sparse_moe_decode_gemv_amd as M  # noqa: E402

TOL = 2e-2          # max-abs-error <= TOL * rms(reference), per token
GAP = 1e-3          # top-k sets compared where the k-th/(k+1)-th gap exceeds this

_POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4))


def pmap(f, xs):
    return _POOL.map(f, xs)


def torch():
    import torch as _t
    return _t


def u16_to_i16(a: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(a).view(np.int16))


def dev_u16(a: np.ndarray):
    return u16_to_i16(a).cuda()


def host_u16(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def shape_of(w: G.Workload):
    return M.make_shape(w.H, w.E, w.k, w.F, w.S, w.Fs)


def weights_of(dl) -> "M.MoeLayerWeights":
    return M.make_weights(dl.router, dl.gate, dl.up, dl.down, dl.s_gate, dl.s_up, dl.s_down)


def workspace(w: G.Workload, T: int):
    t = torch()
    n = M.workspace_size(shape_of(w), T)
    ws = t.empty(n, dtype=t.uint8, device="cuda")
    M.workspace_init(ws)
    return ws


@functools.lru_cache(maxsize=4)
def device_layer(w: G.Workload, layer: int):
    return G.DeviceLayer(w, layer)


def release_device_layers():
    device_layer.cache_clear()
    torch().cuda.empty_cache()


def oracle_layer(w: G.Workload, layer: int, router_host, x_bits, residual_bits):
    hx = G.HostExperts(w, layer)
    return O.moe_layer(x_bits, router_host, w.k, hx.routed, hx.shared(),
                       residual_bits=residual_bits, pmap=pmap)


def pick_tokens(w: G.Workload, router_host, n: int, start: int = 0, adjacent: bool = False):
    """Draw indices (and tokens) whose oracle top-k gap exceeds GAP; with
    ``adjacent`` every consecutive gap among the top k+1 must exceed it."""
    out, d = [], start
    while len(out) < n:
        x = G.token(w, d)
        L = O.router_logits(x, router_host)
        ok = O.topk_gap(L, w.k)[0] > GAP
        if adjacent:
            ok = ok and O.adjacent_gaps(L, w.k)[0] > GAP
        if ok:
            out.append((d, x))
        d += 1
    return out


def check_topk(idx_gpu, ref, k, ordered=None, gap=GAP):
    """Exact set match where the oracle's k-th/(k+1)-th gap exceeds ``gap``
    (returns how many tokens were checked); exact order where every adjacent
    gap among the top k+1 exceeds it (or always, with ``ordered``)."""
    logits = np.atleast_2d(ref["logits"])
    idx_gpu = np.atleast_2d(idx_gpu)
    n = 0
    for t in range(idx_gpu.shape[0]):
        if O.topk_gap(logits[t:t + 1], k)[0] > gap:
            n += 1
            assert sorted(idx_gpu[t].tolist()) == sorted(ref["idx"][t].tolist()), (t, idx_gpu[t], ref["idx"][t])
        if ordered or (ordered is None and O.adjacent_gaps(logits[t:t + 1], k)[0] > gap):
            assert idx_gpu[t].tolist() == ref["idx"][t].tolist(), (t, idx_gpu[t], ref["idx"][t])
    return n


def max_err_ratio(out_bits, ref_out) -> np.ndarray:
    """Per token: max |gpu - ref| / rms(ref)."""
    g = O.bf16_to_f64(np.atleast_2d(out_bits))
    r = np.atleast_2d(ref_out)
    rms = np.sqrt((r * r).mean(axis=1))
    return np.abs(g - r).max(axis=1) / rms
