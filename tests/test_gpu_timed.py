"""The measurement entry point moe_decode_layer_timed against
moe_decode_layer: the same kernels, so identical bits; the kernel count of
each launch sequence (one token, one token with a shared expert of its own
width, batched, batched with such a shared expert); and one start/end event
pair per kernel, in launch order on the launch stream."""
import numpy as np
import pytest

from gpu_helpers import (G, M, dev_u16, device_layer, host_u16, pick_tokens, release_device_layers,
                         shape_of, torch, weights_of, workspace)
from test_gpu_batched import SMALL as BATCHED_SMALL
from test_gpu_layer import SMALL as LAYER_SMALL

pytestmark = pytest.mark.gpu

CASES = [("tiny", 1, 3), ("fs_wide", 1, 4), ("tiny", 5, 6), ("fs_narrow", 17, 8)]


@pytest.mark.parametrize("name,T,n_kernels", CASES)
def test_timed_entry_matches_layer_and_times_every_kernel(name, T, n_kernels):
    t = torch()
    small = LAYER_SMALL if T == 1 else BATCHED_SMALL
    w = small[name] if name in small else G.WORKLOADS[name]
    dl = device_layer(w, 0)
    X = np.stack([x for _, x in pick_tokens(w, dl.router_host, T, start=70)])
    x = dev_u16(X)
    ws = workspace(w, T)
    res = []
    for timed in (False, True):
        out = t.full_like(x, 0x7FC0)
        idx = t.full((T, w.k), -1, dtype=t.int32, device="cuda")
        wts = t.full((T, w.k), -1.0, dtype=t.float32, device="cuda")
        if timed:
            ev = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True))
                  for _ in range(M.MOE_MAX_LAYER_KERNELS)]
            for a, b in ev:  # torch creates an event on its first record
                a.record()
                b.record()
            nk = M.decode_layer_timed(shape_of(w), weights_of(dl), x, x, out, T, idx, wts, ws, ev)
        else:
            M.decode_layer(shape_of(w), weights_of(dl), x, x, out, T, idx, wts, ws)
        t.cuda.synchronize()
        res.append((host_u16(out).copy(), idx.cpu().numpy(), wts.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0])
    assert np.array_equal(res[0][1], res[1][1])
    assert np.array_equal(res[0][2].view(np.uint32), res[1][2].view(np.uint32))
    assert nk == n_kernels, (name, T, nk)
    for i in range(nk):
        assert ev[i][0].elapsed_time(ev[i][1]) > 0.0
        if i + 1 < nk:
            assert ev[i][1].elapsed_time(ev[i + 1][0]) >= 0.0
    release_device_layers()
