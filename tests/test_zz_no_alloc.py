"""The no-allocation layer entry point (moe_decode_layer_noalloc) against
moe_decode_layer with a caller workspace: the same kernels, so the outputs,
indices and weights must be identical bit for bit.  Consecutive calls share
the library's scratch array: a batched K3-shaped call (8 tokens), then a
smaller single-token K3 call, then a single-token call whose down rows are
combined across workgroups through the counters at the head of the scratch,
then a batched call whose shared expert has its own width (its own gate/up
and down launches), then graph replays of a captured call."""
import numpy as np
import pytest

from gpu_helpers import (G, M, dev_u16, device_layer, host_u16, pick_tokens,
                         release_device_layers, shape_of, torch, weights_of, workspace)

pytestmark = pytest.mark.gpu

WIDE = G.Workload("wide_f", T=1, H=2048, E=24, k=4, F=4096, S=1, Fs=4096, seed=0x5EED0105)
FS_NARROW = G.Workload("fs_narrow_b", T=1, H=2048, E=16, k=3, F=1024, S=1, Fs=128, seed=0x5EED0207)


def _tokens(w, dl, T, start):
    return np.stack([x for _, x in pick_tokens(w, dl.router_host, T, start=start)])


def _compare(w, dl, X):
    t = torch()
    T = X.shape[0]
    x = dev_u16(X)
    outs, idxs, wtss = [], [], []
    for noalloc in (False, True):
        out = t.full_like(x, 0x7FC0)
        idx = t.full((T, w.k), -1, dtype=t.int32, device="cuda")
        wts = t.full((T, w.k), -1.0, dtype=t.float32, device="cuda")
        if noalloc:
            M.decode_layer_noalloc(shape_of(w), weights_of(dl), x, x, out, T, idx, wts)
        else:
            M.decode_layer(shape_of(w), weights_of(dl), x, x, out, T, idx, wts, workspace(w, T))
        t.cuda.synchronize()
        outs.append(host_u16(out).copy())
        idxs.append(idx.cpu().numpy())
        wtss.append(wts.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(idxs[0], idxs[1])
    assert np.array_equal(wtss[0].view(np.uint32), wtss[1].view(np.uint32))


def test_noalloc_matches_workspace_entry_on_consecutive_calls():
    w8 = G.WORKLOADS["k3_verify8"]
    dl8 = device_layer(w8, 0)
    _compare(w8, dl8, _tokens(w8, dl8, 8, start=10))          # batched path, larger
    w1 = G.WORKLOADS["k3_batch1"]
    dl1 = device_layer(w1, 0)
    _compare(w1, dl1, _tokens(w1, dl1, 1, start=20))          # one token, smaller
    dlw = device_layer(WIDE, 0)
    _compare(WIDE, dlw, _tokens(WIDE, dlw, 1, start=30))      # cross-workgroup combine
    _compare(WIDE, dlw, _tokens(WIDE, dlw, 1, start=40))      # counters back at zero
    dlf = device_layer(FS_NARROW, 0)
    _compare(FS_NARROW, dlf, _tokens(FS_NARROW, dlf, 17, start=50))  # shared expert apart
    release_device_layers()


def test_noalloc_call_replays_from_a_graph():
    t = torch()
    w = G.WORKLOADS["tiny"]
    dl = device_layer(w, 0)
    toks = [x for _, x in pick_tokens(w, dl.router_host, 3, start=60)]
    x = dev_u16(toks[0].reshape(1, -1))
    out = t.empty_like(x)
    ref = []
    for tk in toks:
        xx = dev_u16(tk.reshape(1, -1))
        o = t.empty_like(xx)
        M.decode_layer(shape_of(w), weights_of(dl), xx, xx, o, 1, None, None, workspace(w, 1))
        t.cuda.synchronize()
        ref.append(host_u16(o).copy())
    M.decode_layer_noalloc(shape_of(w), weights_of(dl), x, x, out, 1, None, None)  # eager first
    t.cuda.synchronize()
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        M.decode_layer_noalloc(shape_of(w), weights_of(dl), x, x, out, 1, None, None)
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        M.decode_layer_noalloc(shape_of(w), weights_of(dl), x, x, out, 1, None, None)
    for rep in range(3):
        for i, tk in enumerate(toks):
            x.copy_(dev_u16(tk.reshape(1, -1)))
            out.zero_()
            g.replay()
            t.cuda.synchronize()
            assert np.array_equal(host_u16(out), ref[i]), (rep, i)
