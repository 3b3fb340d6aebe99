"""GPU parity of the single-token decode layer against the fp64 oracle.

Every test calls the HIP library through its C ABI (ctypes binding) and
compares element by element with the oracle on the same seeded inputs.
Bars: top-k indices exact where the oracle's k-th/(k+1)-th logit gap
exceeds 1e-3; max-abs-error <= 2e-2 * rms(reference output) per token.
"""
import numpy as np
import pytest

from gpu_helpers import (GAP, TOL, G, M, O, check_topk, dev_u16, device_layer, host_u16,
                         max_err_ratio, oracle_layer, pick_tokens, release_device_layers,
                         shape_of, torch, weights_of, workspace)

pytestmark = pytest.mark.gpu

SMALL = {
    # ragged: E not a multiple of the router tiling, H=768 gives 3 blocks per lane
    "ragged": G.Workload("ragged", T=1, H=768, E=40, k=5, F=256, S=1, Fs=256, seed=0x5EED0101),
    "k1": G.Workload("k1", T=1, H=512, E=16, k=1, F=128, S=0, Fs=0, seed=0x5EED0102),
    "kmax": G.Workload("kmax", T=1, H=1024, E=32, k=32, F=512, S=1, Fs=512, seed=0x5EED0103),
    "one_expert": G.Workload("one_expert", T=1, H=256, E=1, k=1, F=128, S=1, Fs=128, seed=0x5EED0104),
    "wide_f": G.Workload("wide_f", T=1, H=2048, E=24, k=4, F=4096, S=1, Fs=4096, seed=0x5EED0105),
    "h8192": G.Workload("h8192", T=1, H=8192, E=20, k=3, F=1024, S=0, Fs=0, seed=0x5EED0106),
    # F/32 not a multiple of the 16 blocks one down load instruction covers
    "f384": G.Workload("f384", T=1, H=512, E=12, k=3, F=384, S=1, Fs=384, seed=0x5EED0108),
    "f640": G.Workload("f640", T=1, H=768, E=10, k=2, F=640, S=0, Fs=0, seed=0x5EED0109),
    "f1536": G.Workload("f1536", T=1, H=1024, E=8, k=2, F=1536, S=1, Fs=1536, seed=0x5EED010A),
    "f8192": G.Workload("f8192", T=1, H=256, E=4, k=2, F=8192, S=1, Fs=8192, seed=0x5EED010B),
    # the most experts and the largest top-k the library accepts together
    "emax": G.Workload("emax", T=1, H=512, E=1024, k=32, F=128, S=1, Fs=128, seed=0x5EED010C),
    # a shared expert wider, and one narrower, than the routed experts
    "fs_wide": G.Workload("fs_wide", T=1, H=1024, E=24, k=4, F=256, S=1, Fs=512, seed=0x5EED010D),
    "fs_narrow": G.Workload("fs_narrow", T=1, H=2048, E=16, k=3, F=1024, S=1, Fs=128,
                            seed=0x5EED010E),
    # FFN 4096 routed experts (cross-workgroup down combine) beside a 2048 shared one
    "fs_wide_f": G.Workload("fs_wide_f", T=1, H=2048, E=12, k=2, F=4096, S=1, Fs=2048,
                            seed=0x5EED010F),
}


def run_layer(w, dl, x_bits, residual="x", want_logits=False):
    return run_layer_ws(w, dl, x_bits, workspace(w, 1), residual)


def run_layer_ws(w, dl, x_bits, ws, residual="x"):
    t = torch()
    x = dev_u16(x_bits.reshape(1, -1))
    out = t.empty_like(x)
    idx = t.empty((1, w.k), dtype=t.int32, device="cuda")
    wts = t.empty((1, w.k), dtype=t.float32, device="cuda")
    res = x if residual == "x" else residual
    M.decode_layer(shape_of(w), weights_of(dl), x, res, out, 1, idx, wts, ws)
    t.cuda.synchronize()
    return host_u16(out)[0], idx.cpu().numpy(), wts.cpu().numpy()


def layer_parity(w, n_tokens=1, adjacent=False):
    dl = device_layer(w, 0)
    for d, x in pick_tokens(w, dl.router_host, n_tokens, adjacent=adjacent):
        out, idx, wts = run_layer(w, dl, x)
        ref = oracle_layer(w, 0, dl.router_host, x, x)
        check_topk(idx, ref, w.k, ordered=True if adjacent else None)
        np.testing.assert_allclose(wts, ref["w"], rtol=0, atol=2e-6)
        assert abs(float(wts.sum()) - 1.0) < 1e-5
        err = max_err_ratio(out, ref["out"])
        print(f"{w.name} draw={d} max_err/rms={err[0]:.3e}")
        assert err[0] <= TOL, (w.name, d, err)


def test_device_filler_matches_host_generator():
    w = G.WORKLOADS["tiny"]
    dl = device_layer(w, 0)
    hx = G.HostExperts(w, 0)
    for e in (0, 7, w.E - 1):
        ex = hx.routed(e)
        nc, ns = w.F * w.H // 2, w.F * w.H // 32
        assert np.array_equal(dl.gate[0][e * nc:(e + 1) * nc].cpu().numpy(), ex["gate"][0].ravel())
        assert np.array_equal(dl.gate[1][e * ns:(e + 1) * ns].cpu().numpy(), ex["gate"][1].ravel())
        ndc = w.H * w.F // 2
        assert np.array_equal(dl.down[0][e * ndc:(e + 1) * ndc].cpu().numpy(), ex["down"][0].ravel())


def test_tiny_layer():
    layer_parity(G.WORKLOADS["tiny"], n_tokens=4)


def test_tiny_layer_ordered_topk():
    layer_parity(G.WORKLOADS["tiny"], n_tokens=2, adjacent=True)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_edge_shapes(name):
    layer_parity(SMALL[name], n_tokens=2)


def test_k3_batch1_layer():
    layer_parity(G.WORKLOADS["k3_batch1"], n_tokens=2)


def test_k3_batch1_ordered_topk():
    layer_parity(G.WORKLOADS["k3_batch1"], n_tokens=1, adjacent=True)


def test_k3_tp16_slice_layer():
    layer_parity(G.WORKLOADS["k3_tp16_slice"], n_tokens=2)
    release_device_layers()


def test_router_topk_and_logits():
    t = torch()
    for name in ("tiny", "k3_batch1"):
        w = G.WORKLOADS[name]
        dl = device_layer(w, 0)
        (d, x), = pick_tokens(w, dl.router_host, 1, start=100)
        xd = dev_u16(x.reshape(1, -1))
        idx = t.empty((1, w.k), dtype=t.int32, device="cuda")
        wts = t.empty((1, w.k), dtype=t.float32, device="cuda")
        logits = t.empty((1, w.E), dtype=t.float32, device="cuda")
        ws = workspace(w, 1)
        M.router_topk(shape_of(w), xd, dl.router, 1, idx, wts, logits, ws)
        t.cuda.synchronize()
        L = O.router_logits(x, dl.router_host)
        ref_idx = O.topk_select(L, w.k)
        np.testing.assert_allclose(logits.cpu().numpy(), L, rtol=0, atol=1e-4)
        check_topk(idx.cpu().numpy(), {"logits": L, "idx": ref_idx}, w.k)
        np.testing.assert_allclose(wts.cpu().numpy(), O.topk_weights(L, ref_idx), atol=2e-6)


def test_expert_gateup_matches_oracle_activation():
    t = torch()
    w = G.WORKLOADS["k3_batch1"]
    dl = device_layer(w, 0)
    hx = G.HostExperts(w, 0)
    x = G.token(w, 7)
    sel = np.array([[3, 895, 0, 511] + list(range(100, 112))], dtype=np.int32)
    act = t.empty((1, w.k, w.F), dtype=t.float32, device="cuda")
    ws = workspace(w, 1)
    M.expert_gateup(shape_of(w), weights_of(dl), dev_u16(x.reshape(1, -1)),
                    t.from_numpy(sel).cuda(), 1, act, ws)
    t.cuda.synchronize()
    a = act.cpu().numpy()[0]
    xf = O.bf16_to_f64(x)
    for j in (0, 1, 2, 3, 15):
        ref = O.expert_activation(xf, hx.routed(int(sel[0, j])))
        rms = np.sqrt((ref ** 2).mean())
        assert np.abs(a[j] - ref).max() <= 1e-4 * rms, (j, np.abs(a[j] - ref).max(), rms)


def test_zero_activation_ties_pick_lowest_experts():
    """x = 0: every logit is 0, so experts 0..k-1 win with weight 1/k, the
    expert outputs vanish and out equals the residual exactly."""
    t = torch()
    w = G.WORKLOADS["tiny"]
    dl = device_layer(w, 0)
    x = np.zeros(w.H, np.uint16)
    r = G.token(w, 3)
    out, idx, wts = run_layer(w, dl, x, residual=dev_u16(r.reshape(1, -1)))
    assert idx[0].tolist() == list(range(w.k))
    np.testing.assert_array_equal(wts[0], np.full(w.k, 1.0 / w.k, np.float32))
    np.testing.assert_array_equal(out, r)


def _router_entry(w, dl, x):
    t = torch()
    idx = t.empty((1, w.k), dtype=t.int32, device="cuda")
    wts = t.empty((1, w.k), dtype=t.float32, device="cuda")
    ws = workspace(w, 1)
    M.router_topk(shape_of(w), dev_u16(x.reshape(1, -1)), dl.router, 1, idx, wts, None, ws)
    t.cuda.synchronize()
    return idx.cpu().numpy(), wts.cpu().numpy()


def test_all_logits_equal_with_many_experts():
    """x = 0 with E = 896: all 896 logits tie, far more than one wave's
    candidate list holds, so the block selection runs; it must still pick
    experts 0..k-1 with weight 1/k, in both entry points."""
    w = G.WORKLOADS["k3_batch1"]
    dl = device_layer(w, 0)
    x = np.zeros(w.H, np.uint16)
    out, idx, wts = run_layer(w, dl, x)
    assert idx[0].tolist() == list(range(w.k))
    np.testing.assert_array_equal(wts[0], np.full(w.k, 1.0 / w.k, np.float32))
    ridx, rwts = _router_entry(w, dl, x)
    assert ridx[0].tolist() == list(range(w.k))
    np.testing.assert_array_equal(rwts[0], np.full(w.k, 1.0 / w.k, np.float32))


@pytest.mark.parametrize("copies", [20, 70])
def test_duplicated_top_router_row(copies):
    """The router row of the token's best expert is copied into `copies`
    other rows, so that many logits tie exactly at the top: the selection is
    the lowest-indexed k of them (20 copies: the one-wave selection; 70: more
    ties than it holds, the block selection).  Checked against the oracle's
    exact selection in both entry points."""
    w = G.WORKLOADS["k3_batch1"]
    dl = device_layer(w, 0)
    try:
        x = G.token(w, 11)
        R = dl.router_host.copy()
        L0 = O.router_logits(x, R)
        best = int(np.argmax(L0))
        rng = np.random.default_rng(copies)
        others = rng.choice([e for e in range(w.E) if e != best], copies, replace=False)
        R[others] = R[best]
        dl.router.copy_(dev_u16(R))
        dl.router_host = R
        L = O.router_logits(x, R)
        ref = O.topk_select(L, w.k)
        ref_w = O.topk_weights(L, ref)[0]
        ref = [int(e) for e in ref[0]]
        out, idx, wts = run_layer(w, dl, x)
        assert idx[0].tolist() == ref, (idx[0].tolist(), ref)
        np.testing.assert_allclose(wts[0], ref_w, atol=2e-6)
        ridx, rwts = _router_entry(w, dl, x)
        assert ridx[0].tolist() == ref
        np.testing.assert_allclose(rwts[0], ref_w, atol=2e-6)
    finally:
        device_layer.cache_clear()


def test_no_residual_and_in_place_output():
    t = torch()
    w = G.WORKLOADS["tiny"]
    dl = device_layer(w, 0)
    (d, x), = pick_tokens(w, dl.router_host, 1, start=50)
    r_bits = G.token(w, 999)
    ref0 = oracle_layer(w, 0, dl.router_host, x, None)
    ref1 = oracle_layer(w, 0, dl.router_host, x, r_bits)
    xd = dev_u16(x.reshape(1, -1))
    ws = workspace(w, 1)
    out = t.empty_like(xd)
    M.decode_layer(shape_of(w), weights_of(dl), xd, None, out, 1, None, None, ws)
    res = dev_u16(r_bits.reshape(1, -1))
    M.decode_layer(shape_of(w), weights_of(dl), xd, res, res, 1, None, None, ws)  # in place
    t.cuda.synchronize()
    assert max_err_ratio(host_u16(out), ref0["out"])[0] <= TOL
    assert max_err_ratio(host_u16(res), ref1["out"])[0] <= TOL


def test_far_logit_weight_is_exactly_zero():
    """k = E with one router row pushed 110+ below the rest: its softmax weight
    underflows to exactly 0 in fp32."""
    t = torch()
    w = G.Workload("far", T=1, H=512, E=8, k=8, F=256, S=0, Fs=0, seed=0x5EED0107)
    dl = device_layer(w, 0)
    x = G.token(w, 0)
    xf = O.bf16_to_f64(x)
    R = O.bf16_to_f64(dl.router_host).copy()
    R[5] = -np.sign(xf) * 2.0            # logit(5) = -2 * sum|x| ~ -800
    rb = O.f64_to_bf16(R)
    dl.router.copy_(dev_u16(rb))
    dl.router_host = rb
    out, idx, wts = run_layer(w, dl, x)
    j = idx[0].tolist().index(5)
    assert wts[0, j] == 0.0
    ref = oracle_layer(w, 0, rb, x, x)
    assert max_err_ratio(out, ref["out"])[0] <= TOL
    device_layer.cache_clear()


def test_deterministic_and_poison_proof():
    """Two calls give identical bits; filling the scratch part of the
    workspace with NaN bytes and the output with garbage before a call
    changes nothing (no read of unwritten data)."""
    t = torch()
    w = G.WORKLOADS["k3_tp16_slice"]
    dl = device_layer(w, 0)
    (d, x), = pick_tokens(w, dl.router_host, 1, start=10)
    xd = dev_u16(x.reshape(1, -1))
    ws = workspace(w, 1)
    outs = []
    for poison in (False, True, True):
        out = t.full_like(xd, 0x7FC0 if poison else 0)
        if poison:
            ws[M_COUNTER:].fill_(0xFF)
        M.decode_layer(shape_of(w), weights_of(dl), xd, xd, out, 1, None, None, ws)
        t.cuda.synchronize()
        outs.append(host_u16(out).copy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    release_device_layers()


M_COUNTER = 256  # MOE_WS_COUNTER_BYTES


@pytest.mark.parametrize("name", ["wide_f", "f8192"])
def test_cross_workgroup_combine_deterministic_and_poison_proof(name):
    """FFN 4096 and 8192 take the down kernel whose row chunks are combined
    across workgroups (counter per chunk).  Repeated calls with the scratch
    part of the workspace poisoned before each give identical bits, match
    the oracle, and leave the counters at zero."""
    t = torch()
    w = SMALL[name]
    dl = device_layer(w, 0)
    (d, x), = pick_tokens(w, dl.router_host, 1, start=20)
    xd = dev_u16(x.reshape(1, -1))
    ws = workspace(w, 1)
    outs = []
    for poison in (False, True, True):
        out = t.full_like(xd, 0x7FC0 if poison else 0)
        if poison:
            ws[M_COUNTER:].fill_(0xFF)
        M.decode_layer(shape_of(w), weights_of(dl), xd, xd, out, 1, None, None, ws)
        t.cuda.synchronize()
        outs.append(host_u16(out).copy())
        assert not ws[:M_COUNTER].any().item(), "counters not left at zero"
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    ref = oracle_layer(w, 0, dl.router_host, x, x)
    assert max_err_ratio(outs[0], ref["out"])[0] <= TOL


@pytest.mark.parametrize("name", ["tiny", "k3_batch1", "wide_f", "fs_wide_f"])
def test_graph_replay_matches_eager(name):
    """One layer captured in a HIP graph, replayed with new inputs copied in
    between; every replay equals the eager call on the same input, and the
    workspace's counter head is left at zero (wide_f: the down rows are
    combined across workgroups through those counters)."""
    t = torch()
    w = SMALL[name] if name in SMALL else G.WORKLOADS[name]
    dl = device_layer(w, 0)
    toks = [x for _, x in pick_tokens(w, dl.router_host, 4, start=200)]
    ws = workspace(w, 1)
    x = dev_u16(toks[0].reshape(1, -1))
    out = t.empty_like(x)
    eager = []
    for tk in toks:
        x.copy_(dev_u16(tk.reshape(1, -1)))
        M.decode_layer(shape_of(w), weights_of(dl), x, x, out, 1, None, None, ws)
        t.cuda.synchronize()
        eager.append(host_u16(out).copy())
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        M.decode_layer(shape_of(w), weights_of(dl), x, x, out, 1, None, None, ws)
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        M.decode_layer(shape_of(w), weights_of(dl), x, x, out, 1, None, None, ws)
    for rep in range(3):
        for i, tk in enumerate(toks):
            x.copy_(dev_u16(tk.reshape(1, -1)))
            out.zero_()
            g.replay()
            t.cuda.synchronize()
            assert np.array_equal(host_u16(out), eager[i]), (rep, i)
    assert not ws[:M_COUNTER].any().item(), "counters not left at zero"
