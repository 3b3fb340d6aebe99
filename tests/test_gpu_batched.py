"""GPU parity of the batched decode path (2 <= T <= 64 tokens) against the
fp64 oracle, through the C ABI.

Bars as for one token: top-k sets exact where the oracle's k-th/(k+1)-th
logit gap exceeds 1e-3 (order exact where every adjacent gap among the top
k+1 does), max-abs-error <= 2e-2 * rms(reference) per token; grouping
bit-exact.  Softmax weights: |dw| <= 2e-6 + 1e-4 w, since a weight's relative
error is at most twice the largest logit error and the Zipf-scaled router
rows reach |logit| ~ 50, where fp32 accumulation over H = 7168 terms leaves
logit errors of a few 1e-5.
"""
import numpy as np
import pytest

from gpu_helpers import (GAP, TOL, G, M, O, check_topk, dev_u16, device_layer, host_u16,
                         max_err_ratio, oracle_layer, pick_tokens, pmap, release_device_layers,
                         shape_of, torch, weights_of, workspace)

pytestmark = pytest.mark.gpu
W_RTOL = 1e-4

SMALL = {
    "tiny": G.WORKLOADS["tiny"],
    "ragged_shared": G.Workload("ragged_shared", T=1, H=768, E=40, k=5, F=256, S=1, Fs=256,
                                seed=0x5EED0201),
    "kmax": G.Workload("kmax_b", T=1, H=1024, E=32, k=32, F=512, S=1, Fs=512, seed=0x5EED0202),
    "k1_f128": G.Workload("k1_f128", T=1, H=512, E=16, k=1, F=128, S=1, Fs=128, seed=0x5EED0203),
    # the largest hidden size: the gate/up chunk loop unrolled for 16 chunks
    "h8192": G.Workload("h8192_b", T=1, H=8192, E=16, k=2, F=256, S=1, Fs=256, seed=0x5EED0204),
    # the most experts and the largest top-k the library accepts together
    "emax": G.Workload("emax_b", T=1, H=512, E=1024, k=32, F=128, S=1, Fs=128, seed=0x5EED0205),
    # a shared expert of its own width: its gate/up and down run as passes of
    # their own (each pairing of down kernels: generic/generic, the FFN-2048
    # stream for the routed experts, the FFN-2048 stream for the shared one)
    "fs_wide": G.Workload("fs_wide_b", T=1, H=1024, E=24, k=4, F=256, S=1, Fs=512, seed=0x5EED0206),
    "fs_narrow": G.Workload("fs_narrow_b", T=1, H=2048, E=16, k=3, F=1024, S=1, Fs=128,
                            seed=0x5EED0207),
    "fs_routed_2048": G.Workload("fs_routed_2048", T=1, H=1024, E=12, k=2, F=2048, S=1, Fs=256,
                                 seed=0x5EED0208),
    "fs_shared_2048": G.Workload("fs_shared_2048", T=1, H=768, E=20, k=3, F=256, S=1, Fs=2048,
                                 seed=0x5EED0209),
    # an expert count that is not a multiple of four: the top-k kernel then
    # requests the router's partial sums one expert at a time
    "odd_e": G.Workload("odd_e_b", T=1, H=512, E=37, k=5, F=256, S=1, Fs=256, seed=0x5EED020A),
    # top-16, the case whose combine requests every slot's rows at once: with
    # and without a shared expert
    "k16_shared": G.Workload("k16_shared_b", T=1, H=512, E=40, k=16, F=256, S=1, Fs=256,
                             seed=0x5EED020B),
    "k16_noshared": G.Workload("k16_noshared_b", T=1, H=512, E=40, k=16, F=256, S=0, Fs=0,
                               seed=0x5EED020C),
}


def tokens_of(w, dl, T, start=0, adjacent=False):
    picked = pick_tokens(w, dl.router_host, T, start=start, adjacent=adjacent)
    return np.stack([x for _, x in picked])


def run_batched(w, dl, X, residual="x"):
    t = torch()
    T = X.shape[0]
    x = dev_u16(X)
    out = t.empty_like(x)
    idx = t.empty((T, w.k), dtype=t.int32, device="cuda")
    wts = t.empty((T, w.k), dtype=t.float32, device="cuda")
    ws = workspace(w, T)
    res = x if residual == "x" else residual
    M.decode_layer(shape_of(w), weights_of(dl), x, res, out, T, idx, wts, ws)
    t.cuda.synchronize()
    return host_u16(out), idx.cpu().numpy(), wts.cpu().numpy()


def batched_parity(w, T, sample=None, start=0):
    dl = device_layer(w, 0)
    X = tokens_of(w, dl, T, start=start)
    out, idx, wts = run_batched(w, dl, X)
    rows = list(range(T)) if sample is None else sample
    ref = oracle_layer(w, 0, dl.router_host, X[rows], X[rows])
    check_topk(idx[rows], ref, w.k)
    np.testing.assert_allclose(wts[rows], ref["w"], rtol=W_RTOL, atol=2e-6)
    np.testing.assert_allclose(wts.sum(axis=1), 1.0, atol=1e-5)
    err = max_err_ratio(out[rows], ref["out"])
    print(f"{w.name} T={T} tokens checked={len(rows)} max_err/rms={err.max():.3e}")
    assert err.max() <= TOL, (w.name, T, err.max())
    return X, out, idx


@pytest.mark.parametrize("E,k,T", [(896, 16, 64), (32, 4, 5), (16, 1, 2), (1024, 32, 64),
                                   (7, 3, 17), (40, 5, 33)])
def test_group_by_expert_is_exact(E, k, T):
    t = torch()
    rng = np.random.default_rng(E * 1000 + k * 10 + T)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    offsets = t.empty(E + 1, dtype=t.int32, device="cuda")
    pairs = t.empty(T * k, dtype=t.int32, device="cuda")
    ws = t.zeros(1 << 20, dtype=t.uint8, device="cuda")
    M.group_by_expert(t.from_numpy(idx).cuda(), T, k, E, offsets, pairs, ws)
    t.cuda.synchronize()
    ref_off, ref_pairs = O.group_by_expert(idx, E)
    assert np.array_equal(offsets.cpu().numpy(), ref_off)
    assert np.array_equal(pairs.cpu().numpy(), ref_pairs)
    assert not ws[:M_COUNTER].any().item(), "grouping wrote into the counter head"


M_COUNTER = 256  # MOE_WS_COUNTER_BYTES


def test_grouping_then_wide_layer_on_one_workspace():
    """A grouping call followed by single-token layers on the same
    workspace: the layer at FFN 4096 combines its down rows across
    workgroups through the counter head, which the grouping must leave at
    zero."""
    from test_gpu_layer import SMALL as LAYER_SMALL, run_layer_ws
    t = torch()
    w = LAYER_SMALL["wide_f"]
    dl = device_layer(w, 0)
    ws = workspace(w, 64)
    rng = np.random.default_rng(5)
    idx = np.stack([rng.permutation(w.E)[:w.k] for _ in range(64)]).astype(np.int32)
    offsets = t.empty(w.E + 1, dtype=t.int32, device="cuda")
    pairs = t.empty(64 * w.k, dtype=t.int32, device="cuda")
    M.group_by_expert(t.from_numpy(idx).cuda(), 64, w.k, w.E, offsets, pairs, ws)
    t.cuda.synchronize()
    assert not ws[:M_COUNTER].any().item()
    for d, x in pick_tokens(w, dl.router_host, 2, start=40):
        out, gidx, _ = run_layer_ws(w, dl, x, ws)
        ref = oracle_layer(w, 0, dl.router_host, x, x)
        check_topk(gidx, ref, w.k)
        err = max_err_ratio(out, ref["out"])[0]
        assert err <= TOL, (d, err)
    assert not ws[:M_COUNTER].any().item()


@pytest.mark.parametrize("name,T", [("tiny", 5), ("k3_batch64_zipf", 64)])
def test_router_topk_batched(name, T):
    t = torch()
    w = G.WORKLOADS[name]
    dl = device_layer(w, 0)
    X = tokens_of(w, dl, T, start=300)
    idx = t.empty((T, w.k), dtype=t.int32, device="cuda")
    wts = t.empty((T, w.k), dtype=t.float32, device="cuda")
    logits = t.empty((T, w.E), dtype=t.float32, device="cuda")
    ws = workspace(w, T)
    M.router_topk(shape_of(w), dev_u16(X), dl.router, T, idx, wts, logits, ws)
    t.cuda.synchronize()
    Lr = O.router_logits(X, dl.router_host)
    ref_idx = O.topk_select(Lr, w.k)
    np.testing.assert_allclose(logits.cpu().numpy(), Lr, rtol=1e-5, atol=1e-4)
    assert check_topk(idx.cpu().numpy(), {"logits": Lr, "idx": ref_idx}, w.k) == T
    np.testing.assert_allclose(wts.cpu().numpy(), O.topk_weights(Lr, ref_idx), rtol=W_RTOL,
                               atol=2e-6)


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("T", [2, 5, 12, 17, 64])  # 12: one pass per group above 8 tokens
def test_batched_small_shapes(name, T):
    batched_parity(SMALL[name], T)


@pytest.mark.parametrize("name", ["ragged_shared", "k16_shared", "k16_noshared"])
def test_batched_no_residual_and_in_place_output(name):
    """Residual absent (the combine adds none), then the residual buffer as
    the output (in place); both against the oracle."""
    t = torch()
    w = SMALL[name]
    T = 5
    dl = device_layer(w, 0)
    X = tokens_of(w, dl, T, start=30)
    R = np.stack([G.token(w, 900 + i) for i in range(T)])
    ref0 = oracle_layer(w, 0, dl.router_host, X, None)
    ref1 = oracle_layer(w, 0, dl.router_host, X, R)
    x = dev_u16(X)
    ws = workspace(w, T)
    out = t.empty_like(x)
    M.decode_layer(shape_of(w), weights_of(dl), x, None, out, T, None, None, ws)
    res = dev_u16(R)
    M.decode_layer(shape_of(w), weights_of(dl), x, res, res, T, None, None, ws)  # in place
    t.cuda.synchronize()
    o0, o1 = host_u16(out), host_u16(res)
    for i in range(T):
        assert max_err_ratio(o0[i], ref0["out"][i])[0] <= TOL, (name, i)
        assert max_err_ratio(o1[i], ref1["out"][i])[0] <= TOL, (name, i)


@pytest.mark.parametrize("name", ["ragged_shared", "h8192"])
def test_identical_tokens_fill_every_group(name):
    """64 copies of one token: every selected expert's group holds the whole
    batch (four 16-token passes per expert).  Each token's column goes
    through the same arithmetic, so all 64 outputs, indices and weights are
    bit-identical; the first row meets the oracle."""
    w = SMALL[name]
    dl = device_layer(w, 0)
    X = np.repeat(tokens_of(w, dl, 1, start=3), 64, axis=0)
    out, idx, wts = run_batched(w, dl, X)
    assert (out == out[0]).all() and (idx == idx[0]).all() and (wts == wts[0]).all()
    ref = oracle_layer(w, 0, dl.router_host, X[:1], X[:1])
    check_topk(idx[:1], ref, w.k)
    err = max_err_ratio(out[:1], ref["out"])
    assert err.max() <= TOL, err.max()


def test_k3_batch64_zipf_layer():
    """The K3-shaped layer at batch 64 with Zipf-skewed routing: every
    token's top-k, weights and output against the oracle."""
    w = G.WORKLOADS["k3_batch64_zipf"]
    X, out, idx = batched_parity(w, 64)
    counts = np.bincount(idx.ravel(), minlength=w.E)
    print(f"touched experts {int((counts > 0).sum())}, max tokens per expert {counts.max()}")
    dl = device_layer(w, 0)
    Lr = O.router_logits(X, dl.router_host)
    assert check_topk(idx, {"logits": Lr, "idx": O.topk_select(Lr, w.k)}, w.k) == 64


def test_k3_verify8_layer():
    """The speculative-decode verify shape: one sequence's token and seven
    drafts (correlated activations, overlapping routing) through the
    K3-shaped layer; every token against the oracle."""
    w = G.WORKLOADS["k3_verify8"]
    X, out, idx = batched_parity(w, 8)
    n = len(np.unique(idx))
    print(f"distinct experts {n} of {8 * w.k} slots")
    assert n < 8 * w.k  # the drafts share experts


def test_batch_matches_single_token_calls():
    """Token t of a T = 64 call agrees with a T = 1 call on the same token:
    same experts, outputs within the layer tolerance of each other."""
    t = torch()
    w = G.WORKLOADS["k3_batch64_zipf"]
    dl = device_layer(w, 0)
    X = tokens_of(w, dl, 64, start=500)
    out_b, idx_b, _ = run_batched(w, dl, X)
    for ti in (0, 17, 63):
        x1 = dev_u16(X[ti:ti + 1])
        o1 = t.empty_like(x1)
        i1 = t.empty((1, w.k), dtype=t.int32, device="cuda")
        M.decode_layer(shape_of(w), weights_of(dl), x1, x1, o1, 1, i1, None, workspace(w, 1))
        t.cuda.synchronize()
        assert idx_b[ti].tolist() == i1.cpu().numpy()[0].tolist()
        a = O.bf16_to_f64(out_b[ti])
        b = O.bf16_to_f64(host_u16(o1)[0])
        assert np.abs(a - b).max() <= TOL * np.sqrt((b * b).mean())
    release_device_layers()


@pytest.mark.parametrize("name,T", [("ragged_shared", 8), ("fs_narrow", 8), ("k3_verify8", 8),
                                    ("fs_routed_2048", 40), ("k3_verify8", 40)])
def test_batched_graph_replay_matches_eager(name, T):
    """A batched layer captured in a HIP graph and replayed with new inputs
    copied in between equals the eager call bit for bit, every replay.  At
    the K3 shape this covers the unrolled gate/up and the unit-stream down
    kernels; the small shapes the generic loops.  Above 16 tokens: the
    two-tile gate/up passes and the down kernel's pass tables (written by
    the grouping kernel in every call)."""
    t = torch()
    w = SMALL[name] if name in SMALL else G.WORKLOADS[name]
    dl = device_layer(w, 0)
    batches = [tokens_of(w, dl, T, start=1000 + 50 * i) for i in range(3)]
    ws = workspace(w, T)
    x = dev_u16(batches[0])
    out = t.empty_like(x)
    eager = []
    for B in batches:
        x.copy_(dev_u16(B))
        M.decode_layer(shape_of(w), weights_of(dl), x, x, out, T, None, None, ws)
        t.cuda.synchronize()
        eager.append(host_u16(out).copy())
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        M.decode_layer(shape_of(w), weights_of(dl), x, x, out, T, None, None, ws)
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        M.decode_layer(shape_of(w), weights_of(dl), x, x, out, T, None, None, ws)
    for rep in range(3):
        for i, B in enumerate(batches):
            x.copy_(dev_u16(B))
            out.zero_()
            g.replay()
            t.cuda.synchronize()
            assert np.array_equal(host_u16(out), eager[i]), (rep, i)
    release_device_layers()


def test_batched_stack_teacher_forced():
    """Three stacked small layers at T = 6 (RMSNorm -> MoE -> residual): each
    layer checked against the oracle fed the GPU's own input."""
    t = torch()
    w = G.Workload("stack_b", T=6, H=768, E=40, k=5, F=256, S=1, Fs=256, L=3, seed=0x5EED0204)
    layers = [G.DeviceLayer(w, l) for l in range(w.L)]
    X = np.stack([G.token(w, d) for d in range(w.T)])
    hidden = dev_u16(X)
    trace = t.empty((w.L, w.T, w.H), dtype=t.int16, device="cuda")
    idx = t.empty((w.L, w.T, w.k), dtype=t.int32, device="cuda")
    ws = workspace(w, w.T)
    M.decode_stack(shape_of(w), [weights_of(dl) for dl in layers], [dl.gamma for dl in layers],
                   w.eps, hidden, w.T, idx, trace, ws)
    t.cuda.synchronize()
    tr = host_u16(trace)
    gi = idx.cpu().numpy()
    ol = []
    for l, dl in enumerate(layers):
        hx = G.HostExperts(w, l)
        ol.append(dict(router=dl.router_host, gamma=dl.gamma_host, k=w.k, routed=hx.routed,
                       shared=hx.shared()))
    teacher = [X] + [tr[l] for l in range(w.L - 1)]
    recs = O.moe_stack(X, ol, w.eps, teacher=teacher, pmap=pmap)
    for l, r in enumerate(recs):
        check_topk(gi[l], r, w.k)
        err = max_err_ratio(tr[l], r["out"]).max()
        print(f"layer {l}: max_err/rms={err:.3e}")
        assert err <= TOL, (l, err)
