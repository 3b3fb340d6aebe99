"""The seeded input generators (CPU): published SplitMix64 outputs, byte
ranges, slice consistency and bfloat16 rounding of drawn values."""
import os

import numpy as np
import pytest

import moe_inputs as G

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_outputs():
    # first outputs of SplitMix64 seeded with 0 (Vigna's splitmix64.c)
    w = G.splitmix64_words(0, 0, 3)
    assert [int(v) for v in w] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                   0x06C45D188009454F]


def test_counter_based_slices_agree():
    full = G.splitmix64_words(12345, 0, 1000)
    assert np.array_equal(G.splitmix64_words(12345, 400, 100), full[400:500])
    cb = G.code_bytes(777, 0, 8 * 50)
    assert np.array_equal(G.code_bytes(777, 80, 160), cb[80:240])


def test_code_and_scale_byte_distributions():
    cb = G.code_bytes(G.stream_key(1, 0, "gate_codes"), 0, 1 << 16)
    nib = np.concatenate([cb & 15, cb >> 4])
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.9 * len(nib) / 16
    sb = G.scale_bytes(G.stream_key(1, 0, "gate_scales"), 0, 50000)
    assert sb.min() == 119 and sb.max() == 123
    assert np.bincount(sb - 119).min() > 9000


def test_stream_keys_distinct():
    keys = {G.stream_key(s, l, t) for s in (1, 2) for l in range(3) for t in G.TENSOR}
    assert len(keys) == 2 * 3 * len(G.TENSOR)


def test_generator_bf16_rounding_hand_cases():
    rows = []
    with open(os.path.join(GOLDEN, "bf16_rne.txt")) as f:
        for line in f:
            p = line.split("#")[0].split()
            if p:
                v = p[0]
                rows.append((float(v) if v in ("nan", "inf", "-inf") else float.fromhex(v),
                             int(p[1], 16)))
    got = G.bf16_from_f64(np.array([v for v, _ in rows]))
    assert [int(g) for g in got] == [want for _, want in rows]


def test_host_expert_is_slice_of_full_stream():
    w = G.WORKLOADS["tiny"]
    hx = G.HostExperts(w, 0)
    e3 = hx.routed(3)
    nc = w.F * w.H // 2
    full = G.code_bytes(G.stream_key(w.seed, 0, "gate_codes"), 0, w.E * nc)
    assert np.array_equal(e3["gate"][0].ravel(), full[3 * nc:4 * nc])
    assert e3["down"][0].shape == (w.H, w.F // 2)
    assert e3["down"][1].shape == (w.H, w.F // 32)


def test_zipf_scales_skew_loads():
    a = G.zipf_row_scales(896, 16, 1.1, 3)
    assert a.shape == (896,) and np.all(a > 0)
    assert a.max() / np.median(a) > 3


def test_verify_tokens_are_correlated_within_a_sequence():
    """k3_verify8 draws: tokens of one sequence (draw // T) have correlation
    close to the workload's rho, tokens of different sequences close to 0."""
    w = G.WORKLOADS["k3_verify8"]
    xs = np.stack([(G.token(w, d).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                   for d in range(2 * w.T)])
    c = np.corrcoef(xs)
    same = [c[i, j] for i in range(w.T) for j in range(w.T) if i < j]
    cross = [c[i, j] for i in range(w.T) for j in range(w.T, 2 * w.T)]
    assert abs(np.mean(same) - w.corr) < 0.03, np.mean(same)
    assert abs(np.mean(cross)) < 0.03, np.mean(cross)
