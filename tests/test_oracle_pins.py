"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test checks the oracle against something it does not compute itself:
hand-worked format tables (tests/golden/), brute force on tiny inputs with a
different method, closed forms and invariants of the layer.  A plausible
slip in the oracle (wrong nibble order, transposed operand, sum instead of
mean, softmax over all experts, wrong tie-break, residual taken from the
normalised input, ...) fails at least one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_num(s):
    s = s.strip()
    if s in ("nan", "inf", "-inf", "+inf"):
        return float(s)
    if "0x" in s:
        return float.fromhex(s)
    return float(s)


def _formats():
    e2m1, e8m0, worked = {}, {}, []
    with open(os.path.join(GOLDEN, "mxfp4_formats.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if not line:
                continue
            if line[0] == "e2m1":
                e2m1[int(line[1], 16)] = _parse_num(line[3])
            elif line[0] == "e8m0":
                e8m0[int(line[1], 16)] = _parse_num(line[2])
            elif line[0] == "byte":
                worked.append((int(line[1], 16), int(line[2], 16),
                               _parse_num(line[3]), _parse_num(line[4])))
    return e2m1, e8m0, worked


def _same(a, b):
    """Equal including the sign of zero, NaN == NaN."""
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


# ------------------------------------------------------------ MXFP4 decode

def test_e2m1_table_matches_hand_table():
    e2m1, _, _ = _formats()
    assert len(e2m1) == 16
    for c in range(16):
        assert _same(O.E2M1[c], e2m1[c]), (c, O.E2M1[c], e2m1[c])


def test_e8m0_matches_hand_values():
    _, e8m0, _ = _formats()
    for b, v in e8m0.items():
        assert _same(float(O.e8m0_value(b)), v), (hex(b), O.e8m0_value(b), v)


def test_mx_decode_all_codes_times_all_listed_scales():
    e2m1, e8m0, _ = _formats()
    scales_b = [0x77, 0x7B, 0x7F, 0x80]
    # one row per scale byte; 32 elements: codes 0..15 then 15..0
    elems = list(range(16)) + list(range(15, -1, -1))
    codes = np.array([[elems[2 * i] | (elems[2 * i + 1] << 4) for i in range(16)]
                      for _ in scales_b], dtype=np.uint8)
    scales = np.array([[s] for s in scales_b], dtype=np.uint8)
    M = O.mx_decode(codes, scales)
    for r, s in enumerate(scales_b):
        for j, c in enumerate(elems):
            assert _same(M[r, j], e2m1[c] * e8m0[s]), (r, j)


def test_mx_decode_worked_bytes():
    _, _, worked = _formats()
    for byte, scale, v0, v1 in worked:
        codes = np.full((1, 16), 0, dtype=np.uint8)
        codes[0, 0] = byte
        M = O.mx_decode(codes, np.array([[scale]], dtype=np.uint8))
        assert _same(M[0, 0], v0) and _same(M[0, 1], v1), (hex(byte), M[0, :2])


def test_block_dot_closed_forms():
    # 16 bytes 0x22 (all elements 1.0) at 2^-4, dotted with ones: 32 * 2^-4 = 2
    M = O.mx_decode(np.full((1, 16), 0x22, np.uint8), np.array([[0x7B]], np.uint8))
    assert M @ np.ones(32) == pytest.approx(2.0, abs=0)
    # 16 bytes 0x71 (0.5 and 6.0) at 2^0: 16 * 6.5 = 104
    M = O.mx_decode(np.full((1, 16), 0x71, np.uint8), np.array([[0x7F]], np.uint8))
    assert (M @ np.ones(32))[0] == 104.0


def test_mx_decode_indexing_one_hot():
    """Hand-placed nibbles land at hand-computed (row, column) positions:
    pins nibble order, byte index, block index and row-major layout."""
    R, C = 4, 64
    codes = np.zeros((R, C // 2), np.uint8)
    scales = np.full((R, C // 32), 0x7F, np.uint8)
    codes[2, 5] = 0x70      # byte 5 high nibble -> element 11 = 6.0
    scales[2, 1] = 0x80     # block 1 (elements 32..63) of row 2 scaled by 2
    codes[2, 20] = 0x02     # byte 20 low nibble -> element 40 = 1.0 * 2
    codes[3, 31] = 0x0B     # byte 31 low nibble -> element 62 = -1.5
    M = O.mx_decode(codes, scales)
    expect = np.zeros((R, C))
    expect[2, 11] = 6.0
    expect[2, 40] = 2.0
    expect[3, 62] = -1.5
    assert np.array_equal(M, expect)
    x = np.zeros(C)
    x[11] = 1.0
    assert np.array_equal(M @ x, [0, 0, 6.0, 0])   # G x picks column 11


# ------------------------------------------------------------- bfloat16

def test_bf16_rounding_hand_cases():
    rows = []
    with open(os.path.join(GOLDEN, "bf16_rne.txt")) as f:
        for line in f:
            p = line.split("#")[0].split()
            if p:
                rows.append((_parse_num(p[0]), int(p[1], 16)))
    assert len(rows) >= 18
    got = O.f64_to_bf16(np.array([v for v, _ in rows]))
    for (v, want), g in zip(rows, got):
        assert int(g) == want, (v.hex() if not math.isnan(v) else v, hex(g), hex(want))


def test_bf16_roundtrip_all_finite_patterns():
    """Every finite bfloat16 value decodes exactly and rounds back to itself."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_to_f64(bits)
    fin = np.isfinite(v)
    sample = bits[fin][::37]                     # keep the Python loop short
    back = O.f64_to_bf16(O.bf16_to_f64(sample))
    assert np.array_equal(back, sample)
    assert O.bf16_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert O.bf16_to_f64(np.array([0xC0C0], np.uint16))[0] == -6.0


# ------------------------------------------------------------------ router

def _bf16_of_ints(a):
    # small integers are exact in bf16: bits = upper half of the float32
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_router_logits_exact_integer_brute_force():
    rng = np.random.default_rng(1)
    T, E, H = 3, 5, 7                      # all different: catches transposes
    xi = rng.integers(-8, 9, (T, H))
    wi = rng.integers(-8, 9, (E, H))
    L = O.router_logits(_bf16_of_ints(xi), _bf16_of_ints(wi))
    assert L.shape == (T, E)
    for t in range(T):
        for e in range(E):
            want = sum(int(xi[t, h]) * int(wi[e, h]) for h in range(H))
            assert L[t, e] == want


def _brute_topk(l, k):
    """The unique k-subset whose members all beat every non-member under
    (logit desc, index asc), then ordered by that key."""
    E = len(l)
    beats = lambda a, b: l[a] > l[b] or (l[a] == l[b] and a < b)
    found = [S for S in itertools.combinations(range(E), k)
             if all(beats(a, b) for a in S for b in range(E) if b not in S)]
    assert len(found) == 1
    S = list(found[0])
    # order by number of members each one beats (a permutation of k-1..0)
    return sorted(S, key=lambda a: -sum(beats(a, b) for b in S))


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(2)
    for trial in range(60):
        E = int(rng.integers(1, 9))
        l = rng.integers(-3, 4, E).astype(np.float64)    # many exact ties
        for k in range(1, E + 1):
            got = O.topk_select(l[None, :], k)[0].tolist()
            assert got == _brute_topk(l, k), (l, k, got)


def test_topk_duplicate_router_rows_prefer_lower_index():
    rng = np.random.default_rng(3)
    H, E = 32, 6
    W = rng.integers(-4, 5, (E, H))
    W[4] = W[1]                                     # experts 1 and 4 tie
    x = rng.integers(-4, 5, (1, H))
    L = O.router_logits(_bf16_of_ints(x), _bf16_of_ints(W))
    assert L[0, 1] == L[0, 4]
    idx = O.topk_select(L, E)[0].tolist()
    assert idx.index(1) < idx.index(4)
    assert idx.index(1) + 1 == idx.index(4)


def test_topk_k_equals_E_is_a_full_sort():
    rng = np.random.default_rng(4)
    l = rng.standard_normal(20)
    got = O.topk_select(l[None, :], 20)[0].tolist()
    assert got == sorted(range(20), key=lambda e: (-l[e], e))


# ---------------------------------------------------------------- softmax

def test_combine_weights_sum_to_one_and_closed_forms():
    rng = np.random.default_rng(5)
    L = rng.standard_normal((4, 40)) * 3
    idx = O.topk_select(L, 7)
    w = O.topk_weights(L, idx)
    assert np.all(np.abs(w.sum(1) - 1) < 1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)          # descending logits
    # two selected experts: w1 = sigmoid(l1 - l2)
    l = np.array([[0.3, 2.0, -1.0]])
    w2 = O.topk_weights(l, O.topk_select(l, 2))[0]
    d = 2.0 - 0.3
    assert w2[0] == pytest.approx(1 / (1 + math.exp(-d)), rel=1e-15)
    # equal selected logits -> 1/k, and logits outside the top-k are ignored
    l = np.array([[5.0, 5.0, 5.0, -100.0, 1e3 * 0 + 4.0]])
    w3 = O.topk_weights(l, O.topk_select(l, 3))[0]
    assert np.all(w3 == 1 / 3)


def test_far_logit_gets_exactly_zero_weight():
    l = np.array([[0.0, -800.0, -1.0]])                # exp(-800) underflows
    idx = O.topk_select(l, 3)
    w = O.topk_weights(l, idx)[0]
    assert w[list(idx[0]).index(1)] == 0.0


# ------------------------------------------------- gaps that gate the checks
# Hand-worked vectors.  l = [3, 1, 4, 1.5, 9, 2.5] sorted descending is
# 9, 4, 3, 2.5, 1.5, 1, so the consecutive differences are 5, 1, 0.5, 1, 0.5.

HAND = np.array([3.0, 1.0, 4.0, 1.5, 9.0, 2.5])


def test_topk_gap_hand_worked():
    # k-th minus (k+1)-th largest: k = 1 -> 9 - 4, k = 2 -> 4 - 3, ...
    want = {1: 5.0, 2: 1.0, 3: 0.5, 4: 1.0, 5: 0.5}
    for k, g in want.items():
        assert O.topk_gap(HAND[None, :], k)[0] == g, k
    assert O.topk_gap(HAND[None, :], 6)[0] == np.inf      # k = E: no (k+1)-th
    # exact ties at the boundary give a zero gap; ties inside the top-k do not
    l = np.array([[2.0, 5.0, 5.0, 1.0]])
    assert O.topk_gap(l, 1)[0] == 0.0
    assert O.topk_gap(l, 2)[0] == 3.0
    assert O.topk_gap(l, 3)[0] == 1.0
    # per token, independent of the order of the experts
    rows = np.stack([HAND, HAND[::-1], np.roll(HAND, 2)])
    assert O.topk_gap(rows, 2).tolist() == [1.0, 1.0, 1.0]
    two = np.stack([HAND, np.array([0.0, 10.0, 9.75, -1.0, 3.0, 2.0])])
    assert O.topk_gap(two, 2).tolist() == [1.0, 6.75]


def test_adjacent_gaps_hand_worked():
    # smallest consecutive difference among the k+1 largest
    want = {1: 5.0, 2: 1.0, 3: 0.5, 4: 0.5, 5: 0.5}
    for k, g in want.items():
        assert O.adjacent_gaps(HAND[None, :], k)[0] == g, k
    # k = E: the ordering of all E logits matters, so all of them are compared
    assert O.adjacent_gaps(HAND[None, :], 6)[0] == 0.5
    # a close pair below the (k+1)-th logit is ignored ...
    l = np.array([[10.0, 8.0, 6.0, 5.9, 0.0]])
    assert O.adjacent_gaps(l, 1)[0] == 2.0
    assert O.adjacent_gaps(l, 2)[0] == 2.0
    assert O.adjacent_gaps(l, 3)[0] == pytest.approx(0.1, abs=1e-15)
    # ... but a close pair at the k-th / (k+1)-th boundary counts
    l = np.array([[10.0, 8.0, 7.99, -3.0]])
    assert O.adjacent_gaps(l, 2)[0] == pytest.approx(0.01, abs=1e-15)
    assert O.adjacent_gaps(l, 1)[0] == 2.0
    # ties inside the top k make the order ambiguous: zero gap
    assert O.adjacent_gaps(np.array([[2.0, 5.0, 5.0, 1.0]]), 1)[0] == 0.0
    # one expert: nothing to order
    assert O.adjacent_gaps(np.array([[1.5]]), 1)[0] == np.inf


def test_gaps_agree_with_brute_force_over_subsets():
    """topk_gap is the margin by which the chosen set wins: the smallest
    selected logit minus the largest unselected one.  adjacent_gaps is the
    smallest difference between any two of the k+1 largest logits (not only
    neighbours, which gives the same minimum).  Both from the brute-force
    top-k, which shares no code with the oracle's sort."""
    rng = np.random.default_rng(41)
    for _ in range(200):
        E = int(rng.integers(2, 9))
        l = rng.integers(-20, 21, E).astype(np.float64) / 4
        for k in range(1, E):
            S = _brute_topk(l, k)
            rest = [e for e in range(E) if e not in S]
            assert O.topk_gap(l[None, :], k)[0] == min(l[S]) - max(l[rest])
            S1 = _brute_topk(l, k + 1)
            want = min(abs(l[a] - l[b]) for a, b in itertools.combinations(S1, 2))
            assert O.adjacent_gaps(l[None, :], k)[0] == want


# ------------------------------------------------------------------ SiLU

def test_silu_textbook_identities():
    v = np.linspace(-30, 30, 1001)
    s = O.silu(v)
    assert np.allclose(s - O.silu(-v), v, rtol=0, atol=1e-13)  # x*sig(x)+x*sig(-x)=x
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert O.silu(np.array([1.0]))[0] == pytest.approx(0.7310585786300049, rel=1e-15)
    assert O.silu(np.array([-1000.0]))[0] == 0.0
    assert O.silu(np.array([1000.0]))[0] == 1000.0


# --------------------------------------------------- expert / layer forms

def _const_expert(H, F, code_byte, s_gu, s_d, s_u=None):
    s_u = s_gu if s_u is None else s_u
    return {"gate": (np.full((F, H // 2), code_byte, np.uint8), np.full((F, H // 32), s_gu, np.uint8)),
            "up": (np.full((F, H // 2), code_byte, np.uint8), np.full((F, H // 32), s_u, np.uint8)),
            "down": (np.full((H, F // 2), code_byte, np.uint8), np.full((H, F // 32), s_d, np.uint8))}


def test_expert_closed_form_all_ones():
    """All codes 0x22 (every element 1.0): g = u = 2^s sum(x),
    a = silu(g) g for every row, y[h] = 2^s' F a."""
    H, F = 64, 32
    rng = np.random.default_rng(6)
    x = rng.integers(-3, 4, H).astype(np.float64) / 4
    s_gu, s_d = 0x7B, 0x78              # 2^-4, 2^-7
    y = O.expert_ffn(x, _const_expert(H, F, 0x22, s_gu, s_d))
    g = 2.0 ** -4 * x.sum()
    a = g / (1 + math.exp(-g)) * g
    assert np.allclose(y, 2.0 ** -7 * F * a, rtol=1e-14, atol=0)
    # distinct gate and up scales: a = silu(g) * u is not symmetric in g, u
    y = O.expert_ffn(x, _const_expert(H, F, 0x22, 0x7B, s_d, s_u=0x7D))
    g, u = 2.0 ** -4 * x.sum(), 2.0 ** -2 * x.sum()
    assert np.allclose(y, 2.0 ** -7 * F * (g / (1 + math.exp(-g)) * u), rtol=1e-14, atol=0)


def test_expert_activation_closed_form():
    """The gated hidden vector alone: with every element 1.0, distinct gate
    and up scales and a different code per gate row, row f of a is
    silu(c_f 2^-4 sum x) * 2^-2 sum x.  Swapping gate and up (silu of the up
    projection), dropping the gating or mixing up rows fails."""
    H, F = 64, 32
    rng = np.random.default_rng(16)
    x = rng.integers(-3, 4, H).astype(np.float64) / 4
    while abs(x.sum()) < 1:
        x = rng.integers(-3, 4, H).astype(np.float64) / 4
    ex = _const_expert(H, F, 0x22, 0x7B, 0x78, s_u=0x7D)
    # gate row f: both nibbles code c in {0.5, 1, 1.5, 2} (codes 1, 2, 3, 4)
    codes = [0x11, 0x22, 0x33, 0x44]
    vals = [0.5, 1.0, 1.5, 2.0]
    g_codes = ex["gate"][0].copy()
    for f in range(F):
        g_codes[f, :] = codes[f % 4]
    ex["gate"] = (g_codes, ex["gate"][1])
    a = O.expert_activation(x, ex)
    s = x.sum()
    for f in range(F):
        g = vals[f % 4] * 2.0 ** -4 * s
        want = g / (1 + math.exp(-g)) * (2.0 ** -2 * s)
        assert a[f] == pytest.approx(want, rel=1e-14, abs=0), f


def test_expert_activation_brute_force_and_down_projection():
    """On random bytes: each row of a from scalar loops over the code bytes
    (values from the hand table in tests/golden/), and D a reproduces the
    expert output."""
    e2m1, e8m0, _ = _formats()
    H, F = 64, 32
    rng = np.random.default_rng(17)
    ex = _rand_expert(rng, H, F)
    table = np.array([0x77, 0x7B, 0x7F, 0x80], np.uint8)   # scale bytes of the hand table
    for m in ("gate", "up", "down"):
        ex[m] = (ex[m][0], table[rng.integers(0, 4, ex[m][1].shape)])
    x = rng.standard_normal(H)

    def row_dot(codes, scales, r):
        acc = 0.0
        for i in range(H // 2):
            b = int(codes[r, i])
            sc = e8m0[int(scales[r, (2 * i) // 32])]
            acc += e2m1[b & 0xF] * sc * x[2 * i] + e2m1[b >> 4] * sc * x[2 * i + 1]
        return acc

    a = O.expert_activation(x, ex)
    for f in range(F):
        g = row_dot(*ex["gate"], f)
        u = row_dot(*ex["up"], f)
        assert a[f] == pytest.approx(g / (1 + math.exp(-g)) * u, rel=1e-12, abs=1e-15), f
    y = O.expert_ffn(x, ex)
    assert np.allclose(O.mx_decode(*ex["down"]) @ a, y, rtol=1e-13, atol=1e-15)


def _rand_expert(rng, H, F):
    def m(R, C):
        return (rng.integers(0, 256, (R, C // 2), dtype=np.uint8),
                rng.integers(119, 124, (R, C // 32), dtype=np.uint8))
    return {"gate": m(F, H), "up": m(F, H), "down": m(H, F)}


def _tiny_layer(rng, H=64, E=6, F=32, shared=True):
    experts = [_rand_expert(rng, H, F) for _ in range(E)]
    W = np.array([[rng.standard_normal() for _ in range(H)] for _ in range(E)]) / 8
    Wb = (W.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = (rng.standard_normal((1, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    sh = _rand_expert(rng, H, F) if shared else None
    return experts, Wb, x, sh


def test_shared_expert_enters_with_weight_one():
    """Routed experts with zero down codes contribute nothing, so the layer
    output is residual + shared expert exactly (all-ones closed form)."""
    rng = np.random.default_rng(7)
    H, F, E, k = 64, 32, 5, 2
    experts = [_rand_expert(rng, H, F) for _ in range(E)]
    for ex in experts:
        ex["down"] = (np.zeros_like(ex["down"][0]), ex["down"][1])
    sh = _const_expert(H, F, 0x22, 0x7B, 0x78)
    x = _bf16_of_ints(rng.integers(-3, 4, (1, H)))
    W = _bf16_of_ints(rng.integers(-2, 3, (E, H)))
    r = O.moe_layer(x, W, k, lambda e: experts[e], sh, residual_bits=x)
    g = 2.0 ** -4 * O.bf16_to_f64(x).sum()
    a = g / (1 + math.exp(-g)) * g
    assert np.allclose(r["out"][0] - O.bf16_to_f64(x)[0], 2.0 ** -7 * F * a, rtol=1e-14)


def test_layer_is_weighted_sum_of_selected_experts():
    """out - residual = sum_j w_j y_j + y_shared with w from the selected
    logits only; unselected experts (here poisoned with NaN scales) never
    enter."""
    rng = np.random.default_rng(8)
    H, F, E, k = 64, 32, 6, 3
    experts, W, x, sh = _tiny_layer(rng, H, E, F)
    L = O.router_logits(x, W)[0]
    sel = sorted(range(E), key=lambda e: (-L[e], e))[:k]
    for e in range(E):
        if e not in sel:
            experts[e]["gate"] = (experts[e]["gate"][0], np.full_like(experts[e]["gate"][1], 0xFF))
    r = O.moe_layer(x, W, k, lambda e: experts[e], sh, residual_bits=x)
    assert r["idx"][0].tolist() == sel
    assert np.all(np.isfinite(r["out"]))
    z = np.exp(L[sel] - L[sel].max())
    w = z / z.sum()
    xf = O.bf16_to_f64(x)[0]
    ys = [O.expert_ffn(xf, experts[e]) for e in sel]
    want = xf + sum(wi * yi for wi, yi in zip(w, ys)) + O.expert_ffn(xf, sh)
    assert np.allclose(r["out"][0], want, rtol=1e-13, atol=1e-9)
    # dropping the residual removes exactly x
    r0 = O.moe_layer(x, W, k, lambda e: experts[e], sh, residual_bits=None)
    assert np.allclose(r["out"][0] - r0["out"][0], xf, rtol=0, atol=1e-9)


def test_zero_weight_expert_contributes_nothing():
    rng = np.random.default_rng(9)
    H, F, E = 64, 32, 4
    experts, W, x, sh = _tiny_layer(rng, H, E, F)
    # expert 2 gets logit -1000*8 below the others: weight exactly 0
    xf = O.bf16_to_f64(x)[0]
    Wf = O.bf16_to_f64(W)
    Wf[2] = -np.sign(xf) * 1000.0
    W2 = O.f64_to_bf16(Wf)
    r1 = O.moe_layer(x, W2, E, lambda e: experts[e], sh, residual_bits=x)
    assert r1["w"][0][list(r1["idx"][0]).index(2)] == 0.0
    other = dict(experts[2])
    other["down"] = (rng.integers(0, 256, other["down"][0].shape, dtype=np.uint8), other["down"][1])
    ex2 = experts[:2] + [other] + experts[3:]
    r2 = O.moe_layer(x, W2, E, lambda e: ex2[e], sh, residual_bits=x)
    assert np.array_equal(r1["out"], r2["out"])
    # an expert whose codes are all zero outputs exactly zero
    z = _rand_expert(rng, H, F)
    z["down"] = (np.zeros_like(z["down"][0]), z["down"][1])
    assert np.array_equal(O.expert_ffn(xf, z), np.zeros(H))


def test_down_scale_plus_one_doubles_moe_contribution():
    rng = np.random.default_rng(10)
    experts, W, x, sh = _tiny_layer(rng)
    bump = lambda ex: dict(ex, down=(ex["down"][0], ex["down"][1] + 1))
    r1 = O.moe_layer(x, W, 3, lambda e: experts[e], sh, residual_bits=None)
    r2 = O.moe_layer(x, W, 3, lambda e: bump(experts[e]), bump(sh), residual_bits=None)
    assert np.array_equal(r2["out"], 2 * r1["out"])


def test_expert_relabelling_leaves_output_unchanged():
    rng = np.random.default_rng(11)
    experts, W, x, sh = _tiny_layer(rng, E=7)
    perm = rng.permutation(7)                   # new label p holds old expert perm[p]
    r1 = O.moe_layer(x, W, 3, lambda e: experts[e], sh, residual_bits=x)
    r2 = O.moe_layer(x, W[perm], 3, lambda e: experts[perm[e]], sh, residual_bits=x)
    assert [perm[e] for e in r2["idx"][0]] == list(r1["idx"][0])
    assert np.allclose(r1["out"], r2["out"], rtol=1e-14, atol=1e-12)


def test_batch_equals_tokens_one_by_one():
    rng = np.random.default_rng(12)
    experts, W, _, sh = _tiny_layer(rng)
    X = (rng.standard_normal((5, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    rb = O.moe_layer(X, W, 2, lambda e: experts[e], sh, residual_bits=X)
    for t in range(5):
        r1 = O.moe_layer(X[t:t + 1], W, 2, lambda e: experts[e], sh, residual_bits=X[t:t + 1])
        assert np.array_equal(rb["idx"][t], r1["idx"][0])
        assert np.allclose(rb["out"][t], r1["out"][0], rtol=1e-14, atol=1e-12)


def test_grouping_hand_example():
    idx = np.array([[2, 0], [0, 1], [2, 3]])
    off, pairs = O.group_by_expert(idx, 5)
    assert off.tolist() == [0, 2, 3, 5, 6, 6]
    # expert 0: (t0,j1)=1, (t1,j0)=2; expert 1: (t1,j1)=3; expert 2: 0, 4; expert 3: 5
    assert pairs.tolist() == [1, 2, 3, 0, 4, 5]


# ------------------------------------------------------------------ stack

def test_rmsnorm_constant_and_pythagorean_vectors():
    H = 4
    one = np.array([0x3F80] * H, np.uint16)
    # h = c*1, eps = 0: h / rms(h) = sign(c)
    for c, want in ((3.0, 0x3F80), (-0.5, 0xBF80)):
        h = O.f64_to_bf16(np.full((1, H), c))
        assert O.rmsnorm_bf16(h, one, 0.0)[0].tolist() == [want] * H
    # h = (3, 4, 0, 0): mean(h^2) = 25/4, rms = 2.5 -> (1.2, 1.6, 0, 0)
    h = O.f64_to_bf16(np.array([[3.0, 4.0, 0.0, 0.0]]))
    assert O.rmsnorm_bf16(h, one, 1e-6)[0].tolist() == [0x3F9A, 0x3FCD, 0, 0]
    # gain multiplies: gamma = 2 doubles (exact in bf16)
    two = np.array([0x4000] * H, np.uint16)
    assert O.rmsnorm_bf16(h, two, 1e-6)[0].tolist() == [0x401A, 0x404D, 0, 0]


def test_stack_residual_is_the_unnormalised_hidden_state():
    """With every down projection zero the MoE adds nothing, so each layer
    must return its input h unchanged (not the normalised xn)."""
    rng = np.random.default_rng(13)
    H, F, E = 64, 32, 4
    experts = [_rand_expert(rng, H, F) for _ in range(E)]
    for ex in experts:
        ex["down"] = (np.zeros_like(ex["down"][0]), ex["down"][1])
    W = _bf16_of_ints(rng.integers(-2, 3, (E, H)))
    h0 = O.f64_to_bf16(rng.standard_normal((1, H)) * 7)
    g = O.f64_to_bf16(rng.uniform(0.9, 1.1, H))
    layers = [dict(router=W, gamma=g, k=2, routed=lambda e: experts[e], shared=None)] * 3
    recs = O.moe_stack(h0, layers, 1e-6)
    for rec in recs:
        assert np.array_equal(rec["h_next"], h0)
        assert not np.array_equal(rec["xn"], h0)
