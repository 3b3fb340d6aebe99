"""Plain float64 CPU oracle of the sparse-MoE decode step.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  It shares no code with the HIP
library: no kernels, headers, helpers, tables or pre/post-processing.  Its
inputs are plain NumPy arrays (bfloat16 values as uint16 bit patterns,
MXFP4 matrices as ``(codes, scales)`` uint8 arrays).

What is computed, and where it comes from
-----------------------------------------
The pages on the Kimi K3 decode work describe the step this oracle follows:
a model with 896 routed experts of which 16 are active per token (page
"英伟达用1.2万行CuTe DSL Megakernel，如何优化Kimi K3？", section
"一个工程师、1.2万行代码、AI辅助开发"; tmtpost page, section "现象"), weights
stored natively as MXFP4 (tmtpost page, section "现象"), an always-active
shared expert that runs beside the selected ones (page "AI手搓1.2万行代码榨干
GB300!…", section 02; smzdm page, section "四步改造"), router scores, and the
residual add of the per-token relay (smzdm page, section "慢的根源").  The
pages give no formulas; the definitions below are the plain readings:

1. MXFP4 (OCP Microscaling Formats v1.0): E2M1 elements (1 sign bit, 2
   exponent bits with bias 1, 1 mantissa bit, exponent field 0 is
   subnormal, no Inf/NaN), one E8M0 scale 2^(b-127) per 32 elements along a
   row (b = 0xFF is NaN).  Element 2i of a row sits in the low nibble of
   byte i.
2. Router logits ``l[t][e] = sum_h x[t][h] * Wr[e][h]``.
3. Top-k: experts ordered by (logit descending, index ascending); the first
   k are selected and returned in that order.
4. Combine weights: softmax over the k selected logits only.
5. Each expert: ``g = G x``, ``u = U x``, ``a = silu(g) * u`` with
   ``silu(v) = v / (1 + exp(-v))``, ``y = D a``.
6. The shared expert's output is added with weight 1.
7. ``out = residual + sum_j w_j y_{i_j} + y_shared`` (kept in float64).
8. Stacked layers: ``xn = bf16(h * gamma / sqrt(mean(h^2) + eps))``,
   ``h <- bf16(h + MoE(xn))``, rounding float64 straight to bfloat16.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against hand-worked format tables, brute force on tiny inputs, closed forms
and invariants.  Where the pages are silent, the readings taken are the
ones stated in the steps above (stable top-k order, float64 accumulation,
bf16 rounding only where a step says so).
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------- formats


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code, from its bit fields (OCP MX v1.0)."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp_field = (code >> 1) & 3
    mant = code & 1
    if exp_field == 0:                       # subnormal: 2^(1-bias) * 0.m
        mag = 2.0 ** (1 - 1) * (mant / 2.0)
    else:                                    # normal: 2^(e-bias) * 1.m
        mag = 2.0 ** (exp_field - 1) * (1.0 + mant / 2.0)
    return sign * mag


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_value(byte) -> np.ndarray:
    """Value of E8M0 scale bytes: 2^(b-127), NaN for 0xFF."""
    b = np.asarray(byte).astype(np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 0xFF, np.nan, v)


def mx_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode an MXFP4 matrix to float64 ``[R][C]``.

    ``codes``: uint8 ``[R][C/2]``; ``scales``: uint8 ``[R][C/32]``.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    R, half = codes.shape
    C = 2 * half
    assert C % 32 == 0 and scales.shape == (R, C // 32), (codes.shape, scales.shape)
    nib = np.empty((R, C), dtype=np.uint8)
    nib[:, 0::2] = codes & 0x0F
    nib[:, 1::2] = codes >> 4
    block_scale = np.repeat(e8m0_value(scales), 32, axis=1)
    return E2M1[nib] * block_scale


def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def f64_to_bf16(v) -> np.ndarray:
    """Round float64 to bfloat16 bits: nearest, ties to even, no detour
    through float32.  Overflow gives +-inf, NaN gives 0x7FC0."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint16)
    for idx, x in np.ndenumerate(v):
        if np.isnan(x):
            out[idx] = 0x7FC0
            continue
        sign = 0x8000 if np.signbit(x) else 0
        a = abs(float(x))
        if a == 0.0:
            out[idx] = sign
            continue
        if np.isinf(a):
            out[idx] = sign | 0x7F80
            continue
        # spacing of bfloat16 values around a: 8 significant bits for normal
        # numbers, fixed 2^-133 below 2^-126 (subnormal range)
        e = int(np.floor(np.log2(a)))
        if 2.0 ** e > a:                     # guard log2 rounding
            e -= 1
        elif 2.0 ** (e + 1) <= a:
            e += 1
        step_exp = max(e - 7, -133)
        q = a / 2.0 ** step_exp              # exact (power-of-two scaling)
        n = int(np.floor(q))
        rem = q - n
        if rem > 0.5 or (rem == 0.5 and (n & 1)):
            n += 1
        r = n * 2.0 ** step_exp
        if r > _BF16_MAX:
            out[idx] = sign | 0x7F80
            continue
        bits32 = int(np.float32(r).view(np.uint32))
        out[idx] = sign | (bits32 >> 16)
    return out


# ------------------------------------------------------------------ router


def router_logits(x_bits: np.ndarray, router_w_bits: np.ndarray) -> np.ndarray:
    """``l[t][e] = sum_h x[t][h] * Wr[e][h]`` in float64.

    ``x_bits``: bf16 ``[T][H]``; ``router_w_bits``: bf16 ``[E][H]``.
    """
    x = bf16_to_f64(np.atleast_2d(x_bits))
    W = bf16_to_f64(router_w_bits)
    return x @ W.T


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per row, ordered by (logit desc,
    index asc), so equal logits prefer the lower expert index."""
    logits = np.atleast_2d(logits)
    T, E = logits.shape
    out = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t]))
        out[t] = order[:k]
    return out


def topk_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over the selected logits only (weights sum to 1 per token)."""
    logits = np.atleast_2d(logits)
    sel = np.take_along_axis(logits, idx, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def topk_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest logit per token (inf if k=E)."""
    logits = np.atleast_2d(logits)
    s = -np.sort(-logits, axis=1)
    if k >= logits.shape[1]:
        return np.full(logits.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


def adjacent_gaps(logits: np.ndarray, k: int) -> np.ndarray:
    """Smallest gap between consecutive logits among the top k+1, per token."""
    logits = np.atleast_2d(logits)
    s = -np.sort(-logits, axis=1)[:, : min(k + 1, logits.shape[1])]
    if s.shape[1] < 2:
        return np.full(logits.shape[0], np.inf)
    return (s[:, :-1] - s[:, 1:]).min(axis=1)


# ----------------------------------------------------------------- experts


def silu(v: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def expert_ffn(x: np.ndarray, expert: dict) -> np.ndarray:
    """One expert on one float64 activation vector: D (silu(G x) * (U x))."""
    G = mx_decode(*expert["gate"])
    U = mx_decode(*expert["up"])
    g = G @ x
    u = U @ x
    del G, U
    a = silu(g) * u
    D = mx_decode(*expert["down"])
    return D @ a


def expert_activation(x: np.ndarray, expert: dict) -> np.ndarray:
    """The gated hidden vector ``a = silu(G x) * (U x)`` of one expert."""
    return silu(mx_decode(*expert["gate"]) @ x) * (mx_decode(*expert["up"]) @ x)


def group_by_expert(idx: np.ndarray, n_experts: int):
    """Token grouping for T > 1: ``offsets[E+1]`` and ``pairs[T*k]`` where
    pairs[offsets[e]:offsets[e+1]] lists ``t*k + j`` for every slot with
    ``idx[t][j] == e``, in increasing ``t*k + j``."""
    idx = np.atleast_2d(idx)
    T, k = idx.shape
    buckets = [[] for _ in range(n_experts)]
    for t in range(T):
        for j in range(k):
            buckets[int(idx[t, j])].append(t * k + j)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + len(buckets[e])
    pairs = np.array([p for b in buckets for p in b], dtype=np.int64)
    return offsets, pairs


def moe_layer(x_bits, router_w_bits, k, routed, shared=None, residual_bits=None, pmap=map):
    """One MoE decode layer in float64.

    ``x_bits``: bf16 ``[T][H]``; ``router_w_bits``: bf16 ``[E][H]``;
    ``routed(e)`` returns expert e as ``{"gate": (codes, scales), "up": ...,
    "down": ...}``; ``shared`` is such a dict or None; ``residual_bits`` is
    bf16 ``[T][H]`` or None (no residual).  ``pmap`` evaluates the
    independent expert outputs (e.g. a thread pool's map); the weighted sum
    is always taken in slot order.  Returns a dict with ``out`` (float64
    ``[T][H]``), ``idx``, ``w``, ``logits``.
    """
    x_bits = np.atleast_2d(x_bits)
    T, H = x_bits.shape
    logits = router_logits(x_bits, router_w_bits)
    idx = topk_select(logits, k)
    w = topk_weights(logits, idx)
    x = bf16_to_f64(x_bits)
    out = np.zeros((T, H)) if residual_bits is None else bf16_to_f64(np.atleast_2d(residual_bits)).copy()
    for t in range(T):
        jobs = [(x[t], int(e)) for e in idx[t]]
        if shared is not None:
            jobs.append((x[t], -1))
        ys = list(pmap(lambda job: expert_ffn(job[0], shared if job[1] < 0 else routed(job[1])), jobs))
        acc = np.zeros(H)
        for j in range(k):
            acc += w[t, j] * ys[j]
        if shared is not None:
            acc += ys[k]
        out[t] += acc
    return {"out": out, "idx": idx, "w": w, "logits": logits}


# ------------------------------------------------------------------- stack


def rmsnorm_bf16(h_bits: np.ndarray, gamma_bits: np.ndarray, eps: float) -> np.ndarray:
    """``bf16(h * gamma / sqrt(mean(h^2) + eps))`` per token, from float64."""
    h = bf16_to_f64(np.atleast_2d(h_bits))
    g = bf16_to_f64(gamma_bits)
    r = np.sqrt((h * h).mean(axis=1, keepdims=True) + eps)
    return f64_to_bf16(h * g / r)


def moe_stack(h_bits, layers, eps, teacher=None, pmap=map):
    """Layers run back to back: RMSNorm, MoE layer, residual add, bf16 round.

    ``layers``: list of dicts with ``router`` (bf16 [E][H]), ``gamma``
    (bf16 [H]), ``k``, ``routed`` (callable), ``shared``.  With
    ``teacher`` (a list of bf16 [T][H] inputs per layer) each layer is fed
    the given input instead of the previous layer's output.  Returns the
    per-layer records (input h, xn, idx, w, logits, float64 out, bf16 h_next).
    """
    h = np.atleast_2d(np.asarray(h_bits, dtype=np.uint16))
    recs = []
    for li, L in enumerate(layers):
        if teacher is not None:
            h = np.atleast_2d(teacher[li])
        xn = rmsnorm_bf16(h, L["gamma"], eps)
        r = moe_layer(xn, L["router"], L["k"], L["routed"], L["shared"], residual_bits=h, pmap=pmap)
        h_next = f64_to_bf16(r["out"])
        recs.append({"h": h, "xn": xn, "idx": r["idx"], "w": r["w"],
                     "logits": r["logits"], "out": r["out"], "h_next": h_next})
        h = h_next
    return recs
