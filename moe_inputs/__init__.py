"""Seeded synthetic inputs for the sparse-MoE decode step.

This module is shared by the fp64 oracle's tests and by the HIP path's tests
and benchmark. It holds none of the method's arithmetic: it only draws
numbers and lays them out in the byte formats the library consumes.

Random streams
--------------
* Expert weight bytes (MXFP4 codes and E8M0 scale bytes) come from a
  counter-based generator: word ``i`` of the stream with 64-bit key ``K`` is
  the ``(i+1)``-th output of SplitMix64 seeded with ``K`` (Steele, Lea and
  Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014; the
  finaliser constants are Vigna's public ``splitmix64.c``).  The same
  definition is implemented by ``fill.hip`` so the multi-GB expert tensors
  can be filled on the device and any slice can be regenerated on the host
  bit for bit.
* Normal and uniform draws (activations, router rows, RMSNorm gains) are
  host-only NumPy PCG64 streams keyed by ``(seed, layer, tensor, draw)`` and
  are rounded to bfloat16 directly from float64 (round to nearest, ties to
  even).

Byte formats
------------
An MXFP4 matrix ``M[R][C]`` is two arrays: ``codes`` uint8 ``[R][C/2]``
(element ``2i`` in bits 3:0 of byte ``i``, element ``2i+1`` in bits 7:4) and
``scales`` uint8 ``[R][C/32]`` (one E8M0 byte per 32 consecutive elements of
a row).  Routed experts are stored expert-major: gate/up ``[E][F][H]`` and
down ``[E][H][F]``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "splitmix64_words", "stream_key", "code_bytes",
    "scale_bytes", "bf16_from_f64", "normal_bf16", "uniform_bf16", "token",
    "router_weights", "gamma", "zipf_row_scales", "HostExperts", "TENSOR",
]

_M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
SCALE_LO = 119          # E8M0 byte of 2^-8
SCALE_COUNT = 5         # bytes 119..123 -> 2^-8 .. 2^-4

# tensor ids fed into the stream keys
TENSOR = {
    "gate_codes": 1, "gate_scales": 2, "up_codes": 3, "up_scales": 4,
    "down_codes": 5, "down_scales": 6,
    "s_gate_codes": 7, "s_gate_scales": 8, "s_up_codes": 9, "s_up_scales": 10,
    "s_down_codes": 11, "s_down_scales": 12,
    "router": 20, "token": 21, "gamma": 22, "zipf_perm": 23, "token_base": 24,
}


@dataclass(frozen=True)
class Workload:
    """One decode-layer workload: T tokens, hidden H, E routed experts, top-k,
    expert FFN width F, S shared experts of width Fs, L stacked layers."""
    name: str
    T: int
    H: int
    E: int
    k: int
    F: int
    S: int
    Fs: int
    L: int = 1
    eps: float = 1e-6
    zipf_s: float | None = None
    corr: float | None = None  # tokens of one sequence share this fraction of variance
    seed: int = 0
    notes: str = field(default="", compare=False)

    def expert_bytes(self, F: int | None = None) -> int:
        F = self.F if F is None else F
        # gate + up + down, each R*C/2 code bytes + R*C/32 scale bytes
        return 3 * (F * self.H // 2 + F * self.H // 32)


WORKLOADS = {
    "tiny": Workload("tiny", T=1, H=512, E=32, k=4, F=256, S=0, Fs=0,
                     seed=0x5EED0000),
    "k3_batch1": Workload("k3_batch1", T=1, H=7168, E=896, k=16, F=2048, S=1,
                          Fs=2048, seed=0x5EED0001),
    "k3_tp16_slice": Workload("k3_tp16_slice", T=1, H=7168, E=896, k=16, F=128,
                              S=1, Fs=128, seed=0x5EED0002),
    "k3_batch64_zipf": Workload("k3_batch64_zipf", T=64, H=7168, E=896, k=16,
                                F=2048, S=1, Fs=2048, zipf_s=1.1,
                                seed=0x5EED0003),
    "k3_stack8": Workload("k3_stack8", T=1, H=7168, E=896, k=16, F=2048, S=1,
                          Fs=2048, L=8, seed=0x5EED0004),
    # speculative-decode verify shape: one sequence's token and 7 drafts
    "k3_verify8": Workload("k3_verify8", T=8, H=7168, E=896, k=16, F=2048, S=1,
                           Fs=2048, corr=0.5, seed=0x5EED0005),
}


# ---------------------------------------------------------------- SplitMix64
def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def splitmix64_words(key: int, start: int, count: int) -> np.ndarray:
    """Words ``start .. start+count-1`` of the stream keyed by ``key``."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(key & _M64) + i * np.uint64(GOLDEN)
        return _mix64(z)


def _word(key: int, i: int) -> int:
    return int(splitmix64_words(key, i, 1)[0])


def stream_key(seed: int, layer: int, tensor: str) -> int:
    """64-bit key of one tensor's byte stream."""
    k = seed & _M64
    for part in (layer, TENSOR[tensor]):
        k = _word(k ^ ((part * 0xD1B54A32D192ED03) & _M64), 0)
    return k


def code_bytes(key: int, byte_start: int, n_bytes: int) -> np.ndarray:
    """Uniform code bytes (both nibbles uniform over the 16 E2M1 codes)."""
    assert byte_start % 8 == 0 and n_bytes % 8 == 0
    w = splitmix64_words(key, byte_start // 8, n_bytes // 8)
    return w.astype("<u8").view(np.uint8)


def scale_bytes(key: int, start: int, n: int) -> np.ndarray:
    """E8M0 scale bytes uniform over {119..123}, i.e. 2^-8 .. 2^-4."""
    w = splitmix64_words(key, start, n)
    pick = ((w >> np.uint64(32)) * np.uint64(SCALE_COUNT)) >> np.uint64(32)
    return (pick + np.uint64(SCALE_LO)).astype(np.uint8)


# ------------------------------------------------------- bf16 input rounding
def bf16_from_f64(v) -> np.ndarray:
    """Round float64 to bfloat16 bits (nearest, ties to even), directly."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    flat, res = v.ravel(), out.ravel()
    nan = np.isnan(flat)
    m, e = np.frexp(flat)                       # flat = m * 2^e, 0.5<=|m|<1
    q = np.maximum(e - 8, -133)                 # spacing of bf16 values there
    r = np.ldexp(np.rint(np.ldexp(flat, -q)), q)
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)              # exact, or +-inf on overflow
    res[:] = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    res[nan] = 0x7FC0
    return out


def _rng(seed: int, layer: int, tensor: str, draw: int = 0):
    return np.random.default_rng([seed & 0xFFFFFFFF, seed >> 32, layer,
                                  TENSOR[tensor], draw])


def normal_bf16(seed, layer, tensor, shape, std=1.0, draw=0) -> np.ndarray:
    return bf16_from_f64(_rng(seed, layer, tensor, draw).standard_normal(shape) * std)


def uniform_bf16(seed, layer, tensor, shape, lo, hi, draw=0) -> np.ndarray:
    return bf16_from_f64(_rng(seed, layer, tensor, draw).uniform(lo, hi, shape))


def token(w: Workload, draw: int) -> np.ndarray:
    """One activation row bf16[H] ~ N(0, 1); ``draw`` selects the sample.

    With ``w.corr`` = rho the draws come in sequences of T consecutive
    draws (draw // T) that share a component: x = sqrt(rho) b + sqrt(1 - rho) z
    with b ~ N(0, 1) per sequence and z ~ N(0, 1) per draw, so tokens of one
    sequence have correlation rho and overlapping routing (the verify step of
    speculative decoding runs one sequence's token and its drafts together)."""
    if w.corr is None:
        return normal_bf16(w.seed, 0, "token", (w.H,), 1.0, draw)
    z = _rng(w.seed, 0, "token", draw).standard_normal(w.H)
    b = _rng(w.seed, 0, "token_base", draw // w.T).standard_normal(w.H)
    return bf16_from_f64(np.sqrt(w.corr) * b + np.sqrt(1.0 - w.corr) * z)


def zipf_row_scales(E: int, k: int, s: float, seed: int, p_max: float = 0.45):
    """Per-expert router-row scales that skew expert loads towards Zipf(s).

    Logits of zero-mean rows are symmetric, so an expert can be picked by at
    most about half of the tokens.  Target inclusion probabilities are
    ``p_r = min(p_max, c r^-s)`` over a seeded random ranking of the experts
    with ``sum p = k``.  Modelling logit ``e`` as ``a_e`` times a common
    normal and selection as crossing the threshold that gives every expert
    ``k/E`` when all ``a_e = 1`` yields ``a_e = z(k/E) / z(p_e)`` with ``z``
    the upper normal quantile.  The realised loads only approximate the
    targets; nothing downstream depends on the fit.
    """
    from scipy.special import ndtri
    ranks = np.arange(1, E + 1, dtype=np.float64)
    lo, hi = 0.0, float(E)
    for _ in range(200):                        # bisection on c
        c = 0.5 * (lo + hi)
        if np.minimum(p_max, c * ranks ** -s).sum() > k:
            hi = c
        else:
            lo = c
    p = np.minimum(p_max, lo * ranks ** -s)
    a_rank = ndtri(1.0 - k / E) / ndtri(1.0 - p)
    perm = np.random.default_rng([seed & 0xFFFFFFFF, TENSOR["zipf_perm"]]).permutation(E)
    a = np.empty(E)
    a[perm] = a_rank                            # expert perm[r] has rank r+1
    return a


def router_weights(w: Workload, layer: int) -> np.ndarray:
    """Router rows bf16[E][H] ~ N(0, 1/512), row-scaled for Zipf loads."""
    z = _rng(w.seed, layer, "router").standard_normal((w.E, w.H)) * (1.0 / 512) ** 0.5
    if w.zipf_s is not None:
        z *= zipf_row_scales(w.E, w.k, w.zipf_s, w.seed)[:, None]
    return bf16_from_f64(z)


def gamma(w: Workload, layer: int) -> np.ndarray:
    """RMSNorm gain bf16[H] ~ U(0.9, 1.1)."""
    return uniform_bf16(w.seed, layer, "gamma", (w.H,), 0.9, 1.1)


# ------------------------------------------------------ host expert slices
class HostExperts:
    """Host copies of individual experts of one layer, regenerated from the
    same streams the device filler uses (bit-identical by construction)."""

    def __init__(self, w: Workload, layer: int):
        self.w, self.layer = w, layer

    def _mat(self, prefix: str, rows: int, cols: int, index: int):
        w = self.w
        nc, ns = rows * cols // 2, rows * cols // 32
        ck = stream_key(w.seed, self.layer, prefix + "_codes")
        sk = stream_key(w.seed, self.layer, prefix + "_scales")
        codes = code_bytes(ck, index * nc, nc).reshape(rows, cols // 2)
        scales = scale_bytes(sk, index * ns, ns).reshape(rows, cols // 32)
        return codes, scales

    def routed(self, e: int) -> dict:
        w = self.w
        return {"gate": self._mat("gate", w.F, w.H, e),
                "up": self._mat("up", w.F, w.H, e),
                "down": self._mat("down", w.H, w.F, e)}

    def shared(self) -> dict | None:
        w = self.w
        if w.S == 0:
            return None
        return {"gate": self._mat("s_gate", w.Fs, w.H, 0),
                "up": self._mat("s_up", w.Fs, w.H, 0),
                "down": self._mat("s_down", w.H, w.Fs, 0)}


# ----------------------------------------------------- device-side filling
_LIB = None
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_inputs.so")


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        lib.moe_inputs_fill_codes.argtypes = [ctypes.c_void_p, ctypes.c_uint64,
                                              ctypes.c_uint64, ctypes.c_uint64,
                                              ctypes.c_void_p]
        lib.moe_inputs_fill_scales.argtypes = [ctypes.c_void_p, ctypes.c_uint64,
                                               ctypes.c_uint64, ctypes.c_uint64,
                                               ctypes.c_int, ctypes.c_int,
                                               ctypes.c_void_p]
        lib.moe_inputs_fill_codes.restype = ctypes.c_int
        lib.moe_inputs_fill_scales.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def fill_codes_device(t, key: int, byte_start: int = 0, stream=None):
    """Fill a CUDA uint8 tensor with the code stream ``key`` from byte_start."""
    n = t.numel()
    assert n % 8 == 0 and byte_start % 8 == 0 and t.data_ptr() % 8 == 0
    s = stream if stream is not None else _current_stream()
    rc = _lib().moe_inputs_fill_codes(t.data_ptr(), key, byte_start // 8, n // 8, s)
    if rc != 0:
        raise RuntimeError(f"moe_inputs_fill_codes failed ({rc})")


def fill_scales_device(t, key: int, start: int = 0, stream=None):
    s = stream if stream is not None else _current_stream()
    rc = _lib().moe_inputs_fill_scales(t.data_ptr(), key, start, t.numel(),
                                       SCALE_LO, SCALE_COUNT, s)
    if rc != 0:
        raise RuntimeError(f"moe_inputs_fill_scales failed ({rc})")


def _current_stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


class DeviceLayer:
    """All weights of one layer resident on the device (torch uint8/int16
    tensors); expert bytes are filled by the device generator."""

    def __init__(self, w: Workload, layer: int, device="cuda"):
        import torch
        self.w, self.layer = w, layer
        u8 = dict(dtype=torch.uint8, device=device)

        def mat(prefix, E, rows, cols):
            c = torch.empty(E * rows * cols // 2, **u8)
            s = torch.empty(E * rows * cols // 32, **u8)
            fill_codes_device(c, stream_key(w.seed, layer, prefix + "_codes"))
            fill_scales_device(s, stream_key(w.seed, layer, prefix + "_scales"))
            return c, s

        self.gate = mat("gate", w.E, w.F, w.H)
        self.up = mat("up", w.E, w.F, w.H)
        self.down = mat("down", w.E, w.H, w.F)
        if w.S:
            self.s_gate = mat("s_gate", 1, w.Fs, w.H)
            self.s_up = mat("s_up", 1, w.Fs, w.H)
            self.s_down = mat("s_down", 1, w.H, w.Fs)
        else:
            self.s_gate = self.s_up = self.s_down = None
        r = router_weights(w, layer)
        self.router = torch.from_numpy(r.view(np.int16)).to(device)
        self.router_host = r
        g = gamma(w, layer)
        self.gamma = torch.from_numpy(g.view(np.int16)).to(device)
        self.gamma_host = g
