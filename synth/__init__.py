"""Seeded synthetic inputs for the BitDelta path (shared by tests and bench).

Holds no arithmetic of the method: it draws numbers (SplitMix64 counter hash,
see synth.c) and shapes them into the tensors the workloads need.  The
fp32 -> bf16 step that turns draws into bf16 weights and activations is
torch's own conversion (round-to-nearest-even), not the method's code.

Workload recipe (sizes and laws of the post's 70B-class model, see the design
notes): W_base ~ N(0, 0.02) bf16; Delta ~ Laplace(0, b) fp32 with b = 1e-3
(single layers) or b_v log-uniform in [3e-4, 3e-3] (one per variant);
W_ft = fl32(W_base + Delta); activations x ~ N(0, 1) bf16; variant ids from a
Zipf(1.1) split, largest-remainder rounded, then Fisher-Yates shuffled.

Stream tags (element streams never collide): a tensor's tag is
64 * index + kind, kind in TAG_*.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

TAG_WBASE, TAG_DELTA, TAG_X, TAG_IDS, TAG_SCALE, TAG_FACTOR, TAG_NOISE, TAG_OMEGA, TAG_VARIANT = \
    1, 2, 3, 4, 5, 6, 7, 8, 16

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"synth library not built: {_LIB_PATH} (run __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    U64, I64, P, D = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
    lib.synth_key.argtypes = [U64, U64]
    lib.synth_key.restype = U64
    lib.synth_u64.argtypes = [U64, U64, I64, P]
    lib.synth_uniform_f64.argtypes = [U64, U64, I64, P]
    lib.synth_normal_f32.argtypes = [U64, U64, I64, D, D, P]
    lib.synth_laplace_f32.argtypes = [U64, U64, I64, D, P]
    _lib = lib
    return lib


def tag(kind: int, index: int = 0) -> int:
    return 64 * int(index) + int(kind)


def _shape_n(shape):
    shape = (shape,) if isinstance(shape, int) else tuple(shape)
    return shape, int(np.prod(shape)) if shape else 1


def u64(shape, seed: int, tg: int) -> np.ndarray:
    shape, n = _shape_n(shape)
    out = np.empty(n, dtype=np.uint64)
    _load().synth_u64(seed, tg, n, out.ctypes.data_as(ctypes.c_void_p))
    return out.reshape(shape)


def uniform(shape, seed: int, tg: int) -> np.ndarray:
    shape, n = _shape_n(shape)
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform_f64(seed, tg, n, out.ctypes.data_as(ctypes.c_void_p))
    return out.reshape(shape)


def normal_f32(shape, std: float, seed: int, tg: int, mean: float = 0.0) -> np.ndarray:
    shape, n = _shape_n(shape)
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal_f32(seed, tg, n, float(mean), float(std), out.ctypes.data_as(ctypes.c_void_p))
    return out.reshape(shape)


def laplace_f32(shape, b: float, seed: int, tg: int) -> np.ndarray:
    shape, n = _shape_n(shape)
    out = np.empty(n, dtype=np.float32)
    _load().synth_laplace_f32(seed, tg, n, float(b), out.ctypes.data_as(ctypes.c_void_p))
    return out.reshape(shape)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns via torch's round-to-nearest-even conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact: place the 16 bits on top)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def layer(d_out: int, d_in: int, seed: int = 0, index: int = 0, b: float = 1e-3,
          std: float = 0.02, ft_bf16: bool = False):
    """One weight matrix pair: W_base bf16 bits [d_out, d_in] and W_ft [d_out, d_in]
    (fp32 = fl32(W_base + Delta), or bf16 bits of it when ft_bf16)."""
    w_base = to_bf16_bits(normal_f32((d_out, d_in), std, seed, tag(TAG_WBASE, index)))
    delta = laplace_f32((d_out, d_in), b, seed, tag(TAG_DELTA, index))
    w_ft = bf16_bits_to_f32(w_base) + delta  # fp32 add, round-to-nearest-even
    if ft_bf16:
        w_ft = to_bf16_bits(w_ft)
    return w_base, w_ft


def variant_ft(w_base: np.ndarray, v: int, b: float, seed: int = 0, index: int = 0):
    """Fine-tuned weights of variant v over a shared base: fl32(W_base + Delta_v)."""
    delta = laplace_f32(w_base.shape, b, seed, tag(TAG_VARIANT + v, index))
    return bf16_bits_to_f32(w_base) + delta


def lowrank_spectrum(rank: int, rms: float, d_out: int, d_in: int) -> np.ndarray:
    """Singular values s_j = s_0 10^(-j/(rank-1)) (one decade), scaled so the
    low-rank part has entry RMS `rms` over a [d_out, d_in] matrix."""
    if rank == 0:
        return np.zeros(0)
    s = np.power(10.0, -np.arange(rank) / max(rank - 1, 1))
    return s * (rms * math.sqrt(d_out * d_in) / math.sqrt(float(np.sum(s * s))))


def checkpoints(d_out: int, d_in: int, k: int, rank: int, noise: float, rms: float = 1e-3, seed: int = 0,
                index: int = 0, std: float = 0.02):
    """k fine-tuned checkpoints of one matrix over a shared base whose task
    vectors are low rank plus a noise floor: Delta_i = G_i diag(s) H_i^T + E_i,
    G_i [d_out, rank] ~ N(0, 1/d_out), H_i [d_in, rank] ~ N(0, 1/d_in),
    s = lowrank_spectrum(rank, rms, ...), E_i ~ N(0, noise^2) entries.
    Returns W_base bf16 bits [d_out, d_in] and W_ft = fl32(W_base + fl32(Delta_i))
    fp32 [k, d_out, d_in]."""
    w_base = to_bf16_bits(normal_f32((d_out, d_in), std, seed, tag(TAG_WBASE, index)))
    base = bf16_bits_to_f32(w_base)
    s = lowrank_spectrum(rank, rms, d_out, d_in)
    w_ft = np.empty((k, d_out, d_in), dtype=np.float32)
    for i in range(k):
        g = normal_f32((d_out, rank), 1.0 / math.sqrt(d_out), seed,
                       tag(TAG_FACTOR, index + (1 << 20) * (2 * i))).astype(np.float64)
        h = normal_f32((d_in, rank), 1.0 / math.sqrt(d_in), seed,
                       tag(TAG_FACTOR, index + (1 << 20) * (2 * i + 1))).astype(np.float64)
        delta = (g * s) @ h.T
        if noise > 0:
            delta += normal_f32((d_out, d_in), noise, seed, tag(TAG_NOISE, index + (1 << 20) * i))
        w_ft[i] = base + delta.astype(np.float32)
    return w_base, w_ft


def omega(d_in: int, width: int = 64, seed: int = 0, index: int = 0) -> np.ndarray:
    """Gaussian test matrix [d_in, width], i.i.d. N(0, 1) fp32."""
    return normal_f32((d_in, width), 1.0, seed, tag(TAG_OMEGA, index))


def activations(m: int, d_in: int, seed: int = 0, index: int = 0) -> np.ndarray:
    """x ~ N(0, 1), bf16 bits [m, d_in]."""
    return to_bf16_bits(normal_f32((m, d_in), 1.0, seed, tag(TAG_X, index)))


def variant_scales(n_variants: int, lo: float = 3e-4, hi: float = 3e-3, seed: int = 0) -> np.ndarray:
    """Laplace scales b_v, log-uniform in [lo, hi]."""
    u = uniform(n_variants, seed, tag(TAG_SCALE))
    return lo * np.power(hi / lo, u)


def zipf_counts(m: int, n_variants: int, s: float = 1.1) -> list[int]:
    """Group sizes of m tokens over variants of rank 1..V with weights k^-s,
    rounded by largest remainder (ties to the lower rank)."""
    w = [k ** (-s) for k in range(1, n_variants + 1)]
    H = math.fsum(w)
    exact = [m * wk / H for wk in w]
    counts = [int(math.floor(e)) for e in exact]
    rest = m - sum(counts)
    order = sorted(range(n_variants), key=lambda k: (-(exact[k] - counts[k]), k))
    for k in order[:rest]:
        counts[k] += 1
    return counts


def variant_ids(counts, seed: int = 0, shuffle: bool = True) -> np.ndarray:
    """Token -> variant id: segments of the given sizes, then a Fisher-Yates
    shuffle driven by the counter stream (j = floor(u_i * (i + 1)))."""
    ids = np.concatenate([np.full(c, v, dtype=np.int32) for v, c in enumerate(counts)])
    if shuffle and ids.size > 1:
        u = uniform(ids.size, seed, tag(TAG_IDS))
        for i in range(ids.size - 1, 0, -1):
            j = int(u[i] * (i + 1))
            ids[i], ids[j] = ids[j], ids[i]
    return ids


# ------------------------------------------------------------ device side
# Large benchmark inputs are drawn on the GPU with torch's seeded Philox
# generator (same laws as above; values differ from the host streams, which
# is fine: these feed timing runs, parity tests use the host streams).


def _gen(seed: int, tg: int, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1000003 + int(tg)) & ((1 << 63) - 1))
    return g


def device_normal(shape, std: float, seed: int, tg: int, device="cuda", dtype=None):
    import torch

    t = torch.randn(shape, generator=_gen(seed, tg, device), device=device, dtype=torch.float32).mul_(std)
    return t if dtype is None else t.to(dtype)


def device_laplace(shape, b: float, seed: int, tg: int, device="cuda"):
    """Inverse-CDF Laplace(0, b) draws, fp32."""
    import torch

    t = torch.rand(shape, generator=_gen(seed, tg, device), device=device, dtype=torch.float64) - 0.5
    return (-b * torch.sign(t) * torch.log1p(-2.0 * t.abs())).to(torch.float32)


def device_layer(d_out: int, d_in: int, seed: int = 0, index: int = 0, b: float = 1e-3,
                 std: float = 0.02, device="cuda"):
    """(W_base bf16, W_ft fp32 = fl32(W_base + Delta)) on the device."""
    import torch

    w_base = device_normal((d_out, d_in), std, seed, tag(TAG_WBASE, index), device, torch.bfloat16)
    w_ft = w_base.float().add_(device_laplace((d_out, d_in), b, seed, tag(TAG_DELTA, index), device))
    return w_base, w_ft


def device_checkpoints(d_out: int, d_in: int, k: int, rank: int, noise: float, rms: float = 1e-3, seed: int = 0,
                       index: int = 0, std: float = 0.02, device="cuda"):
    """The checkpoints() recipe drawn on the device: (W_base bf16 [d_out, d_in],
    W_ft fp32 [k, d_out, d_in])."""
    import torch

    w_base = device_normal((d_out, d_in), std, seed, tag(TAG_WBASE, index), device, torch.bfloat16)
    s = torch.from_numpy(lowrank_spectrum(rank, rms, d_out, d_in)).to(device=device, dtype=torch.float32)
    w_ft = torch.empty((k, d_out, d_in), dtype=torch.float32, device=device)
    for i in range(k):
        g = device_normal((d_out, rank), 1.0 / math.sqrt(d_out), seed, tag(TAG_FACTOR, index + (1 << 20) * (2 * i)),
                          device)
        h = device_normal((d_in, rank), 1.0 / math.sqrt(d_in), seed,
                          tag(TAG_FACTOR, index + (1 << 20) * (2 * i + 1)), device)
        delta = torch.mm(g * s, h.t().contiguous())
        if noise > 0:
            delta += device_normal((d_out, d_in), noise, seed, tag(TAG_NOISE, index + (1 << 20) * i), device)
        w_ft[i] = w_base.float() + delta
        del delta
    return w_base, w_ft


def device_activations(m: int, d_in: int, seed: int = 0, index: int = 0, device="cuda"):
    import torch

    return device_normal((m, d_in), 1.0, seed, tag(TAG_X, index), device, torch.bfloat16)
