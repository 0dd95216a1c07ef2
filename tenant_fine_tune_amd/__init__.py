"""BitDelta on MI355X: thin Python binding of libbitdelta.so (include/bitdelta.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
the library.  torch supplies device memory (outputs and workspaces are
allocated with torch on the input's device) and the current stream, which is
handed to the library as a hipStream_t.  There is no fallback: if the
library is missing or a call fails, an exception is raised.

Method: "BitDelta: Serving 14 Zen Models from One GPU Cluster" (hanzo.blog,
2026-02-28), "Mathematical Foundation", "Serving Architecture" and
"Infrastructure Details"; `linear` mirrors the post's conceptual
fused_bitdelta_linear(x, w_base, delta_sign, alpha) signature.  `similarity`
is step 1 of "K-Merge: Online LoRA Adapter Management for the Edge" on the
variants' BitDelta task vectors.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["lib", "lib_path", "BitDeltaError", "compress", "reconstruct", "linear", "linear_grouped", "similarity",
           "probe_read", "probe_mfma", "probe_lds",
           "linear_grouped_noalloc", "similarity_delta", "monosoup", "MONOSOUP_SKETCH", "DeltaCache", "LOADER",
           "BD_OK", "BD_EINVAL", "BD_ESHAPE", "BD_EALIGN", "BD_EWORKSPACE", "BD_EDEVICE", "BD_EBUSY",
           "BD_CACHE_HIT", "BD_CACHE_MISS", "BD_CACHE_JOINED",
           "BD_BF16", "BD_F32", "BD_ALPHA_ROW", "BD_ALPHA_MATRIX", "EXPORTS"]

BD_OK, BD_EINVAL, BD_ESHAPE, BD_EALIGN, BD_EWORKSPACE, BD_EDEVICE, BD_EBUSY = range(7)
BD_CACHE_HIT, BD_CACHE_MISS, BD_CACHE_JOINED = 0, 1, 2
BD_BF16, BD_F32 = 0, 1
BD_ALPHA_ROW, BD_ALPHA_MATRIX = 0, 1
MONOSOUP_SKETCH = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libbitdelta.so")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_INT = ctypes.c_int
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); every symbol declared in include/bitdelta.h
EXPORTS = {
    "bitdelta_version": (_INT, []),
    "bitdelta_status_string": (ctypes.c_char_p, [_INT]),
    "bitdelta_last_error": (ctypes.c_char_p, []),
    "bitdelta_compress_workspace": (_SZ, [_I64, _I64, _INT]),
    "bitdelta_compress": (_INT, [_P, _P, _INT, _I64, _I64, _INT, _P, _P, _P, _SZ, _P]),
    "bitdelta_reconstruct": (_INT, [_P, _P, _P, _INT, _I64, _I64, _P, _P]),
    "bitdelta_linear_workspace": (_SZ, [_I64, _I64, _I64]),
    "bitdelta_linear": (_INT, [_P, _I64, _P, _P, _P, _INT, _I64, _I64, _P, _P, _SZ, _P]),
    "bitdelta_linear_grouped_workspace": (_SZ, [_I64, _I32, _I64, _I64]),
    "bitdelta_linear_grouped": (_INT, [_P, _I64, _P, _I32, _P, _P, _P, _INT, _I64, _I64, _P, _P, _SZ, _P]),
    "bitdelta_linear_grouped_noalloc": (_INT, [_P, _I64, _P, _I32, _P, _P, _P, _INT, _I64, _I64, _P, _P]),
    "bitdelta_similarity_workspace": (_SZ, [_I32, _I64, _I64]),
    "bitdelta_similarity": (_INT, [_P, _P, _INT, _I32, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "bitdelta_similarity_delta_workspace": (_SZ, [_I32, _I64, _I64]),
    "bitdelta_similarity_delta": (_INT, [_P, _P, _INT, _I32, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "bitdelta_monosoup_workspace": (_SZ, [_I64, _I64, _I32, _I32]),
    "bitdelta_monosoup": (_INT, [_P, _P, _P, _I32, _I64, _I64, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "bitdelta_probe_read_sink_words": (_I64, [_I64]),
    "bitdelta_probe_read": (_INT, [_P, _I64, _P, _P]),
    "bitdelta_probe_mfma": (_INT, [_I32, _I32, ctypes.c_float, ctypes.c_float, _P, _P]),
    "bitdelta_probe_lds": (_INT, [_I32, _I32, _I32, _I32, _P, _I64, _P, _P, _P]),
    # include/bitdelta_cache.h
    "bitdelta_cache_create": (_INT, [_I32, _I32, _I32, _I64, _P, _SZ, _P, _P, _P]),
    "bitdelta_cache_destroy": (None, [_P]),
    "bitdelta_cache_acquire": (_INT, [_P, _I32, _P, _P]),
    "bitdelta_cache_release": (_INT, [_P, _I32]),
    "bitdelta_cache_release_on_stream": (_INT, [_P, _I32, _P]),
    "bitdelta_cache_slot_of": (_I32, [_P, _I32]),
    "bitdelta_cache_counters": (None, [_P, _P, _P, _P, _P, _P]),
    "bitdelta_cache_host_loader": (_INT, [_P, _I32, _P, _SZ]),
}

# bd_delta_loader: int (*)(void *user, int32_t variant, void *dst, size_t slot_bytes)
LOADER = ctypes.CFUNCTYPE(_INT, _P, _I32, _P, _SZ)


class BitDeltaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{lib.bitdelta_status_string(status).decode()}: {detail}")
        self.status = status


def _load():
    if not os.path.exists(lib_path):
        raise ImportError(f"libbitdelta.so is not built at {lib_path}; run __graft_entry__.build()")
    handle = ctypes.CDLL(lib_path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


lib = _load()


def check(status: int) -> None:
    if status != BD_OK:
        raise BitDeltaError(status, lib.bitdelta_last_error().decode())


# --------------------------------------------------------------- torch glue


def _torch():
    import torch

    return torch


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(dev):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dev_tensor(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _alpha_mode(alpha, d_out, per_matrix):
    if per_matrix is None:
        per_matrix = alpha.numel() == 1 and d_out != 1
    want = 1 if per_matrix else d_out
    if alpha.numel() != want:
        raise ValueError(f"alpha has {alpha.numel()} values, expected {want}")
    return BD_ALPHA_MATRIX if per_matrix else BD_ALPHA_ROW


def compress(w_base, w_ft, per_matrix: bool = False):
    """Delta = W_ft - W_base -> (packed signs uint8 [d_out, d_in/8], alpha fp32 [d_out] or [1])."""
    torch = _torch()
    _dev_tensor(w_base, torch.bfloat16, "w_base")
    if w_ft.dtype == torch.float32:
        ft = BD_F32
    elif w_ft.dtype == torch.bfloat16:
        ft = BD_BF16
    else:
        raise TypeError("w_ft must be float32 or bfloat16")
    _dev_tensor(w_ft, w_ft.dtype, "w_ft")
    d_out, d_in = w_base.shape
    if tuple(w_ft.shape) != (d_out, d_in):
        raise ValueError("w_ft shape differs from w_base")
    mode = BD_ALPHA_MATRIX if per_matrix else BD_ALPHA_ROW
    dev = w_base.device
    signs = torch.empty((d_out, d_in // 8), dtype=torch.uint8, device=dev)
    alpha = torch.empty((1 if per_matrix else d_out,), dtype=torch.float32, device=dev)
    nws = lib.bitdelta_compress_workspace(d_out, d_in, mode)
    ws = torch.empty((nws,), dtype=torch.uint8, device=dev) if nws else None
    check(lib.bitdelta_compress(_ptr(w_base), _ptr(w_ft), ft, d_out, d_in, mode, _ptr(signs), _ptr(alpha),
                                _ptr(ws), nws, _stream(dev)))
    return signs, alpha


def reconstruct(w_base, signs, alpha, per_matrix: bool | None = None):
    """Materialised W_eff = bf16(W_base + alpha * sign) [d_out, d_in]."""
    torch = _torch()
    _dev_tensor(w_base, torch.bfloat16, "w_base")
    _dev_tensor(signs, torch.uint8, "signs")
    _dev_tensor(alpha, torch.float32, "alpha")
    d_out, d_in = w_base.shape
    mode = _alpha_mode(alpha, d_out, per_matrix)
    w_eff = torch.empty_like(w_base)
    check(lib.bitdelta_reconstruct(_ptr(w_base), _ptr(signs), _ptr(alpha), mode, d_out, d_in, _ptr(w_eff),
                                   _stream(w_base.device)))
    return w_eff


def linear(x, w_base, delta_sign, alpha, per_matrix: bool | None = None):
    """Fused y = x (W_base + alpha * sign(Delta))^T; x [..., d_in] -> y [..., d_out] bf16."""
    torch = _torch()
    _dev_tensor(x, torch.bfloat16, "x")
    _dev_tensor(w_base, torch.bfloat16, "w_base")
    _dev_tensor(delta_sign, torch.uint8, "delta_sign")
    _dev_tensor(alpha, torch.float32, "alpha")
    d_out, d_in = w_base.shape
    if x.shape[-1] != d_in:
        raise ValueError(f"x has width {x.shape[-1]}, w_base expects {d_in}")
    mode = _alpha_mode(alpha, d_out, per_matrix)
    lead = tuple(x.shape[:-1])
    m = 1
    for s in lead:
        m *= s
    y = torch.empty(lead + (d_out,), dtype=torch.bfloat16, device=x.device)
    nws = lib.bitdelta_linear_workspace(m, d_out, d_in)
    ws = torch.empty((nws,), dtype=torch.uint8, device=x.device) if nws else None
    check(lib.bitdelta_linear(_ptr(x), m, _ptr(w_base), _ptr(delta_sign), _ptr(alpha), mode, d_out, d_in,
                              _ptr(y), _ptr(ws), nws, _stream(x.device)))
    return y


def linear_grouped(x, variant_ids, w_base, signs, alpha, per_matrix: bool | None = None):
    """Multi-variant linear over one shared W_base: token i uses variant variant_ids[i].
    signs [V, d_out, d_in/8]; alpha [V, d_out] or [V]."""
    torch = _torch()
    _dev_tensor(x, torch.bfloat16, "x")
    _dev_tensor(variant_ids, torch.int32, "variant_ids")
    _dev_tensor(w_base, torch.bfloat16, "w_base")
    _dev_tensor(signs, torch.uint8, "signs")
    _dev_tensor(alpha, torch.float32, "alpha")
    d_out, d_in = w_base.shape
    V = signs.shape[0]
    if tuple(signs.shape) != (V, d_out, d_in // 8):
        raise ValueError("signs must be [V, d_out, d_in/8]")
    if per_matrix is None:
        per_matrix = alpha.dim() == 1 and d_out != 1
    if alpha.numel() != (V if per_matrix else V * d_out):
        raise ValueError("alpha must be [V, d_out] (per row) or [V] (per matrix)")
    mode = BD_ALPHA_MATRIX if per_matrix else BD_ALPHA_ROW
    m = x.shape[0]
    if x.dim() != 2 or variant_ids.numel() != m:
        raise ValueError("x must be [m, d_in] with one variant id per row")
    y = torch.empty((m, d_out), dtype=torch.bfloat16, device=x.device)
    nws = lib.bitdelta_linear_grouped_workspace(m, V, d_out, d_in)
    ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device=x.device)
    check(lib.bitdelta_linear_grouped(_ptr(x), m, _ptr(variant_ids), V, _ptr(w_base), _ptr(signs), _ptr(alpha),
                                      mode, d_out, d_in, _ptr(y), _ptr(ws), nws, _stream(x.device)))
    return y


def linear_grouped_noalloc(x, variant_ids, w_base, signs, alpha, per_matrix: bool | None = None, out=None):
    """linear_grouped with the library's own device-resident bucketing table
    (bitdelta_linear_grouped_noalloc): no workspace; at most
    BD_GROUPED_NOALLOC_MAX_TOKENS (65536) tokens.  `out` (bf16 [m, d_out])
    receives y when given, so the call itself allocates nothing."""
    torch = _torch()
    _dev_tensor(x, torch.bfloat16, "x")
    _dev_tensor(variant_ids, torch.int32, "variant_ids")
    _dev_tensor(w_base, torch.bfloat16, "w_base")
    _dev_tensor(signs, torch.uint8, "signs")
    _dev_tensor(alpha, torch.float32, "alpha")
    d_out, d_in = w_base.shape
    V = signs.shape[0]
    if tuple(signs.shape) != (V, d_out, d_in // 8):
        raise ValueError("signs must be [V, d_out, d_in/8]")
    if per_matrix is None:
        per_matrix = alpha.dim() == 1 and d_out != 1
    if alpha.numel() != (V if per_matrix else V * d_out):
        raise ValueError("alpha must be [V, d_out] (per row) or [V] (per matrix)")
    mode = BD_ALPHA_MATRIX if per_matrix else BD_ALPHA_ROW
    m = x.shape[0]
    if x.dim() != 2 or variant_ids.numel() != m:
        raise ValueError("x must be [m, d_in] with one variant id per row")
    y = torch.empty((m, d_out), dtype=torch.bfloat16, device=x.device) if out is None else out
    _dev_tensor(y, torch.bfloat16, "out")
    if tuple(y.shape) != (m, d_out):
        raise ValueError("out must be [m, d_out]")
    check(lib.bitdelta_linear_grouped_noalloc(_ptr(x), m, _ptr(variant_ids), V, _ptr(w_base), _ptr(signs),
                                              _ptr(alpha), mode, d_out, d_in, _ptr(y), _stream(x.device)))
    return y


def similarity(signs, alpha, per_matrix: bool | None = None):
    """Gram matrix <tau_a, tau_b> and cosines of V variants' task vectors
    tau_v = alpha_v * sign_v over one matrix.  signs [V, d_out, d_in/8];
    alpha [V, d_out] or [V].  Returns (gram, cosine), float64 [V, V] on the
    signs' device."""
    torch = _torch()
    _dev_tensor(signs, torch.uint8, "signs")
    _dev_tensor(alpha, torch.float32, "alpha")
    if signs.dim() != 3:
        raise ValueError("signs must be [V, d_out, d_in/8]")
    V, d_out, g = signs.shape
    d_in = 8 * g
    if per_matrix is None:
        per_matrix = alpha.dim() == 1 and d_out != 1
    if alpha.numel() != (V if per_matrix else V * d_out):
        raise ValueError("alpha must be [V, d_out] (per row) or [V] (per matrix)")
    mode = BD_ALPHA_MATRIX if per_matrix else BD_ALPHA_ROW
    gram = torch.empty((V, V), dtype=torch.float64, device=signs.device)
    cos = torch.empty((V, V), dtype=torch.float64, device=signs.device)
    nws = lib.bitdelta_similarity_workspace(V, d_out, d_in)
    ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device=signs.device)
    check(lib.bitdelta_similarity(_ptr(signs), _ptr(alpha), mode, V, d_out, d_in, _ptr(gram), _ptr(cos), _ptr(ws),
                                  nws, _stream(signs.device)))
    return gram, cos


def similarity_delta(w_base, w_ft):
    """Gram matrix <Delta_a, Delta_b> and cosines of V variants' full task
    vectors Delta_v = fl32(W_ft_v - W_base) over one matrix.  w_base bf16
    [d_out, d_in]; w_ft fp32 or bf16 [V, d_out, d_in].  Returns (gram,
    cosine), float64 [V, V] on the weights' device."""
    torch = _torch()
    _dev_tensor(w_base, torch.bfloat16, "w_base")
    if w_ft.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("w_ft must be float32 or bfloat16")
    _dev_tensor(w_ft, w_ft.dtype, "w_ft")
    if w_ft.dim() != 3 or w_base.dim() != 2 or tuple(w_ft.shape[1:]) != tuple(w_base.shape):
        raise ValueError("w_ft must be [V, d_out, d_in] over w_base [d_out, d_in]")
    V, d_out, d_in = w_ft.shape
    gram = torch.empty((V, V), dtype=torch.float64, device=w_base.device)
    cos = torch.empty((V, V), dtype=torch.float64, device=w_base.device)
    nws = lib.bitdelta_similarity_delta_workspace(V, d_out, d_in)
    ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device=w_base.device)
    ft = BD_F32 if w_ft.dtype == torch.float32 else BD_BF16
    check(lib.bitdelta_similarity_delta(_ptr(w_base), _ptr(w_ft), ft, V, d_out, d_in, _ptr(gram), _ptr(cos),
                                        _ptr(ws), nws, _stream(w_base.device)))
    return gram, cos


def monosoup(w_base, w_ft, omega, rank: int, power_iters: int = 1, out=None, sigma: bool = True):
    """MonoSoup merge W_base + (1/k) sum_i tau_i of k checkpoints, tau_i the
    rank-`rank` truncation of Delta_i = fl32(W_i - W_base) from a 64-column
    randomized range finder.  w_base bf16 [R, C]; w_ft fp32 [k, R, C]; omega
    fp32 [C, 64] (the caller's Gaussian test matrix).  Returns (merged fp32
    [R, C], sigma fp64 [k, rank] or None)."""
    torch = _torch()
    _dev_tensor(w_base, torch.bfloat16, "w_base")
    _dev_tensor(w_ft, torch.float32, "w_ft")
    if w_base.dim() != 2 or w_ft.dim() != 3 or tuple(w_ft.shape[1:]) != tuple(w_base.shape):
        raise ValueError("w_base must be [R, C] and w_ft [k, R, C]")
    k, R, C = w_ft.shape
    if rank > 0:
        _dev_tensor(omega, torch.float32, "omega")
        if tuple(omega.shape) != (C, MONOSOUP_SKETCH):
            raise ValueError(f"omega must be [{C}, {MONOSOUP_SKETCH}]")
    if out is None:
        out = torch.empty((R, C), dtype=torch.float32, device=w_base.device)
    else:
        _dev_tensor(out, torch.float32, "out")
        if tuple(out.shape) != (R, C):
            raise ValueError("out must be [R, C]")
    sig = torch.empty((k, rank), dtype=torch.float64, device=w_base.device) if sigma and rank > 0 else None
    nws = lib.bitdelta_monosoup_workspace(R, C, k, rank)
    ws = torch.empty((max(nws, 256),), dtype=torch.uint8, device=w_base.device)
    check(lib.bitdelta_monosoup(_ptr(w_base), _ptr(w_ft), _ptr(omega) if rank > 0 else None, k, R, C, rank,
                                power_iters, _ptr(out), _ptr(sig) if sig is not None else None, _ptr(ws), nws,
                                _stream(w_base.device)))
    return out, sig


def probe_read(src, sink=None):
    """Measurement probe (no part of the method): read the bytes of the
    device tensor `src` once with 1 KB-per-instruction streaming loads.
    Returns the int32 sink (one XOR word per wave, so the XOR of all of them
    is the XOR of the buffer's 32-bit words)."""
    torch = _torch()
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    words = lib.bitdelta_probe_read_sink_words(nbytes)
    if sink is None:
        sink = torch.empty((max(words, 1),), dtype=torch.int32, device=src.device)
    check(lib.bitdelta_probe_read(_ptr(src), nbytes, _ptr(sink), _stream(src.device)))
    return sink


def probe_mfma(blocks: int, iters: int, a: float = 1.0, b: float = 1.0, sink=None, device=None):
    """Measurement probe (no part of the method): `blocks` workgroups of 4
    waves, each running iters x 8 independent bf16 32x32x16 MFMAs on register
    operands.  Returns the float32 sink, one word per wave, each equal to
    128 * iters * bf16(a) * bf16(b)."""
    torch = _torch()
    dev = torch.device("cuda") if device is None else torch.device(device)
    if sink is None:
        sink = torch.empty((blocks * 4,), dtype=torch.float32, device=dev)
    check(lib.bitdelta_probe_mfma(blocks, iters, a, b, _ptr(sink), _stream(dev)))
    return sink


def probe_lds(blocks: int, iters: int, mode: int, stride: int = 17, src=None, device=None):
    """Measurement probe (no part of the method): LDS reads of 16 bytes per
    lane (mode 0), of 8 bytes (mode 1), writes of 16 bytes (mode 2) or
    direct-to-LDS copies of the device tensor `src` (mode 3, a power of two
    from 1 KB to 1 GiB), each wave of `blocks` 16-wave workgroups moving
    iters x 8 contiguous blocks (include/bitdelta.h).  Returns (sink int32
    [blocks * 16], cycles int64 [blocks])."""
    torch = _torch()
    dev = torch.device("cuda") if device is None else torch.device(device)
    sink = torch.empty((blocks * 16,), dtype=torch.int32, device=dev)
    cycles = torch.empty((blocks,), dtype=torch.int64, device=dev)
    nbytes = 0 if src is None else src.numel() * src.element_size()
    check(lib.bitdelta_probe_lds(blocks, iters, mode, stride, _ptr(src) if src is not None else None, nbytes,
                                 _ptr(sink), _ptr(cycles), _stream(dev)))
    return sink, cycles


class DeltaCache:
    """Delta cache over `n_slots` slots of `slot_bytes` in a device region
    (include/bitdelta_cache.h).  `loader(variant, dst_ptr, slot_bytes) -> int`
    fills a slot (0 = success); `slots` is a device tensor of at least
    n_slots * slot_bytes bytes that must outlive the cache."""

    def __init__(self, n_variants, n_slots, n_pinned, window, slots, slot_bytes, loader=None, host=None):
        """Either `loader` (a Python callable) or `host`: a list of n_variants
        host tensors (pinned, slot_bytes each), copied by the library's own
        loader (bitdelta_cache_host_loader) on the current stream."""
        torch = _torch()
        if not isinstance(slots, torch.Tensor) or slots.device.type != "cuda":
            raise TypeError("slots must be a device tensor")
        if slots.numel() * slots.element_size() < n_slots * slot_bytes:
            raise ValueError("slots region too small")
        if (loader is None) == (host is None):
            raise ValueError("give exactly one of loader and host")
        self._slots = slots
        if host is not None:
            if len(host) != n_variants or any(h.numel() * h.element_size() < slot_bytes or h.device.type != "cpu"
                                              for h in host):
                raise ValueError("host must hold n_variants host tensors of slot_bytes each")
            self._host = host
            self._table = (ctypes.c_void_p * n_variants)(*[h.data_ptr() for h in host])

            class _HostLoader(ctypes.Structure):
                _fields_ = [("host_ptrs", ctypes.c_void_p), ("stream", ctypes.c_void_p)]

            self._hl = _HostLoader(ctypes.cast(self._table, ctypes.c_void_p), _stream(slots.device))
            self._cb = ctypes.cast(lib.bitdelta_cache_host_loader, LOADER)
            user = ctypes.cast(ctypes.pointer(self._hl), ctypes.c_void_p)
        else:
            self._cb = LOADER(lambda user, v, dst, n: int(loader(v, dst, n)))
            user = None
        h = ctypes.c_void_p()
        check(lib.bitdelta_cache_create(n_variants, n_slots, n_pinned, window, _ptr(slots), slot_bytes, self._cb,
                                        user, ctypes.byref(h)))
        self._h = h

    def acquire(self, variant):
        """(device pointer of the slot, outcome BD_CACHE_HIT / _MISS / _JOINED)."""
        p, o = ctypes.c_void_p(), ctypes.c_int()
        check(lib.bitdelta_cache_acquire(self._h, variant, ctypes.byref(p), ctypes.byref(o)))
        return p.value, o.value

    def release(self, variant):
        """Give up a hold; every GPU read of the slot must be complete."""
        check(lib.bitdelta_cache_release(self._h, variant))

    def release_on_stream(self, variant, stream=None):
        """Give up a hold once the work queued so far on `stream` (torch's
        current stream by default) is done."""
        torch = _torch()
        st = (stream or torch.cuda.current_stream(self._slots.device)).cuda_stream
        check(lib.bitdelta_cache_release_on_stream(self._h, variant, ctypes.c_void_p(st)))

    def slot_of(self, variant):
        return lib.bitdelta_cache_slot_of(self._h, variant)

    def counters(self):
        v = [ctypes.c_int64() for _ in range(5)]
        lib.bitdelta_cache_counters(self._h, *[ctypes.byref(x) for x in v])
        return dict(zip(("hits", "misses", "joins", "evictions", "busy"), (x.value for x in v)))

    def close(self):
        if self._h:
            lib.bitdelta_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()
