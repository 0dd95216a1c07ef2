"""BitDelta oracle: numpy-facing wrapper of the plain C reference.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this package; the product path never does.  It shares
no code with the GPU library (see bitdelta_oracle.c for the method, the
citations of "BitDelta: Serving 14 Zen Models from One GPU Cluster" and the
readings taken where the post is silent).

Arrays are numpy: bf16 values travel as their uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

ROW, MATRIX = 0, 1


def _bind(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.oracle_f32_from_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_f32_from_bf16.restype = ctypes.c_float
    lib.oracle_bf16_from_f32.argtypes = [ctypes.c_float]
    lib.oracle_bf16_from_f32.restype = ctypes.c_uint16
    lib.oracle_compress.argtypes = [P, P, I, I64, I64, I, P, P, P]
    lib.oracle_compress.restype = I
    lib.oracle_reconstruct.argtypes = [P, P, P, I, I64, I64, P]
    lib.oracle_reconstruct.restype = I
    lib.oracle_linear_rows.argtypes = [P, I64, P, P, P, I, I64, I64, P, I64, P, P]
    lib.oracle_linear_rows.restype = I
    lib.oracle_linear_grouped_rows.argtypes = [P, I64, P, ctypes.c_int32, P, P, P, I, I64, I64,
                                               P, I64, P, P]
    lib.oracle_linear_grouped_rows.restype = I
    lib.oracle_similarity.argtypes = [P, P, I, ctypes.c_int32, I64, I64, P, P]
    lib.oracle_similarity.restype = I
    lib.oracle_similarity_delta.argtypes = [P, P, I, ctypes.c_int32, I64, I64, P, P]
    lib.oracle_similarity_delta.restype = I
    lib.oracle_monosoup.argtypes = [P, P, ctypes.c_int32, I64, I64, ctypes.c_int32, P, P]
    lib.oracle_monosoup.restype = I
    lib.oracle_num_threads.restype = I
    lib.oracle_set_num_threads.argtypes = [I]
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


class Oracle:
    """One loaded build of the oracle library (the default one, or a test build)."""

    def __init__(self, lib_path: str = LIB_PATH):
        if not os.path.exists(lib_path):
            raise RuntimeError(f"oracle library not built: {lib_path} (run __graft_entry__.build())")
        self.path = lib_path
        self.lib = _bind(ctypes.CDLL(lib_path))

    def num_threads(self) -> int:
        return self.lib.oracle_num_threads()

    def set_num_threads(self, n: int) -> None:
        self.lib.oracle_set_num_threads(int(n))

    def f32_from_bf16(self, bits) -> np.ndarray:
        """Widen bf16 bit patterns to fp32 values (exact)."""
        b = np.asarray(bits, dtype=np.uint16)
        f = self.lib.oracle_f32_from_bf16
        return np.array([f(int(v)) for v in b.ravel()], dtype=np.float32).reshape(b.shape)

    def bf16_from_f32(self, vals) -> np.ndarray:
        """Round fp32 values to bf16 bits, nearest-even (element by element, slow)."""
        v = np.asarray(vals, dtype=np.float32)
        f = self.lib.oracle_bf16_from_f32
        return np.array([f(float(t)) for t in v.ravel()], dtype=np.uint16).reshape(v.shape)

    def compress(self, w_base, w_ft, per_matrix: bool = False, return_row_sums: bool = False):
        """Delta = fl32(W_ft - W_base); signs packed LSB-first; alpha = mean |Delta|.

        w_base: uint16 [R, C] (bf16 bits); w_ft: float32 [R, C] or uint16 (bf16 bits).
        Returns (signs uint8 [R, C/8], alpha float32 [R] or [1][, row sums fp64 [R]]).
        """
        lib = self.lib
        w_base = _c(w_base, np.uint16)
        w_ft = np.ascontiguousarray(w_ft)
        if w_ft.dtype == np.float32:
            is_f32 = 1
        elif w_ft.dtype == np.uint16:
            is_f32 = 0
        else:
            raise TypeError("w_ft must be float32 or uint16 (bf16 bits)")
        R, C = w_base.shape
        if w_ft.shape != (R, C):
            raise ValueError("w_ft shape mismatch")
        signs = np.zeros((R, C // 8), dtype=np.uint8)
        alpha = np.zeros((1 if per_matrix else R,), dtype=np.float32)
        sums = np.zeros((R,), dtype=np.float64)
        rc = lib.oracle_compress(_ptr(w_base), _ptr(w_ft), is_f32, R, C, int(per_matrix),
                                 _ptr(signs), _ptr(alpha), _ptr(sums))
        if rc != 0:
            raise ValueError(f"oracle_compress failed ({rc})")
        return (signs, alpha, sums) if return_row_sums else (signs, alpha)

    def reconstruct(self, w_base, signs, alpha, per_matrix: bool = False) -> np.ndarray:
        """W_eff = bf16_rne(f32(W_base) + (bit ? alpha : -alpha)) -> uint16 [R, C]."""
        lib = self.lib
        w_base = _c(w_base, np.uint16)
        signs = _c(signs, np.uint8)
        alpha = _c(alpha, np.float32)
        R, C = w_base.shape
        out = np.zeros((R, C), dtype=np.uint16)
        rc = lib.oracle_reconstruct(_ptr(w_base), _ptr(signs), _ptr(alpha), int(per_matrix), R, C, _ptr(out))
        if rc != 0:
            raise ValueError(f"oracle_reconstruct failed ({rc})")
        return out

    def linear(self, x, w_base, signs, alpha, per_matrix: bool = False, rows=None):
        """y64 = x W_eff^T in fp64, plus the tolerance normaliser sum |x||W_eff|.

        x: uint16 [M, C]; rows: optional int64 list of W rows (output columns).
        Returns (y64 [M, n_rows], scale [M, n_rows]) as float64.
        """
        lib = self.lib
        x = _c(x, np.uint16)
        w_base = _c(w_base, np.uint16)
        signs = _c(signs, np.uint8)
        alpha = _c(alpha, np.float32)
        M, C = x.shape
        R = w_base.shape[0]
        if w_base.shape[1] != C:
            raise ValueError("x / w_base width mismatch")
        rr = None if rows is None else _c(np.asarray(rows, dtype=np.int64), np.int64)
        if rr is not None and rr.size and (rr.min() < 0 or rr.max() >= R):
            raise ValueError(f"rows must lie in [0, {R})")
        n = R if rr is None else rr.shape[0]
        y = np.zeros((M, n), dtype=np.float64)
        sc = np.zeros((M, n), dtype=np.float64)
        rc = lib.oracle_linear_rows(_ptr(x), M, _ptr(w_base), _ptr(signs), _ptr(alpha), int(per_matrix),
                                    R, C, _ptr(rr), n, _ptr(y), _ptr(sc))
        if rc != 0:
            raise ValueError(f"oracle_linear_rows failed ({rc})")
        return y, sc

    def linear_grouped(self, x, ids, w_base, signs, alpha, per_matrix: bool = False, rows=None):
        """Per-token variant linear; signs [V, R, C/8], alpha [V, R] or [V]."""
        lib = self.lib
        x = _c(x, np.uint16)
        ids = _c(ids, np.int32)
        w_base = _c(w_base, np.uint16)
        signs = _c(signs, np.uint8)
        alpha = _c(alpha, np.float32)
        M, C = x.shape
        R = w_base.shape[0]
        V = signs.shape[0]
        rr = None if rows is None else _c(np.asarray(rows, dtype=np.int64), np.int64)
        if rr is not None and rr.size and (rr.min() < 0 or rr.max() >= R):
            raise ValueError(f"rows must lie in [0, {R})")
        n = R if rr is None else rr.shape[0]
        y = np.zeros((M, n), dtype=np.float64)
        sc = np.zeros((M, n), dtype=np.float64)
        rc = lib.oracle_linear_grouped_rows(_ptr(x), M, _ptr(ids), V, _ptr(w_base), _ptr(signs), _ptr(alpha),
                                            int(per_matrix), R, C, _ptr(rr), n, _ptr(y), _ptr(sc))
        if rc != 0:
            raise ValueError(f"oracle_linear_grouped_rows failed ({rc})")
        return y, sc


    def similarity(self, signs, alpha, per_matrix: bool = False):
        """Gram matrix and cosines of the variants' task vectors (R7).

        signs: uint8 [V, R, C/8]; alpha: fp32 [V, R] or [V].
        Returns (gram [V, V], cos [V, V]) as float64.
        """
        lib = self.lib
        signs = _c(signs, np.uint8)
        alpha = _c(alpha, np.float32)
        V, R, G = signs.shape
        gram = np.zeros((V, V), dtype=np.float64)
        cos = np.zeros((V, V), dtype=np.float64)
        rc = lib.oracle_similarity(_ptr(signs), _ptr(alpha), int(per_matrix), V, R, 8 * G, _ptr(gram), _ptr(cos))
        if rc != 0:
            raise ValueError(f"oracle_similarity failed ({rc})")
        return gram, cos


    def similarity_delta(self, w_base, w_ft):
        """Gram matrix and cosines of the variants' full task vectors (R9):
        Delta_v = fl32(W_ft_v - W_base), summed in the fixed fp64 order.

        w_base: uint16 [R, C]; w_ft: float32 or uint16 (bf16 bits) [V, R, C].
        Returns (gram [V, V], cos [V, V]) as float64.
        """
        lib = self.lib
        w_base = _c(w_base, np.uint16)
        w_ft = np.ascontiguousarray(w_ft)
        if w_ft.dtype == np.float32:
            is_f32 = 1
        elif w_ft.dtype == np.uint16:
            is_f32 = 0
        else:
            raise TypeError("w_ft must be float32 or uint16 (bf16 bits)")
        V, R, C = w_ft.shape
        if w_base.shape != (R, C):
            raise ValueError("w_base shape mismatch")
        gram = np.zeros((V, V), dtype=np.float64)
        cos = np.zeros((V, V), dtype=np.float64)
        rc = lib.oracle_similarity_delta(_ptr(w_base), _ptr(w_ft), is_f32, V, R, C, _ptr(gram), _ptr(cos))
        if rc != 0:
            raise ValueError(f"oracle_similarity_delta failed ({rc})")
        return gram, cos

    def monosoup(self, w_base, w_ft, rank: int):
        """MonoSoup merge (R8): W_base + (1/k) sum_i tau_i, tau_i the rank-`rank`
        truncated SVD of Delta_i = fl32(W_i - W_base).  w_base: uint16 [R, C];
        w_ft: fp32 [k, R, C].  Returns (merged fp64 [R, C], sigma fp64 [k, min(R, C)])."""
        lib = self.lib
        w_base = _c(w_base, np.uint16)
        w_ft = _c(w_ft, np.float32)
        k, R, C = w_ft.shape
        out = np.zeros((R, C), dtype=np.float64)
        sig = np.zeros((k, min(R, C)), dtype=np.float64)
        rc = lib.oracle_monosoup(_ptr(w_base), _ptr(w_ft), k, R, C, rank, _ptr(out), _ptr(sig))
        if rc != 0:
            raise ValueError(f"oracle_monosoup failed ({rc})")
        return out, sig


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def num_threads() -> int:
    return default().num_threads()


def set_num_threads(n: int) -> None:
    default().set_num_threads(n)


def f32_from_bf16(bits):
    return default().f32_from_bf16(bits)


def bf16_from_f32(vals):
    return default().bf16_from_f32(vals)


def compress(*a, **k):
    return default().compress(*a, **k)


def reconstruct(*a, **k):
    return default().reconstruct(*a, **k)


def linear(*a, **k):
    return default().linear(*a, **k)


def linear_grouped(*a, **k):
    return default().linear_grouped(*a, **k)


def similarity(*a, **k):
    return default().similarity(*a, **k)


def similarity_delta(*a, **k):
    return default().similarity_delta(*a, **k)


def monosoup(*a, **k):
    return default().monosoup(*a, **k)
