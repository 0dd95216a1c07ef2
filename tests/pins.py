"""Pins of the oracle to facts other than itself.

Each pin takes an oracle build `o` (oracle.Oracle) and raises AssertionError on
a mismatch.  The sources of truth are the post ("BitDelta: Serving 14 Zen
Models from One GPU Cluster", hanzo.blog 2026-02-28), closed forms,
independent libraries (torch's bf16 conversion, numpy's bit unpacking and
float64 matmul, Python's exact math.fsum and fractions) and hand-derived
fixtures under tests/golden/.  They are chosen so that a plausible slip in the
oracle (a dropped term, a wrong sign, bit order or index, a transposed
operand, a wrong divisor) fails at least one of them; tests/test_oracle_mutants.py
checks exactly that on deliberately broken builds.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _json(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32_bits(h: str) -> np.float32:
    return np.array([int(h, 16)], dtype=np.uint32).view(np.float32)[0]


def _torch_bf16_bits(vals: np.ndarray) -> np.ndarray:
    import torch

    return torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _torch_widen(bits: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.float().numpy()


def _ulp_diff_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ia = np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, dtype=np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


# --------------------------------------------------------------------- bf16


def pin_bf16_widen(o):
    """Widening bf16 -> fp32 agrees with torch on every finite pattern class."""
    bits = np.concatenate([np.arange(0, 0x7F80, 97, dtype=np.uint16),
                           (np.arange(0, 0x7F80, 89) | 0x8000).astype(np.uint16),
                           np.array([0x0001, 0x007F, 0x0080, 0x7F7F, 0x7F80, 0xFF80, 0x8000], dtype=np.uint16)])
    got = o.f32_from_bf16(bits)
    ref = _torch_widen(bits)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def pin_bf16_round(o):
    """Nearest-even rounding to bf16 agrees with torch's conversion, including
    exact ties, subnormals and overflow."""
    rng_vals = synth.normal_f32(4000, 1.0, 7, 901) * np.float32(3e-2)
    big = synth.normal_f32(1000, 1.0, 7, 902) * np.float32(1e30)
    # construct exact ties: a bf16 value plus exactly half of its last place
    base = synth.to_bf16_bits(synth.normal_f32(1000, 1.0, 7, 903))
    ties = (base.astype(np.uint32) << 16 | 0x8000).view(np.float32)
    near = (base.astype(np.uint32) << 16 | 0x7FFF).view(np.float32)
    sub = np.array([1e-40, -1e-40, 5e-39, 1.2e-38, 3.4e38, -3.4e38, 0.0, -0.0], dtype=np.float32)
    vals = np.concatenate([rng_vals, big, ties, near, sub]).astype(np.float32)
    got = o.bf16_from_f32(vals)
    ref = _torch_bf16_bits(vals)
    assert np.array_equal(got, ref), np.nonzero(got != ref)


def pin_bf16_hand_ties(o):
    """Hand-derived ties (tests/golden/reconstruct_cases.json, first cases)."""
    assert o.bf16_from_f32(np.float32(1 + 2 ** -8)) == 0x3F80
    assert o.bf16_from_f32(np.float32(1 + 3 * 2 ** -8)) == 0x3F82
    assert o.bf16_from_f32(np.float32(1 - 2 ** -8)) == 0x3F7F
    assert o.bf16_from_f32(np.float32(-1 - 2 ** -8)) == 0xBF80


# ----------------------------------------------------------------- compress


def _handbuilt_4x16():
    """Inputs of tests/golden/compress_4x16.json, built from its stated rules."""
    j = np.arange(16)
    wb = np.zeros((4, 16), dtype=np.float64)
    wb[0:3] = (j - 8) * 2.0 ** -6
    wb[3] = (j - 15) * 2.0 ** -6
    d = np.zeros((4, 16), dtype=np.float64)
    d[0] = np.where(j % 2 == 0, 2.0 ** -10, -(2.0 ** -10))
    d[1] = np.where(j < 8, 3 * 2.0 ** -9, 0.0)
    d[2] = -(j + 1) * 2.0 ** -12
    d[3] = -(2.0 ** -11)
    d[3, 0] = 2.0 ** -8
    d[3, 15] = 0.0
    w_base = synth.to_bf16_bits(wb.astype(np.float32))
    w_ft = (wb + d).astype(np.float32)
    w_ft[3, 15] = np.float32(-0.0)  # W_base[3,15] = +0, so Delta = -0
    assert synth.bf16_bits_to_f32(w_base)[3, 15] == 0.0
    return w_base, w_ft


def pin_compress_handbuilt(o):
    g = _json("compress_4x16.json")
    w_base, w_ft = _handbuilt_4x16()
    signs, alpha = o.compress(w_base, w_ft)
    assert signs.tolist() == g["expected_signs"], signs.tolist()
    assert alpha.tolist() == g["expected_alpha_row"], alpha.tolist()
    s2, a2 = o.compress(w_base, w_ft, per_matrix=True)
    assert np.array_equal(s2, signs)
    assert a2.tolist() == [g["expected_alpha_matrix"]]
    # A bf16 W_ft is widened exactly first: same result as its fp32 value.
    ft16 = synth.to_bf16_bits(w_ft)
    s3, a3 = o.compress(w_base, ft16)
    s4, a4 = o.compress(w_base, synth.bf16_bits_to_f32(ft16))
    assert np.array_equal(s3, s4) and np.array_equal(a3, a4)


def pin_compress_packing_vs_numpy(o):
    """Packed bits equal numpy's little-endian unpacking of (Delta >= 0)."""
    w_base, w_ft = synth.layer(37, 200, seed=3, index=5)
    signs, _ = o.compress(w_base, w_ft)
    assert signs.shape == (37, 25)
    d = w_ft - synth.bf16_bits_to_f32(w_base)  # numpy fp32 subtract
    bits = np.unpackbits(signs, axis=1, bitorder="little")
    assert np.array_equal(bits.astype(bool), d >= 0)


def pin_alpha_exact_mean(o):
    """alpha_r is the mean |Delta| rounded to fp32: compare with an exact sum
    (math.fsum) divided by C.  fp64 accumulation may straddle a rounding
    boundary only rarely, so: all within 1 ulp, nearly all exact."""
    for (R, C, seed) in ((64, 4096, 11), (256, 512, 0), (16, 28672, 12)):
        w_base, w_ft = synth.layer(R, C, seed=seed)
        _, alpha, sums = o.compress(w_base, w_ft, return_row_sums=True)
        d = np.abs(w_ft - synth.bf16_bits_to_f32(w_base)).astype(np.float64)
        exact = np.array([math.fsum(row) for row in d])
        ref = (exact / C).astype(np.float32)
        ud = _ulp_diff_f32(alpha, ref)
        assert ud.max() <= 1, ud.max()
        assert (ud == 0).mean() >= 0.98
        # the fp64 row sums are within C * 2^-52 relative of the exact sums
        assert np.all(np.abs(sums - exact) <= exact * C * 2.0 ** -52)
        _, am = o.compress(w_base, w_ft, per_matrix=True)
        tot = math.fsum(d.ravel()) / (R * C)
        assert _ulp_diff_f32(am, np.float32(tot)).max() <= 1


def pin_alpha_laplace(o):
    """Delta ~ Laplace(0, b) has E|Delta| = b and sd |Delta| = b, so every
    row's alpha_r / b - 1 is about N(0, 1/C): bound it by 6 / sqrt(C)."""
    b = 1e-3
    R, C = 64, 4096
    w_base = synth.to_bf16_bits(synth.normal_f32((R, C), 0.02, 5, 1))
    delta = synth.laplace_f32((R, C), b, 5, 2)
    w_ft = synth.bf16_bits_to_f32(w_base) + delta
    _, alpha = o.compress(w_base, w_ft)
    dev = np.abs(alpha / b - 1.0)
    assert dev.max() < 6.0 / math.sqrt(C), dev.max()
    assert abs(alpha.mean() / b - 1.0) < 6.0 / math.sqrt(R * C)


def pin_alpha_least_squares(o):
    """For the stored signs s, alpha minimises ||Delta - a s||^2 over scalar a
    (the derivative sum s (Delta - a s) vanishes at a = mean |Delta|)."""
    w_base, w_ft = synth.layer(8, 1024, seed=21)
    signs, alpha = o.compress(w_base, w_ft)
    d = (w_ft - synth.bf16_bits_to_f32(w_base)).astype(np.float64)
    s = np.unpackbits(signs, axis=1, bitorder="little").astype(np.float64) * 2 - 1
    for r in range(8):
        f = lambda a: float(np.sum((d[r] - a * s[r]) ** 2))  # noqa: E731
        a = float(alpha[r])
        assert f(a) <= f(a * (1 + 1e-4)) and f(a) <= f(a * (1 - 1e-4))
        grad = float(np.sum(s[r] * (d[r] - a * s[r])))
        assert abs(grad) <= 1e-6 * float(np.sum(np.abs(d[r])))


# -------------------------------------------------------------- reconstruct


def pin_reconstruct_hand_cases(o):
    g = _json("reconstruct_cases.json")
    for wb, ab, bit, exp, why in g["cases"]:
        w_base = np.full((1, 8), int(wb, 16), dtype=np.uint16)
        alpha = np.array([_f32_bits(ab)], dtype=np.float32)
        signs = np.array([[0xFF if bit else 0x00]], dtype=np.uint8)
        out = o.reconstruct(w_base, signs, alpha)
        assert np.all(out == int(exp, 16)), (why, hex(int(out[0, 0])))


def pin_reconstruct_vs_torch(o):
    """Random layer: W_eff equals torch's fp32 add + bf16 conversion of
    W_base + alpha_r * s (s from numpy's bit unpacking)."""
    import torch

    w_base, w_ft = synth.layer(96, 640, seed=4, index=3)
    signs, alpha = o.compress(w_base, w_ft)
    s = np.unpackbits(signs, axis=1, bitorder="little").astype(np.float32) * 2 - 1
    for per_matrix in (False, True):
        a = alpha if not per_matrix else o.compress(w_base, w_ft, per_matrix=True)[1]
        wf = torch.from_numpy(synth.bf16_bits_to_f32(w_base))
        av = torch.from_numpy(a.reshape(-1, 1) if not per_matrix else a.reshape(1, 1))
        ref = (wf + av * torch.from_numpy(s)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        got = o.reconstruct(w_base, signs, a, per_matrix=per_matrix)
        assert np.array_equal(got, ref)


# ------------------------------------------------------------------- linear


def pin_linear_exact_rational(o):
    """Tiny case: y64 equals the exact rational product (fractions) to within
    fp64 rounding of the sum, and the normaliser equals sum |x| |W_eff|."""
    M, R, C = 3, 5, 24
    w_base, w_ft = synth.layer(R, C, seed=8)
    x = synth.activations(M, C, seed=8)
    signs, alpha = o.compress(w_base, w_ft)
    weff = _torch_widen(o.reconstruct(w_base, signs, alpha)).astype(np.float64)
    xf = _torch_widen(x).astype(np.float64)
    y, sc = o.linear(x, w_base, signs, alpha)
    for m in range(M):
        for r in range(R):
            exact = sum(Fraction(float(xf[m, j])) * Fraction(float(weff[r, j])) for j in range(C))
            absum = sum(abs(Fraction(float(xf[m, j])) * Fraction(float(weff[r, j]))) for j in range(C))
            assert abs(Fraction(y[m, r]) - exact) <= absum * Fraction(C, 2 ** 52)
            assert abs(Fraction(sc[m, r]) - absum) <= absum * Fraction(C, 2 ** 52)


def pin_linear_vs_numpy(o):
    """Tiny single layer (256 x 512, 4 tokens): y64 equals numpy's float64
    matmul of x and torch-reconstructed W_eff, to fp64 rounding."""
    import torch

    w_base, w_ft = synth.layer(256, 512, seed=0)
    x = synth.activations(4, 512, seed=0)
    signs, alpha = o.compress(w_base, w_ft)
    s = np.unpackbits(signs, axis=1, bitorder="little").astype(np.float32) * 2 - 1
    weff = (torch.from_numpy(synth.bf16_bits_to_f32(w_base)) + torch.from_numpy(alpha).view(-1, 1)
            * torch.from_numpy(s)).to(torch.bfloat16).float().numpy().astype(np.float64)
    xf = _torch_widen(x).astype(np.float64)
    ref = xf @ weff.T
    y, sc = o.linear(x, w_base, signs, alpha)
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * (np.abs(xf) @ np.abs(weff).T).max())
    assert np.allclose(sc, np.abs(xf) @ np.abs(weff).T, rtol=1e-13)
    # selected rows in any order give the same columns
    rows = np.array([255, 3, 77, 3], dtype=np.int64)
    y2, _ = o.linear(x, w_base, signs, alpha, rows=rows)
    assert np.array_equal(y2, y[:, rows])


def dyadic_case(M: int, R: int, C: int, seed: int, n_variants: int = 1):
    """Exact-arithmetic inputs: W_base in {k 2^-8 : |k| <= 8}, alpha_r =
    (1 + (r + v) mod 4) 2^-8 for variant v, x in {-1, 0, 1} with at most 8
    non-zeros per row.  Every product and partial sum is exact in fp32 and
    |y| 2^8 <= 8 * 12 = 96 < 256, so y is exact in bf16 whatever the order."""
    u = synth.u64((R, C), seed, 7001)
    k = (u % np.uint64(17)).astype(np.int64) - 8
    w_base = synth.to_bf16_bits((k * 2.0 ** -8).astype(np.float32))
    sign_bytes = synth.u64((n_variants, R, C // 8), seed, 7002).astype(np.uint8)
    alpha = np.stack([((1 + (np.arange(R) + v) % 4) * 2.0 ** -8).astype(np.float32)
                      for v in range(n_variants)])
    x = np.zeros((M, C), dtype=np.float32)
    cols = synth.u64((M, 8), seed, 7003) % np.uint64(C)
    vals = (synth.u64((M, 8), seed, 7004) % np.uint64(3)).astype(np.float32) - 1
    for m in range(M):
        for t in range(8):
            x[m, int(cols[m, t])] = vals[m, t]
    return synth.to_bf16_bits(x), w_base, k, sign_bytes, alpha


def pin_linear_dyadic(o):
    """Exact inputs: y64 equals the integer-arithmetic product exactly."""
    M, R, C = 6, 40, 64
    x, w_base, k, sb, alpha = dyadic_case(M, R, C, seed=31)
    signs, a = sb[0], alpha[0]
    y, _ = o.linear(x, w_base, signs, a)
    s = np.unpackbits(signs, axis=1, bitorder="little").astype(np.int64) * 2 - 1
    wq = k + (1 + np.arange(R)[:, None] % 4) * s        # W_eff * 2^8, integers
    xi = synth.bf16_bits_to_f32(x).astype(np.int64)
    assert np.array_equal(y * 256.0, (xi @ wq.T).astype(np.float64))


# ------------------------------------------------------------------ grouped


def pin_grouped(o):
    """Grouped = per-token linear with that token's variant; ids out of range
    give zero rows; the result is equivariant under token permutation."""
    V, M, R, C = 3, 9, 20, 32
    w_base = synth.to_bf16_bits(synth.normal_f32((R, C), 0.02, 9, 1))
    signs = np.zeros((V, R, C // 8), dtype=np.uint8)
    alpha = np.zeros((V, R), dtype=np.float32)
    for v in range(V):
        w_ft = synth.variant_ft(w_base, v, b=1e-3 * (v + 1), seed=9)
        signs[v], alpha[v] = o.compress(w_base, w_ft)
    x = synth.activations(M, C, seed=9)
    ids = np.array([0, 2, 1, 5, 0, -1, 2, 2, 1], dtype=np.int32)
    y, sc = o.linear_grouped(x, ids, w_base, signs, alpha)
    for m in range(M):
        v = ids[m]
        if 0 <= v < V:
            ym, _ = o.linear(x[m:m + 1], w_base, signs[v], alpha[v])
            assert np.array_equal(y[m], ym[0])
            # the variant's own deltas matter: another variant gives another row
            yo, _ = o.linear(x[m:m + 1], w_base, signs[(v + 1) % V], alpha[(v + 1) % V])
            assert not np.array_equal(ym, yo)
        else:
            assert np.all(y[m] == 0) and np.all(sc[m] == 0)
    perm = np.array([4, 2, 8, 0, 1, 7, 3, 6, 5])
    yp, _ = o.linear_grouped(x[perm], ids[perm], w_base, signs, alpha)
    assert np.array_equal(yp, y[perm])
    # per-matrix alpha: alpha [V]
    am = np.array([alpha[v].mean() for v in range(V)], dtype=np.float32)
    y3, _ = o.linear_grouped(x, ids, w_base, signs, am, per_matrix=True)
    for m in (0, 1, 2):
        ym, _ = o.linear(x[m:m + 1], w_base, signs[ids[m]], am[ids[m]:ids[m] + 1], per_matrix=True)
        assert np.array_equal(y3[m], ym[0])


def pin_shape_4096(o):
    """A 4096 x 4096 layer packs to a [4096, 512] byte tensor ('Infrastructure
    Details' storage format)."""
    R = C = 4096
    w_base = np.zeros((R, C), dtype=np.uint16)
    w_ft = np.zeros((R, C), dtype=np.float32)
    signs, alpha = o.compress(w_base, w_ft)
    assert signs.shape == (4096, 512) and signs.dtype == np.uint8
    assert np.all(signs == 0xFF) and np.all(alpha == 0)


STACK_SHAPES = {"q": (8192, 8192), "k": (1024, 8192), "v": (1024, 8192), "o": (8192, 8192),
                "gate": (28672, 8192), "up": (28672, 8192), "down": (8192, 28672)}
STACK_LAYERS = 80


def _sign_bytes_written(o, R, C):
    """Bytes of packed signs the C oracle writes for an R x C matrix whose
    deltas are all >= 0, counted in a buffer with a sentinel tail (the
    wrapper's own allocation is bypassed, so an oracle that wrote more or
    fewer than one bit per weight shows here)."""
    import ctypes

    w_base = np.zeros((R, C), dtype=np.uint16)
    w_ft = np.zeros((R, C), dtype=np.float32)
    n = R * C // 8
    buf = np.full(n + 4096, 0xA5, dtype=np.uint8)
    alpha = np.zeros(R, dtype=np.float32)
    sums = np.zeros(R, dtype=np.float64)
    P = ctypes.c_void_p
    rc = o.lib.oracle_compress(w_base.ctypes.data_as(P), w_ft.ctypes.data_as(P), 1, R, C, 0,
                               buf.ctypes.data_as(P), alpha.ctypes.data_as(P), sums.ctypes.data_as(P))
    assert rc == 0
    assert np.all(buf[n:] == 0xA5), "the oracle wrote past one bit per weight"
    written = int(np.count_nonzero(buf[:n] == 0xFF))
    assert written == n, "the oracle left part of the packed code unwritten"
    return written


def pin_storage_arithmetic(o):
    """The post's storage arithmetic ("Mathematical Foundation"): a 70B model
    in bf16 is 140 GB; fourteen full copies are 1.96 TB; one bit per weight is
    8.75 GB per variant, so the base plus 14 delta sets is 262.5 GB, 86.6%
    less ("-87%").  The oracle's packed code holds exactly one bit per weight
    on every matrix shape of the 70B-shaped stack (80 layers of q, k, v, o,
    gate, up, down, counted with a sentinel past the code), so one variant of
    the stack's 68,451,041,280 weights is 8,556,380,160 sign bytes; its fp32
    alpha per output row adds 26,869,760 bytes, 0.31% of the signs (32/d_in,
    not the post's 'about 0.1%', a reading recorded in the design notes)."""
    n = 70e9
    assert n * 2 == 140e9
    assert n / 8 == 8.75e9
    assert 14 * n * 2 == 1.96e12
    total = n * 2 + 14 * n / 8
    assert total == 262.5e9
    assert round(100 * (1 - total / 1.96e12), 1) == 86.6
    per_row = {}
    for d_out, d_in in set(STACK_SHAPES.values()):
        per_row[d_in] = _sign_bytes_written(o, 2, d_in) // 2
        assert per_row[d_in] * 8 == d_in
    params = STACK_LAYERS * sum(d_out * d_in for d_out, d_in in STACK_SHAPES.values())
    sign_bytes = STACK_LAYERS * sum(d_out * per_row[d_in] for d_out, d_in in STACK_SHAPES.values())
    assert params == 68_451_041_280
    assert sign_bytes == 8_556_380_160 == params // 8
    alpha_bytes = STACK_LAYERS * sum(4 * d_out for d_out, _ in STACK_SHAPES.values())
    assert alpha_bytes == 26_869_760
    assert round(100 * alpha_bytes / sign_bytes, 2) == 0.31
    # the post's [4096, 4096] -> [4096, 512] example ("Infrastructure Details")
    assert _sign_bytes_written(o, 4096, 4096) == 4096 * 512
    # "1/32 of the full-precision delta": the packed code of a matrix is
    # exactly 1/32 of its fp32 delta (1/16 of a bf16 one) on every shape
    for d_out, d_in in set(STACK_SHAPES.values()):
        code = per_row[d_in] * d_out
        assert 32 * code == 4 * d_out * d_in and 16 * code == 2 * d_out * d_in
    for d_out, d_in in ((4096, 4096), (3, 8), (5, 1032)):
        code = _sign_bytes_written(o, d_out, d_in)
        assert 32 * code == 4 * d_out * d_in and 16 * code == 2 * d_out * d_in


# --------------------------------------------------------------- similarity


def _sim_case(V, R, C, seed, dyadic):
    sb = synth.u64((V, R, C // 8), seed, 7101).astype(np.uint8)
    if dyadic:   # alpha = k 2^-10, k in 1..16: every product and sum below is exact in fp64
        alpha = ((1 + synth.u64((V, R), seed, 7102) % np.uint64(16)).astype(np.float64) * 2.0 ** -10).astype(np.float32)
    else:
        alpha = np.abs(synth.normal_f32((V, R), 1e-3, seed, 7103)).astype(np.float32) + np.float32(1e-5)
    return sb, alpha


def _unpack_pm1(sb):
    """+-1 as int64 from packed bytes, LSB first (numpy's little-endian unpacking)."""
    bits = np.unpackbits(sb, axis=-1, bitorder="little").astype(np.int64)
    return 2 * bits - 1


def pin_similarity_exact_rational(o):
    """K-Merge's cosine similarity of task vectors: with dyadic alpha the Gram
    matrix is exact, so it must equal the exact rational sum over every weight
    of tau_a tau_b (tau = alpha * s), per-row and per-matrix alpha; the
    cosines match the exact value to fp64 rounding."""
    V, R, C = 3, 7, 24
    sb, alpha = _sim_case(V, R, C, seed=51, dyadic=True)
    s = _unpack_pm1(sb)
    for per_matrix in (False, True):
        al = alpha[:, 0].copy() if per_matrix else alpha
        gram, cos = o.similarity(sb, al, per_matrix=per_matrix)
        for a in range(V):
            for b in range(V):
                exact = Fraction(0)
                for r in range(R):
                    fa = Fraction(float(al[a] if per_matrix else al[a, r]))
                    fb = Fraction(float(al[b] if per_matrix else al[b, r]))
                    exact += fa * fb * int(np.dot(s[a, r], s[b, r]))
                assert gram[a, b] == float(exact), (per_matrix, a, b)
        for a in range(V):
            for b in range(V):
                ref = float(gram[a, b]) / math.sqrt(float(gram[a, a]) * float(gram[b, b]))
                assert abs(cos[a, b] - ref) <= 2 * np.spacing(abs(ref) + 1e-300)


def pin_similarity_vs_numpy(o):
    """Random alpha, rows past 256 (every partial visited twice): the Gram
    matrix agrees with numpy's float64 einsum over the unpacked task vectors
    to a relative 1e-12 (a different summation order)."""
    V, R, C = 4, 300, 64
    sb, alpha = _sim_case(V, R, C, seed=52, dyadic=False)
    tau = alpha.astype(np.float64)[:, :, None] * _unpack_pm1(sb).astype(np.float64)
    ref = np.einsum("arj,brj->ab", tau, tau)
    gram, cos = o.similarity(sb, alpha)
    assert np.allclose(gram, ref, rtol=1e-12, atol=0)
    nrm = np.sqrt(np.diag(ref))
    assert np.allclose(cos, ref / nrm[:, None] / nrm[None, :], rtol=1e-12, atol=1e-15)


def pin_similarity_invariants(o):
    """Symmetry, unit self-similarity, -1 for the complementary sign pattern
    with the same alpha, equivariance under a permutation of the variants,
    and near-zero cosine for independent random signs."""
    V, R, C = 5, 40, 128
    sb, alpha = _sim_case(V, R, C, seed=53, dyadic=False)
    sb[3] = ~sb[0]
    alpha[3] = alpha[0]
    gram, cos = o.similarity(sb, alpha)
    assert np.array_equal(gram, gram.T)
    assert np.all(np.abs(np.diag(cos) - 1.0) <= 2.0 ** -52)
    assert gram[0, 3] == -gram[0, 0] and abs(cos[0, 3] + 1.0) <= 2.0 ** -52
    perm = np.array([2, 4, 0, 1, 3])
    gp, _ = o.similarity(sb[perm], alpha[perm])
    assert np.array_equal(gp, gram[np.ix_(perm, perm)])
    for a, b in ((0, 1), (1, 2), (2, 4)):
        assert abs(cos[a, b]) < 6.0 / math.sqrt(R * C)


# ------------------------------------------- similarity of full task vectors


def _delta_case(V, R, C, seed, dyadic, ft_bf16=False):
    """W_base and V fine-tuned copies.  dyadic: W_base = k 2^-8 (|k| <= 8) and
    Delta = k 2^-10 (|k| <= 8), so every difference, product and sum below is
    exact; otherwise W_base ~ N(0, 0.02) bf16 and Delta ~ Laplace(0, b) with a
    different b per variant (fp32 W_ft = fl32(W_base + Delta))."""
    if dyadic:
        kb = (synth.u64((R, C), seed, 7201) % np.uint64(17)).astype(np.int64) - 8
        base = (kb * 2.0 ** -8).astype(np.float32)
        kd = (synth.u64((V, R, C), seed, 7202) % np.uint64(17)).astype(np.int64) - 8
        ft = (base[None] + (kd * 2.0 ** -10)).astype(np.float32)
        wb = _torch_bf16_bits(base)
        return wb, (_torch_bf16_bits(ft) if ft_bf16 else ft)
    wb = synth.to_bf16_bits(synth.normal_f32((R, C), 0.02, seed, 7203))
    base = synth.bf16_bits_to_f32(wb)
    fts = []
    for v in range(V):
        d = synth.laplace_f32((R, C), 1e-3 * (1 + v), seed, 7204 + v)
        fts.append((base + d).astype(np.float32))
    ft = np.stack(fts)
    return wb, (_torch_bf16_bits(ft) if ft_bf16 else ft)


def _deltas64(wb, ft):
    """Delta = fl32(W_ft - W_base) by numpy's IEEE fp32 subtraction, as fp64."""
    base = synth.bf16_bits_to_f32(wb)
    f = synth.bf16_bits_to_f32(ft) if ft.dtype == np.uint16 else ft
    return (f - base[None]).astype(np.float32).astype(np.float64)


def pin_similarity_delta_exact_rational(o):
    """K-Merge's similarity over the task vector Delta = W_ft - W_base: on
    dyadic inputs every difference, product and partial sum is exact, so the
    Gram matrix must equal the exact rational sum of Delta_a Delta_b over every
    weight (fp32 and bf16 W_ft), and the cosines the exact ratio to fp64
    rounding."""
    V, R, C = 3, 5, 24
    for ft_bf16 in (False, True):
        wb, ft = _delta_case(V, R, C, seed=61, dyadic=True, ft_bf16=ft_bf16)
        base = [Fraction(float(v)) for v in synth.bf16_bits_to_f32(wb).ravel()]
        f = synth.bf16_bits_to_f32(ft) if ft_bf16 else ft
        d = [[Fraction(float(x)) - base[i] for i, x in enumerate(f[v].ravel())] for v in range(V)]
        gram, cos = o.similarity_delta(wb, ft)
        for a in range(V):
            for b in range(V):
                exact = sum((d[a][i] * d[b][i] for i in range(R * C)), Fraction(0))
                assert gram[a, b] == float(exact), (ft_bf16, a, b)
        for a in range(V):
            for b in range(V):
                ref = float(gram[a, b]) / math.sqrt(float(gram[a, a]) * float(gram[b, b]))
                assert abs(cos[a, b] - ref) <= 2 * np.spacing(abs(ref) + 1e-300)


def pin_similarity_delta_rounding_bound(o):
    """Random Laplace deltas over 300 rows of 1024 columns (every one of the
    64 column partials and the 256 row partials visited at least twice): each
    Gram entry lies within the worst-case rounding of its summation tree of
    the correctly rounded exact sum (math.fsum of the exact fp64 products),
    and agrees with numpy's float64 einsum over the fp32 differences to a
    relative 1e-12."""
    V, R, C = 3, 300, 1024
    wb, ft = _delta_case(V, R, C, seed=62, dyadic=False)
    d = _deltas64(wb, ft)
    gram, cos = o.similarity_delta(wb, ft)
    depth = (C // 8) // 64 * 8 + 6 + (R + 255) // 256 + 8 + 1
    for a in range(V):
        for b in range(V):
            prods = (d[a] * d[b]).ravel()
            exact = math.fsum(prods)
            bound = depth * 2.0 ** -53 * float(np.sum(np.abs(prods)))
            assert abs(gram[a, b] - exact) <= bound, (a, b, gram[a, b], exact, bound)
    ref = np.einsum("arj,brj->ab", d, d)
    assert np.allclose(gram, ref, rtol=1e-12, atol=0)
    nrm = np.sqrt(np.diag(ref))
    assert np.allclose(cos, ref / nrm[:, None] / nrm[None, :], rtol=1e-12, atol=1e-15)


def pin_similarity_delta_invariants(o):
    """Symmetry, unit self-similarity, -1 for the negated delta, +1 and four
    times the squared norm for the doubled delta (exact on dyadic inputs),
    equivariance under a permutation of the variants, near-zero cosine for
    independent Laplace deltas."""
    V, R, C = 4, 40, 136
    wb, ft = _delta_case(V, R, C, seed=63, dyadic=True)
    base = synth.bf16_bits_to_f32(wb)
    ft[2] = (base - (ft[0] - base)).astype(np.float32)          # Delta_2 = -Delta_0
    ft[3] = (base + 2 * (ft[0] - base)).astype(np.float32)      # Delta_3 = 2 Delta_0
    gram, cos = o.similarity_delta(wb, ft)
    assert np.array_equal(gram, gram.T)
    assert np.all(np.abs(np.diag(cos) - 1.0) <= 2.0 ** -52)
    assert gram[0, 2] == -gram[0, 0] and abs(cos[0, 2] + 1.0) <= 2.0 ** -52
    assert gram[3, 3] == 4 * gram[0, 0] and abs(cos[0, 3] - 1.0) <= 2.0 ** -52
    perm = np.array([2, 0, 3, 1])
    gp, _ = o.similarity_delta(wb, ft[perm])
    assert np.array_equal(gp, gram[np.ix_(perm, perm)])
    wb2, ft2 = _delta_case(3, 64, 256, seed=64, dyadic=False)
    _, c2 = o.similarity_delta(wb2, ft2)
    for a, b in ((0, 1), (1, 2)):
        assert abs(c2[a, b]) < 6.0 / math.sqrt(64 * 256)


def pin_similarity_delta_matches_code(o):
    """A delta of one magnitude per row (Delta = alpha_r s, alpha_r dyadic) is
    exactly what the 1-bit code stores: compress gives back alpha_r and s, and
    the Gram matrix of the full task vectors then equals the Gram matrix of
    the code (a second oracle function), bit for bit."""
    V, R, C = 3, 20, 64
    kb = (synth.u64((R, C), 65, 7205) % np.uint64(17)).astype(np.int64) - 8
    base = (kb * 2.0 ** -8).astype(np.float32)
    wb = _torch_bf16_bits(base)
    alpha = ((1 + synth.u64((V, R), 65, 7206) % np.uint64(8)).astype(np.float64) * 2.0 ** -11).astype(np.float32)
    s = 2.0 * (synth.u64((V, R, C), 65, 7207) % np.uint64(2)).astype(np.float64) - 1.0
    ft = (base[None] + alpha[:, :, None] * s).astype(np.float32)
    signs, alphas = [], []
    for v in range(V):
        sv, av = o.compress(wb, ft[v])
        assert np.array_equal(av, alpha[v])
        signs.append(sv)
        alphas.append(av)
    g_code, c_code = o.similarity(np.stack(signs), np.stack(alphas))
    g_full, c_full = o.similarity_delta(wb, ft)
    assert np.array_equal(g_code, g_full)
    assert np.array_equal(c_code, c_full)


def _orthonormal(rng, n, k):
    q, _ = np.linalg.qr(rng.standard_normal((n, k)))
    return q


def _bf16_normal(rng, shape, std):
    return _torch_bf16_bits((std * rng.standard_normal(shape)).astype(np.float32))


def pin_monosoup_known_svd(o):
    """MonoSoup's rank-r truncation on task vectors built with a known SVD
    (orthonormal U, V from a QR, distinct singular values): the singular
    values come back in decreasing order, the merge of k = 1 equals W_base +
    U_r S_r V_r^T, and with two checkpoints the merge is W_base plus the mean
    of the two closed-form truncations.  Tall and wide shapes; W_base nonzero,
    so the task vector must be W_i - W_base.  Tolerances: fp32 rounding of W_i
    (the task vector is the fp32 difference)."""
    rng = np.random.default_rng(61)
    for R, C in ((48, 20), (18, 40)):
        n = min(R, C)
        wb = _bf16_normal(rng, (R, C), 0.02)
        base = _torch_widen(wb).astype(np.float64)
        s = np.sort(rng.uniform(0.1, 1.0, n))[::-1] * np.geomspace(1.0, 0.05, n)
        taus, wfs, sig_true = [], [], []
        for _ in range(2):
            U, V = _orthonormal(rng, R, n), _orthonormal(rng, C, n)
            si = s * rng.uniform(0.9, 1.1)
            wfs.append((base + (U * si) @ V.T).astype(np.float32))
            taus.append(lambda r, U=U, V=V, si=si: (U[:, :r] * si[:r]) @ V[:, :r].T)
            sig_true.append(si)
        for r in (1, 3, n - 2):
            m1, sig = o.monosoup(wb, wfs[0][None], r)
            assert np.allclose(sig[0], sig_true[0], rtol=0, atol=2e-6), r
            assert np.all(np.diff(sig[0]) <= 0)
            assert np.abs(m1 - (base + taus[0](r))).max() <= 2e-6, r
            m2, sig2 = o.monosoup(wb, np.stack(wfs), r)
            assert np.allclose(sig2[1], sig_true[1], rtol=0, atol=2e-6), r
            assert np.abs(m2 - (base + 0.5 * (taus[0](r) + taus[1](r)))).max() <= 2e-6, r


def pin_monosoup_vs_numpy(o):
    """Full-rank random task vectors, k = 3, rank 4: the merge equals
    W_base + (1/3) sum_i U_i,4 S_i,4 Vh_i,4 from numpy's LAPACK SVD of the same
    fp32 differences, to a relative 1e-10; the singular values match numpy's."""
    rng = np.random.default_rng(62)
    R, C, k, r = 30, 26, 3, 4
    wb = _bf16_normal(rng, (R, C), 0.02)
    base = _torch_widen(wb)
    wf = (base[None] + 1e-3 * rng.standard_normal((k, R, C))).astype(np.float32)
    m, sig = o.monosoup(wb, wf, r)
    acc = np.zeros((R, C))
    for i in range(k):
        d = (wf[i] - base).astype(np.float64)     # fp32 subtraction, then widened
        u, sv, vh = np.linalg.svd(d, full_matrices=False)
        assert np.allclose(sig[i], sv, rtol=1e-12, atol=1e-18)
        acc += (u[:, :r] * sv[:r]) @ vh[:r]
    ref = base.astype(np.float64) + acc / k
    scale = np.abs(acc / k).max()
    assert np.abs(m - ref).max() <= 1e-10 * scale


def pin_monosoup_special_cases(o):
    """Rank 0 gives W_base exactly; full rank with k = 1 gives W_base plus the
    whole fp32 difference (every component kept); k identical checkpoints merge as one; Eckart-Young: the
    squared residual of the rank-r truncation equals the sum of the dropped
    squared singular values; the frobenius norm of Delta equals the norm of
    its singular values."""
    rng = np.random.default_rng(63)
    R, C = 21, 17
    wb = _bf16_normal(rng, (R, C), 0.02)
    base = _torch_widen(wb).astype(np.float64)
    wf = (base + 1e-3 * rng.standard_normal((R, C))).astype(np.float32)
    d = (wf - base.astype(np.float32)).astype(np.float64)    # the fp32 difference
    m0, _ = o.monosoup(wb, wf[None], 0)
    assert np.array_equal(m0, base)
    mf, sig = o.monosoup(wb, wf[None], min(R, C))
    assert np.abs(mf - (base + d)).max() <= 1e-15
    assert abs(np.sqrt(np.sum(sig[0] ** 2)) - np.linalg.norm(d)) <= 1e-13 * np.linalg.norm(d)
    for r in (2, 9):
        m1, _ = o.monosoup(wb, wf[None], r)
        m3, _ = o.monosoup(wb, np.stack([wf, wf, wf]), r)
        assert np.abs(m3 - m1).max() <= 1e-16
        resid = np.sum((d - (m1 - base)) ** 2)
        assert abs(resid - np.sum(sig[0][r:] ** 2)) <= 1e-10 * np.sum(d ** 2)


ALL = [pin_bf16_widen, pin_bf16_round, pin_bf16_hand_ties, pin_compress_handbuilt,
       pin_compress_packing_vs_numpy, pin_alpha_exact_mean, pin_alpha_laplace,
       pin_alpha_least_squares, pin_reconstruct_hand_cases, pin_reconstruct_vs_torch,
       pin_linear_exact_rational, pin_linear_vs_numpy, pin_linear_dyadic, pin_grouped,
       pin_shape_4096, pin_storage_arithmetic, pin_similarity_exact_rational, pin_similarity_vs_numpy, pin_similarity_invariants,
       pin_similarity_delta_exact_rational, pin_similarity_delta_rounding_bound, pin_similarity_delta_invariants,
       pin_similarity_delta_matches_code,
       pin_monosoup_known_svd, pin_monosoup_vs_numpy, pin_monosoup_special_cases]
