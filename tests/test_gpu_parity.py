"""GPU tier: the HIP path against the oracle, through the C ABI.

compress / pack / reconstruct must match bit for bit; linear outputs must meet
the official normalised tolerance (1e-2) and the tight bound of gpu_util,
and the exact-arithmetic cases (identity / one-hot x, dyadic inputs) must
match bit for bit, because the official tolerance alone cannot see the deltas.
Inputs are seeded synthetic tensors with the laws of the post's 70B-class
workloads (see synth).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import pins
from tests.gpu_util import (bf16_dev, check_linear, f32_dev, host, host_bits, i32_dev, same_bits_pm0,
                            u8_dev)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def bd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tenant_fine_tune_amd as bd

    return bd


def _bits32(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


# ------------------------------------------------------------------ compress

# includes rows of 2048..8192 columns (1..4 whole groups per thread) and row counts that are
# not a multiple of 4
COMPRESS_SHAPES = [(256, 512), (5, 24), (1, 8), (3, 2056), (64, 28672), (300, 4096), (4096, 4096),
                   (7, 2048), (13, 6144), (10, 8192), (301, 4096)]


@pytest.mark.parametrize("ft_bf16", [False, True], ids=["ft_f32", "ft_bf16"])
@pytest.mark.parametrize("per_matrix", [False, True], ids=["alpha_row", "alpha_matrix"])
@pytest.mark.parametrize("shape", COMPRESS_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_compress_bit_exact(bd, shape, per_matrix, ft_bf16):
    R, C = shape
    w_base, w_ft = synth.layer(R, C, seed=0, index=R % 61 + C % 53, ft_bf16=ft_bf16)
    so, ao = oracle.compress(w_base, w_ft, per_matrix=per_matrix)
    ft_dev = bf16_dev(w_ft) if ft_bf16 else f32_dev(w_ft)
    sg, ag = bd.compress(bf16_dev(w_base), ft_dev, per_matrix=per_matrix)
    torch.cuda.synchronize()
    assert np.array_equal(host(sg), so)
    assert np.array_equal(_bits32(host(ag)), _bits32(ao))


def test_compress_handbuilt(bd):
    g = json.load(open(os.path.join(GOLDEN, "compress_4x16.json")))
    w_base, w_ft = pins._handbuilt_4x16()
    sg, ag = bd.compress(bf16_dev(w_base), f32_dev(w_ft))
    assert host(sg).tolist() == g["expected_signs"]
    assert host(ag).tolist() == g["expected_alpha_row"]
    _, am = bd.compress(bf16_dev(w_base), f32_dev(w_ft), per_matrix=True)
    assert host(am).tolist() == [g["expected_alpha_matrix"]]


def test_compress_deterministic(bd):
    w_base, w_ft = synth.layer(512, 4096, seed=1)
    a = bd.compress(bf16_dev(w_base), f32_dev(w_ft), per_matrix=True)
    b = bd.compress(bf16_dev(w_base), f32_dev(w_ft), per_matrix=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# --------------------------------------------------------------- reconstruct

RECON_SHAPES = [(256, 512), (5, 24), (3, 2056), (300, 4096), (2048, 8192)]


@pytest.mark.parametrize("per_matrix", [False, True], ids=["alpha_row", "alpha_matrix"])
@pytest.mark.parametrize("shape", RECON_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_reconstruct_bit_exact(bd, shape, per_matrix):
    R, C = shape
    w_base, w_ft = synth.layer(R, C, seed=2, index=R % 61)
    so, ao = oracle.compress(w_base, w_ft, per_matrix=per_matrix)
    wo = oracle.reconstruct(w_base, so, ao, per_matrix=per_matrix)
    wg = bd.reconstruct(bf16_dev(w_base), u8_dev(so), f32_dev(ao), per_matrix=per_matrix)
    assert np.array_equal(host_bits(wg), wo)


def test_reconstruct_hand_cases(bd):
    g = json.load(open(os.path.join(GOLDEN, "reconstruct_cases.json")))
    cases = g["cases"]
    n = len(cases)
    w_base = np.array([[int(c[0], 16)] * 8 for c in cases], dtype=np.uint16)
    alpha = np.array([int(c[1], 16) for c in cases], dtype=np.uint32).view(np.float32)
    signs = np.array([[0xFF if c[2] else 0x00] for c in cases], dtype=np.uint8)
    wg = host_bits(bd.reconstruct(bf16_dev(w_base), u8_dev(signs), f32_dev(alpha), per_matrix=False))
    for i in range(n):
        assert np.all(wg[i] == int(cases[i][3], 16)), (cases[i][4], hex(int(wg[i, 0])))


# -------------------------------------------------------------------- linear


def _layer_dev(R, C, seed, index=0, b=1e-3, per_matrix=False):
    w_base, w_ft = synth.layer(R, C, seed=seed, index=index, b=b)
    so, ao = oracle.compress(w_base, w_ft, per_matrix=per_matrix)
    return w_base, so, ao, (bf16_dev(w_base), u8_dev(so), f32_dev(ao))


DECODE_CASES = [((256, 512), m) for m in (1, 2, 3, 4, 5, 8, 9, 16)] + \
               [((4096, 4096), m) for m in (1, 4, 16)] + \
               [((300, 200), 3), ((7, 8), 16), ((1000, 1032), 7), ((33, 24), 1)] + \
               [((1000, 1024), 9), ((512, 8192), 16), ((1000, 28672), 16), ((300, 28672), 1),  # the kernels' steady loops, D = 1
                ((300, 28672), 4), ((40, 8704), 2), ((1000, 6144), 12)] + \
               [((1000, 4096), 13), ((33, 8192), 5), ((24, 4096), 16), ((7, 12288), 8)] + \
               [((1024, 8192), 8), ((2048, 8192), 5), ((1000, 28672), 3), ((1025, 12288), 16)]  # row steps in parts


@pytest.mark.parametrize("per_matrix", [False, True], ids=["alpha_row", "alpha_matrix"])
@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"{c[0][0]}x{c[0][1]}_m{c[1]}")
def test_linear_decode(bd, case, per_matrix):
    (R, C), M = case
    w_base, so, ao, (wd, sd, ad) = _layer_dev(R, C, seed=3, index=M, per_matrix=per_matrix)
    x = synth.activations(M, C, seed=3, index=M)
    y = bd.linear(bf16_dev(x), wd, sd, ad, per_matrix=per_matrix)
    y64, sc = oracle.linear(x, w_base, so, ao, per_matrix=per_matrix)
    check_linear(host_bits(y), y64, sc, f"decode {R}x{C} m={M}")


PREFILL_CASES = [((256, 512), 17), ((256, 512), 64), ((256, 512), 256), ((256, 512), 300),
                 ((300, 200), 257), ((1000, 1032), 513), ((520, 64), 40), ((64, 4096), 600),
                 # split-K: few output tiles, K cut into 2..16 ranges
                 ((200, 4096), 64), ((520, 1024), 300), ((1024, 8192), 40), ((300, 2112), 17 + 256),
                 # eight-wave kernel (d_out a multiple of 32) with ragged tiles and token counts
                 ((224, 4096), 64), ((544, 1024), 300), ((288, 2112), 17 + 256), ((96, 640), 33)]


@pytest.mark.parametrize("per_matrix", [False, True], ids=["alpha_row", "alpha_matrix"])
@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: f"{c[0][0]}x{c[0][1]}_m{c[1]}")
def test_linear_prefill(bd, case, per_matrix):
    (R, C), M = case
    w_base, so, ao, (wd, sd, ad) = _layer_dev(R, C, seed=4, index=M % 61, per_matrix=per_matrix)
    x = synth.activations(M, C, seed=4, index=M % 61)
    y = bd.linear(bf16_dev(x), wd, sd, ad, per_matrix=per_matrix)
    y64, sc = oracle.linear(x, w_base, so, ao, per_matrix=per_matrix)
    check_linear(host_bits(y), y64, sc, f"prefill {R}x{C} m={M}")


def test_linear_3d_input_and_determinism(bd):
    R, C = 256, 512
    w_base, so, ao, (wd, sd, ad) = _layer_dev(R, C, seed=5)
    x = synth.activations(2 * 150, C, seed=5)
    xd = bf16_dev(x).view(2, 150, C)
    y1 = bd.linear(xd, wd, sd, ad)
    y2 = bd.linear(xd, wd, sd, ad)
    assert y1.shape == (2, 150, R)
    assert torch.equal(y1, y2)
    y64, sc = oracle.linear(x, w_base, so, ao)
    check_linear(host_bits(y1.view(300, R)), y64, sc, "3d input")


# (m, d_in): d_in = 1032 takes the ragged-step kernels; (4, 4096), (2, 512) and
# (3, 8704), whole 512-column steps with x small enough to sit in LDS; (16, 8192)
# and (3, 28672) on 1000 rows, the whole-row kernel with the row's steps in parts
@pytest.mark.parametrize("M,C", [(1, 1032), (16, 1032), (4, 4096), (2, 512), (3, 8704), (16, 8192), (3, 28672)],
                         ids=lambda v: str(v))
def test_identity_decode(bd, M, C):
    """One-hot x: y[t, r] must equal W_eff[r, j_t] bit for bit."""
    R = 1000
    w_base, so, ao, (wd, sd, ad) = _layer_dev(R, C, seed=6)
    weff = oracle.reconstruct(w_base, so, ao)
    cols = np.linspace(0, C - 1, M).astype(int)
    x = np.zeros((M, C), dtype=np.float32)
    x[np.arange(M), cols] = 1.0
    y = host_bits(bd.linear(bf16_dev(synth.to_bf16_bits(x)), wd, sd, ad))
    assert same_bits_pm0(y, weff[:, cols].T)


@pytest.mark.parametrize("shape", [(384, 512), (300, 264)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_identity_prefill(bd, shape):
    """x = I (m = d_in tokens): y = W_eff^T bit for bit."""
    R, C = shape
    w_base, so, ao, (wd, sd, ad) = _layer_dev(R, C, seed=7)
    weff = oracle.reconstruct(w_base, so, ao)
    eye = synth.to_bf16_bits(np.eye(C, dtype=np.float32))
    y = host_bits(bd.linear(bf16_dev(eye), wd, sd, ad))
    assert same_bits_pm0(y, weff.T)


@pytest.mark.parametrize("M,C", [(1, 256), (5, 256), (16, 256), (40, 256), (300, 256), (4, 2048), (2, 512),
                                 (3, 4096)], ids=lambda v: str(v))
def test_dyadic_exact(bd, M, C):
    """Exact-arithmetic inputs: every sign bit and alpha shows in y, bit for bit."""
    R = 200
    x, w_base, _, sb, alpha = pins.dyadic_case(M, R, C, seed=40 + M)
    y = host_bits(bd.linear(bf16_dev(x), bf16_dev(w_base), u8_dev(sb[0]), f32_dev(alpha[0])))
    y64, _ = oracle.linear(x, w_base, sb[0], alpha[0])
    assert np.array_equal(synth.bf16_bits_to_f32(y).astype(np.float64), y64)


@pytest.mark.parametrize("case", [((224, 4096), 64), ((1024, 8192), 40), ((256, 2048), 300)],
                         ids=lambda c: f"{c[0][0]}x{c[0][1]}_m{c[1]}")
def test_split_k_dyadic_exact(bd, case):
    """Split-K shapes on exact-arithmetic inputs: y bit for bit, and the
    fixed-order reduce gives the same bits on every call."""
    (R, C), M = case
    assert bd.lib.bitdelta_linear_workspace(M, R, C) > 0
    x, w_base, _, sb, alpha = pins.dyadic_case(M, R, C, seed=50 + M)
    xd, wd, sd, ad = bf16_dev(x), bf16_dev(w_base), u8_dev(sb[0]), f32_dev(alpha[0])
    y = bd.linear(xd, wd, sd, ad)
    y64, _ = oracle.linear(x, w_base, sb[0], alpha[0])
    assert np.array_equal(synth.bf16_bits_to_f32(host_bits(y)).astype(np.float64), y64)
    x2 = bf16_dev(synth.activations(M, C, seed=50, index=M))
    assert torch.equal(bd.linear(x2, wd, sd, ad), bd.linear(x2, wd, sd, ad))


@pytest.mark.parametrize("shape", [(256, 2048), (544, 1024)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_identity_prefill_split_k(bd, shape):
    """x = I on split-K shapes: each y element comes from one split, the
    others add zeros, so y = W_eff^T bit for bit."""
    R, C = shape
    assert bd.lib.bitdelta_linear_workspace(C, R, C) > 0
    w_base, so, ao, (wd, sd, ad) = _layer_dev(R, C, seed=12)
    weff = oracle.reconstruct(w_base, so, ao)
    eye = torch.eye(C, dtype=torch.bfloat16, device="cuda")
    y = host_bits(bd.linear(eye, wd, sd, ad))
    assert same_bits_pm0(y, weff.T)


@pytest.mark.parametrize("case", [((1024, 8192), 2048, 4 * 64), ((4096, 4096), 1024, 2 * 128),
                                  ((160, 4096), 700, 8 * 6)], ids=lambda c: f"{c[0][0]}x{c[0][1]}_m{c[1]}")
def test_narrow_tiles_dyadic_exact(bd, case):
    """Few tiles of 256 x 256 with short K ranges: the kernel runs tiles 128
    features wide (twice as many) with half the K ranges (k/v at m = 2048, a
    4096-wide layer at m = 1024, a ragged d_out of 160 whose last narrow tile
    holds 32 rows); the workspace holds one 256 x 128 fp32 partial per narrow
    tile and range.  Exact-arithmetic inputs: both edge features of every
    narrow tile and random ones, bit for bit; repeated calls give the same
    bits."""
    (R, C), M, partials = case
    assert bd.lib.bitdelta_linear_workspace(M, R, C) == partials * 256 * 128 * 4
    x, w_base, _, sb, alpha = pins.dyadic_case(M, R, C, seed=70 + M % 11)
    xd, wd, sd, ad = bf16_dev(x), bf16_dev(w_base), u8_dev(sb[0]), f32_dev(alpha[0])
    y = host_bits(bd.linear(xd, wd, sd, ad))
    edges = np.concatenate([np.arange(0, R, 128), np.minimum(np.arange(127, R + 127, 128), R - 1)])
    rows = np.unique(np.concatenate([edges, synth.u64(16, 0, 9200 + R) % np.uint64(R)]).astype(np.int64))
    y64, _ = oracle.linear(x, w_base, sb[0], alpha[0], rows=rows)
    assert np.array_equal(synth.bf16_bits_to_f32(y[:, rows]).astype(np.float64), y64)
    x2 = bf16_dev(synth.activations(M, C, seed=71, index=M))
    assert torch.equal(bd.linear(x2, wd, sd, ad), bd.linear(x2, wd, sd, ad))


@pytest.mark.parametrize("case", [((4128, 4096), 4000), ((4352, 8192), 4096), ((4096, 4096), 4608)],
                         ids=lambda c: f"{c[0][0]}x{c[0][1]}_m{c[1]}")
def test_last_wave_split_dyadic_exact(bd, case):
    """More tiles than CUs with a last partial wave (16, 17 or 32 tiles of 272
    or 288): that wave runs as a second launch with K cut in ranges (the last
    case has d_out < m, so its tiles are numbered feature tiles fastest and the
    split wave is the last two token tiles).  Exact-arithmetic inputs: sampled
    output features, every one of the last tile column, bit for bit; repeated
    calls give the same bits."""
    (R, C), M = case
    tile = 256 * 256 * 4
    assert bd.lib.bitdelta_linear_workspace(M, R, C) >= 2 * 16 * tile
    x, w_base, _, sb, alpha = pins.dyadic_case(M, R, C, seed=60 + M % 7)
    xd, wd, sd, ad = bf16_dev(x), bf16_dev(w_base), u8_dev(sb[0]), f32_dev(alpha[0])
    y = host_bits(bd.linear(xd, wd, sd, ad))
    rows = np.unique(np.concatenate([np.arange(4096, R), [0, 255, 256, 2047, 4095],
                                     synth.u64(16, 0, 9100 + R) % np.uint64(R)]).astype(np.int64))
    y64, _ = oracle.linear(x, w_base, sb[0], alpha[0], rows=rows)
    assert np.array_equal(synth.bf16_bits_to_f32(y[:, rows]).astype(np.float64), y64)
    x2 = bf16_dev(synth.activations(M, C, seed=61, index=M))
    assert torch.equal(bd.linear(x2, wd, sd, ad), bd.linear(x2, wd, sd, ad))


def test_identity_last_wave_split(bd):
    """x = I on 4128 x 4096 (272 tiles, the last 16 split in K): each y element
    comes from one K range, the other adds zeros, so y = W_eff^T bit for bit."""
    R, C = 4128, 4096
    assert bd.lib.bitdelta_linear_workspace(C, R, C) > 0
    w_base, so, ao, (wd, sd, ad) = _layer_dev(R, C, seed=13)
    weff = oracle.reconstruct(w_base, so, ao)
    eye = torch.eye(C, dtype=torch.bfloat16, device="cuda")
    y = host_bits(bd.linear(eye, wd, sd, ad))
    assert same_bits_pm0(y, weff.T)


def test_zero_tokens_and_misaligned(bd):
    R, C = 64, 128
    w_base, so, ao, (wd, sd, ad) = _layer_dev(R, C, seed=8)
    y = bd.linear(torch.empty((0, C), dtype=torch.bfloat16, device="cuda"), wd, sd, ad)
    assert y.shape == (0, R)
    big = bf16_dev(synth.activations(5, C + 1, seed=8))
    x_bad = big.view(-1)[1:1 + 4 * C].view(4, C)   # 2-byte offset: not 16-byte aligned
    with pytest.raises(bd.BitDeltaError) as e:
        bd.linear(x_bad, wd, sd, ad)
    assert e.value.status == bd.BD_EALIGN


# -------------------------------------------- prefill on the 70B layer shapes


SHAPES_70B = [(8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672)]
SAMPLED_ROWS = 512   # output features checked per matrix at full size


def _sample_rows(R, fixed, tag):
    """Sorted output features to check: the fixed ones (first, last, tile
    edges) and seeded random ones, SAMPLED_ROWS in all (every row if R is
    smaller)."""
    if R <= SAMPLED_ROWS:
        return np.arange(R, dtype=np.int64)
    chosen = set(int(r) for r in fixed if 0 <= r < R)
    extra = synth.u64(4 * SAMPLED_ROWS, 0, tag) % np.uint64(R)
    for r in extra:
        if len(chosen) >= SAMPLED_ROWS:
            break
        chosen.add(int(r))
    return np.array(sorted(chosen), dtype=np.int64)


@pytest.mark.parametrize("shape", SHAPES_70B, ids=lambda s: f"{s[0]}x{s[1]}")
def test_prefill_70b_shapes(bd, shape):
    """M = 2048 tokens: full bit-exact compress, linear checked on sampled
    output features (first, last, tile edges, random) for every token."""
    R, C = shape
    M = 2048
    w_base, w_ft = synth.layer(R, C, seed=0, index=100 + R % 57)
    so, ao = oracle.compress(w_base, w_ft)
    wd = bf16_dev(w_base)
    sg, ag = bd.compress(wd, f32_dev(w_ft))
    assert np.array_equal(host(sg), so)
    assert np.array_equal(_bits32(host(ag)), _bits32(ao))
    del w_ft
    x = synth.activations(M, C, seed=0, index=100 + R % 57)
    y = host_bits(bd.linear(bf16_dev(x), wd, sg, ag))
    rows = _sample_rows(R, [0, 1, 255, 256, R - 1, *range(0, R, R // 8)], 9000 + R)
    y64, sc = oracle.linear(x, w_base, so, ao, rows=rows)
    check_linear(y[:, rows], y64, sc, f"prefill {R}x{C}")


def test_identity_prefill_8192(bd):
    """x = I on an 8192 x 8192 layer: y = W_eff^T over the whole matrix."""
    R = C = 8192
    w_base, so, ao, (wd, sd, ad) = _layer_dev(R, C, seed=9)
    weff = oracle.reconstruct(w_base, so, ao)
    eye = torch.eye(C, dtype=torch.bfloat16, device="cuda")
    y = host_bits(bd.linear(eye, wd, sd, ad))
    assert same_bits_pm0(y, weff.T)


# ------------------------------------------------- decode on long rows, full size

# Decode plans that only long rows reach: x of m = 4 tokens up to 64 KB in LDS (8192 wide); m = 3..4
# with a larger x on the whole-row MFMA kernel; at least 8192 rows of a width above 4096 on its two-row
# plan (32-row workgroups, two tile buffers), whose last workgroup holds only 16 rows at 8208.
LONG_DECODE = [((8208, 8192), 16, False), ((8208, 8192), 5, True), ((8192, 12288), 3, False),
               ((8208, 8192), 4, True), ((8192, 12288), 4, False)]


@pytest.mark.parametrize("case", LONG_DECODE, ids=lambda c: f"{c[0][0]}x{c[0][1]}_m{c[1]}_{'matrix' if c[2] else 'row'}")
def test_linear_decode_long_rows(bd, case):
    (R, C), M, per_matrix = case
    w_base, so, ao, (wd, sd, ad) = _layer_dev(R, C, seed=5, index=M, per_matrix=per_matrix)
    x = synth.activations(M, C, seed=5, index=M)
    y = host_bits(bd.linear(bf16_dev(x), wd, sd, ad, per_matrix=per_matrix))
    rows = _sample_rows(R, [0, 1, 15, 16, 31, 32, 33, 8191, 8192, R - 1, *range(0, R, R // 8)], 7000 + R + M)
    y64, sc = oracle.linear(x, w_base, so, ao, per_matrix=per_matrix, rows=rows)
    check_linear(y[:, rows], y64, sc, f"decode {R}x{C} m={M}")


@pytest.mark.parametrize("R,C,M", [(1024, 8192, 16), (1000, 28672, 5)], ids=lambda v: str(v))
def test_dyadic_exact_split_rows(bd, R, C, M):
    """Exact-arithmetic inputs with the row's steps in parts (few rows, long
    width): every output bit for bit."""
    x, w_base, _, sb, alpha = pins.dyadic_case(M, R, C, seed=91)
    y = host_bits(bd.linear(bf16_dev(x), bf16_dev(w_base), u8_dev(sb[0]), f32_dev(alpha[0])))
    y64, _ = oracle.linear(x, w_base, sb[0], alpha[0])
    assert np.array_equal(synth.bf16_bits_to_f32(y).astype(np.float64), y64)


def test_dyadic_exact_two_row_plan(bd):
    """Exact-arithmetic inputs through the two-row plan, bit for bit on the
    sampled rows (the partial last workgroup included)."""
    R, C, M = 8208, 8192, 16
    x, w_base, _, sb, alpha = pins.dyadic_case(M, R, C, seed=77)
    y = host_bits(bd.linear(bf16_dev(x), bf16_dev(w_base), u8_dev(sb[0]), f32_dev(alpha[0])))
    rows = _sample_rows(R, [0, 15, 16, 31, 32, 8191, 8192, 8207], 7777)
    y64, _ = oracle.linear(x, w_base, sb[0], alpha[0], rows=rows)
    assert np.array_equal(synth.bf16_bits_to_f32(y[:, rows]).astype(np.float64), y64)


@pytest.mark.parametrize("M,C", [(16, 8192), (4, 12288)], ids=lambda v: str(v))
def test_identity_decode_two_row_plan(bd, M, C):
    """One-hot x through the two-row plan: y[t, r] = W_eff[r, j_t] bit for bit on every row."""
    R = 8208
    w_base, so, ao, (wd, sd, ad) = _layer_dev(R, C, seed=8)
    weff = oracle.reconstruct(w_base, so, ao)
    cols = np.linspace(0, C - 1, M).astype(int)
    x = np.zeros((M, C), dtype=np.float32)
    x[np.arange(M), cols] = 1.0
    y = host_bits(bd.linear(bf16_dev(synth.to_bf16_bits(x)), wd, sd, ad))
    assert same_bits_pm0(y, weff[:, cols].T)


# ------------------------------------------------------------------- grouped


def _variants(R, C, V, seed, per_matrix=False):
    w_base = synth.to_bf16_bits(synth.normal_f32((R, C), 0.02, seed, synth.tag(synth.TAG_WBASE)))
    bv = synth.variant_scales(V, seed=seed)
    signs = np.zeros((V, R, C // 8), dtype=np.uint8)
    alpha = np.zeros((V, 1 if per_matrix else R), dtype=np.float32)
    for v in range(V):
        signs[v], alpha[v] = oracle.compress(w_base, synth.variant_ft(w_base, v, float(bv[v]), seed=seed),
                                             per_matrix=per_matrix)
    if per_matrix:
        alpha = alpha[:, 0].copy()
    return w_base, signs, alpha


@pytest.mark.parametrize("per_matrix", [False, True], ids=["alpha_row", "alpha_matrix"])
def test_grouped_small(bd, per_matrix):
    R, C, V, M = 300, 200, 3, 600
    w_base, signs, alpha = _variants(R, C, V, seed=11, per_matrix=per_matrix)
    x = synth.activations(M, C, seed=11)
    ids = (synth.u64(M, 11, 500) % np.uint64(V)).astype(np.int32)
    ids[[5, 77, 300]] = [-1, V, 1000]   # out of range: zero rows
    y = host_bits(bd.linear_grouped(bf16_dev(x), i32_dev(ids), bf16_dev(w_base), u8_dev(signs), f32_dev(alpha),
                                    per_matrix=per_matrix))
    y64, sc = oracle.linear_grouped(x, ids, w_base, signs, alpha, per_matrix=per_matrix)
    check_linear(y, y64, sc, "grouped small")
    assert np.all(y[[5, 77, 300]] == 0)


def test_grouped_equals_linear_per_variant(bd):
    R, C, V, M = 256, 512, 4, 300
    w_base, signs, alpha = _variants(R, C, V, seed=12)
    x = bf16_dev(synth.activations(M, C, seed=12))
    wd, sd, ad = bf16_dev(w_base), u8_dev(signs), f32_dev(alpha)
    for v in range(V):
        ids = torch.full((M,), v, dtype=torch.int32, device="cuda")
        yg = bd.linear_grouped(x, ids, wd, sd, ad)
        yl = bd.linear(x, wd, sd[v].contiguous(), ad[v].contiguous())
        assert torch.equal(yg, yl), v


def test_grouped_dyadic_exact(bd):
    R, C, V, M = 96, 128, 14, 400
    x, w_base, _, sb, alpha = pins.dyadic_case(M, R, C, seed=13, n_variants=V)
    ids = (synth.u64(M, 13, 501) % np.uint64(V)).astype(np.int32)
    y = host_bits(bd.linear_grouped(bf16_dev(x), i32_dev(ids), bf16_dev(w_base), u8_dev(sb), f32_dev(alpha)))
    y64, _ = oracle.linear_grouped(x, ids, w_base, sb, alpha)
    assert np.array_equal(synth.bf16_bits_to_f32(y).astype(np.float64), y64)


def test_grouped_edge_sizes(bd):
    R, C, V = 64, 64, 2
    w_base, signs, alpha = _variants(R, C, V, seed=14)
    wd, sd, ad = bf16_dev(w_base), u8_dev(signs), f32_dev(alpha)
    y0 = bd.linear_grouped(torch.empty((0, C), dtype=torch.bfloat16, device="cuda"),
                           torch.empty((0,), dtype=torch.int32, device="cuda"), wd, sd, ad)
    assert y0.shape == (0, R)
    x = synth.activations(1, C, seed=14)
    ids = np.array([1], dtype=np.int32)
    y = host_bits(bd.linear_grouped(bf16_dev(x), i32_dev(ids), wd, sd, ad))
    y64, sc = oracle.linear_grouped(x, ids, w_base, signs, alpha)
    check_linear(y, y64, sc, "grouped m=1")


def test_grouped_zipf_14_variants(bd):
    """One 8192 x 8192 base, 14 variants, 4096 tokens in a Zipf(1.1) split:
    per-variant compress bit-exact, sampled output features for every token."""
    R = C = 8192
    V, M = 14, 4096
    w_base = synth.to_bf16_bits(synth.normal_f32((R, C), 0.02, 0, synth.tag(synth.TAG_WBASE, 200)))
    wd = bf16_dev(w_base)
    bv = synth.variant_scales(V, seed=0)
    rows = _sample_rows(R, [0, 255, 256, R - 1], 9100)
    signs = torch.empty((V, R, C // 8), dtype=torch.uint8, device="cuda")
    alpha = torch.empty((V, R), dtype=torch.float32, device="cuda")
    # The oracle sees only its own compress output, on the sampled rows (the
    # rows it is asked about); the other rows stay zero and are never read.
    so_rows = np.zeros((V, R, C // 8), dtype=np.uint8)
    ao_all = np.zeros((V, R), dtype=np.float32)
    for v in range(V):
        w_ft = synth.variant_ft(w_base, v, float(bv[v]), seed=0, index=200)
        sg, ag = bd.compress(wd, f32_dev(w_ft))
        signs[v], alpha[v] = sg, ag
        so, ao = oracle.compress(w_base[rows], w_ft[rows])
        assert np.array_equal(host(sg)[rows], so) and np.array_equal(_bits32(host(ag)[rows]), _bits32(ao))
        so_rows[v][rows], ao_all[v][rows] = so, ao
    counts = synth.zipf_counts(M, V, 1.1)
    ids = synth.variant_ids(counts, seed=0)
    x = synth.activations(M, C, seed=0, index=200)
    y = host_bits(bd.linear_grouped(bf16_dev(x), i32_dev(ids), wd, signs, alpha))
    y64, sc = oracle.linear_grouped(x, ids, w_base, so_rows, ao_all, rows=rows)
    check_linear(y[:, rows], y64, sc, "grouped zipf")


# ----------------------------------------------------------- 70B-shaped stack


def test_stack_two_layers(bd):
    """The stack driver with two layers of every 70B shape and 14 delta sets:
    variant 0 compressed from streamed fine-tuned weights (bit-exact on
    sampled rows), the others random packed signs; prefill (m = 512) and decode
    (m = 1) passes checked on sampled output features of every matrix."""
    from tenant_fine_tune_amd.stack import LinearStack

    st = LinearStack(n_layers=2, n_variants=14)
    st.reserve(512)
    dev = st.device
    bv = synth.variant_scales(14, seed=3)
    rows_of = {}
    orc_rows = {}  # (l, name) -> (w_base rows, so rows, ao rows) from the oracle's own compress
    for l, name, d_out, d_in in st.matrices():
        idx = 1000 + 10 * l + [s[0] for s in st.shapes].index(name)
        wb = synth.device_normal((d_out, d_in), 0.02, 3, synth.tag(synth.TAG_WBASE, idx), dev, torch.bfloat16)
        st.base[l, name].copy_(wb)
        w_ft = wb.float().add_(synth.device_laplace((d_out, d_in), float(bv[0]), 3, synth.tag(synth.TAG_DELTA, idx), dev))
        st.compress_into(0, l, name, w_ft)
        rows = np.unique(np.concatenate([[0, 255, d_out - 1], synth.u64(5, 3, 9300 + idx) % np.uint64(d_out)]))
        rows_of[l, name] = rows.astype(np.int64)
        r_t = torch.from_numpy(rows.astype(np.int64)).to(dev)
        wb_rows = host_bits(wb.index_select(0, r_t))
        ft_rows = host(w_ft.index_select(0, r_t))
        so, ao = oracle.compress(wb_rows, ft_rows)
        assert np.array_equal(host(st.signs[0, l, name].index_select(0, r_t)), so)
        assert np.array_equal(_bits32(host(st.alpha[0, l, name].index_select(0, r_t))), _bits32(ao))
        orc_rows[l, name] = (wb_rows, so, ao)
        for v in range(1, 14):
            g = torch.Generator(device=dev)
            g.manual_seed(77 + 1000 * v + idx)
            st.signs[v, l, name].copy_(torch.randint(0, 256, st.signs[v, l, name].shape, generator=g, device=dev,
                                                     dtype=torch.int32).to(torch.uint8))
            st.alpha[v, l, name].copy_(torch.rand(st.alpha[v, l, name].shape, generator=g, device=dev) * 2e-3)
        del w_ft, wb
    widths = {name: d_in for name, _, d_in in st.shapes}
    outs = {name: d_out for name, d_out, _ in st.shapes}
    for m in (512, 1):
        xs_h = {name: synth.activations(m, widths[name], seed=3, index=m + i) for i, name in enumerate(widths)}
        xs = {name: bf16_dev(a) for name, a in xs_h.items()}
        ys = {name: torch.empty((m, outs[name]), dtype=torch.bfloat16, device=dev) for name in outs}
        st.forward(0, xs, ys)  # ys now hold layer 1
        for name in outs:
            wb_rows, so, ao = orc_rows[1, name]
            y64, sc = oracle.linear(xs_h[name], wb_rows, so, ao)
            check_linear(host_bits(ys[name])[:, rows_of[1, name]], y64, sc, f"stack layer 1 {name} m={m}")
        for name in outs:  # layer 0, and a random variant on layer 0
            st.linear(0, 0, name, xs[name], ys[name])
            wb_rows, so, ao = orc_rows[0, name]
            y64, sc = oracle.linear(xs_h[name], wb_rows, so, ao)
            check_linear(host_bits(ys[name])[:, rows_of[0, name]], y64, sc, f"stack layer 0 {name} m={m}")
            r_t = torch.from_numpy(rows_of[0, name]).to(dev)
            st.linear(9, 0, name, xs[name], ys[name])
            s9 = host(st.signs[9, 0, name].index_select(0, r_t))
            a9 = host(st.alpha[9, 0, name].index_select(0, r_t))
            y64, sc = oracle.linear(xs_h[name], wb_rows, s9, a9)
            check_linear(host_bits(ys[name])[:, rows_of[0, name]], y64, sc, f"stack variant 9 {name} m={m}")
    assert st.resident_bytes() == st.params() * 2 + 14 * (st.params() // 8 + 4 * 2 * sum(o for _, o, _ in st.shapes))


def test_stack_full_80_layers(bd):
    """The whole 70B-shaped stack resident on the GPU (80 layers x 7 linears,
    14 packed delta sets, 257 GB, as the post's memory arithmetic has it):
    variant 0 compressed matrix by matrix from streamed fine-tuned weights,
    the other 13 random packed codes.  Compress is bit-exact on sampled rows of
    layers 0 and 79; the fused linear at m = 512 (prefill) and m = 1, 4, 16
    (decode: the stream, x-in-LDS and two-row plans on these shapes) matches
    the oracle on sampled output features of every matrix of layers 0 and 79,
    for variant 0 and for variant 9; a full pass through all 560 linears runs
    and gives finite outputs."""
    from tenant_fine_tune_amd.stack import LinearStack

    torch.cuda.empty_cache()
    free, total = torch.cuda.mem_get_info()
    if free < 270e9:
        pytest.skip(f"needs about 260 GB of free device memory ({free / 1e9:.0f} GB free of {total / 1e9:.0f})")
    print("stack 80 layers: allocating", flush=True)
    st = LinearStack(n_layers=80, n_variants=14)
    st.reserve(512)
    dev = st.device
    names = [s[0] for s in st.shapes]
    bv = synth.variant_scales(14, seed=5)
    checked = (0, 79)
    rows_of, orc_rows = {}, {}
    for l, name, d_out, d_in in st.matrices():
        idx = 2000 + 10 * l + names.index(name)
        st.base[l, name].copy_(synth.device_normal((d_out, d_in), 0.02, 5, synth.tag(synth.TAG_WBASE, idx), dev,
                                                   torch.bfloat16))
        w_ft = st.base[l, name].float().add_(synth.device_laplace((d_out, d_in), float(bv[0]), 5,
                                                                  synth.tag(synth.TAG_DELTA, idx), dev))
        st.compress_into(0, l, name, w_ft)
        if l in checked:
            rows = np.unique(np.concatenate([[0, d_out - 1], synth.u64(6, 5, 9400 + idx) % np.uint64(d_out)]))
            rows_of[l, name] = rows.astype(np.int64)
            r_t = torch.from_numpy(rows_of[l, name]).to(dev)
            wb_rows = host_bits(st.base[l, name].index_select(0, r_t))
            so, ao = oracle.compress(wb_rows, host(w_ft.index_select(0, r_t)))
            assert np.array_equal(host(st.signs[0, l, name].index_select(0, r_t)), so), (l, name)
            assert np.array_equal(_bits32(host(st.alpha[0, l, name].index_select(0, r_t))), _bits32(ao)), (l, name)
            orc_rows[l, name] = (wb_rows, so, ao)
        del w_ft
        g = torch.Generator(device=dev)
        g.manual_seed(idx)
        for v in range(1, 14):
            st.signs[v, l, name].copy_(torch.randint(0, 256, st.signs[v, l, name].shape, generator=g, device=dev,
                                                     dtype=torch.int32).to(torch.uint8))
            st.alpha[v, l, name].copy_(torch.rand(st.alpha[v, l, name].shape, generator=g, device=dev)
                                       .mul_(float(bv[v])).add_(float(bv[v]) * 0.5))
        if name == names[-1] and l % 20 == 19:
            torch.cuda.synchronize()
            print(f"stack 80 layers: layer {l + 1} filled and compressed", flush=True)
    widths = {name: d_in for name, _, d_in in st.shapes}
    outs = {name: d_out for name, d_out, _ in st.shapes}
    for m in (512, 1, 4, 16):
        xs_h = {name: synth.activations(m, widths[name], seed=5, index=m + i) for i, name in enumerate(widths)}
        xs = {name: bf16_dev(a) for name, a in xs_h.items()}
        ys = {name: torch.empty((m, outs[name]), dtype=torch.bfloat16, device=dev) for name in outs}
        st.forward(0, xs, ys)
        torch.cuda.synchronize()
        assert all(torch.isfinite(ys[n].float()).all() for n in outs)
        for l in checked:
            for v in (0, 9):
                for name in outs:
                    st.linear(v, l, name, xs[name], ys[name])
                    wb_rows, so, ao = orc_rows[l, name]
                    if v != 0:
                        r_t = torch.from_numpy(rows_of[l, name]).to(dev)
                        so = host(st.signs[v, l, name].index_select(0, r_t))
                        ao = host(st.alpha[v, l, name].index_select(0, r_t))
                    y64, sc = oracle.linear(xs_h[name], wb_rows, so, ao)
                    check_linear(host_bits(ys[name])[:, rows_of[l, name]], y64, sc,
                                 f"stack 80 layers: layer {l} {name} variant {v} m={m}")
        print(f"stack 80 layers: m={m} checked on layers {checked}, variants 0 and 9", flush=True)
    # 136.9 GB of bf16 base + 14 x (8,556,380,160 sign bytes + 26,869,760 alpha bytes), the storage the pins
    # derive from the post's arithmetic
    assert st.resident_bytes() == 136_902_082_560 + 14 * (8_556_380_160 + 26_869_760) == 257_067_581_440
    del st, xs, ys
    torch.cuda.empty_cache()
