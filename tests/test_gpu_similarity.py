"""GPU tier: K-Merge similarity of BitDelta task vectors against the oracle,
through the C ABI.  The Gram matrix must match bit for bit (its summation
order is fixed); the cosines, one fp64 multiply, square root and divide on
top of it, to within 1 ulp.  Inputs are seeded packed signs: independent
ones, and correlated ones (each variant flips a shared pattern with its own
probability) so that the cosines span (0, 1]."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import f32_dev, host, u8_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tenant_fine_tune_amd as bd

    return bd


def _signs(V, R, C, seed, correlated):
    G = C // 8
    if not correlated:
        return synth.u64((V, R, G), seed, 7201).astype(np.uint8)
    base = np.unpackbits(synth.u64((R, G), seed, 7202).astype(np.uint8), axis=-1, bitorder="little")
    out = np.empty((V, R, G), dtype=np.uint8)
    for v in range(V):
        u = (synth.u64((R, C), seed, 7210 + v) >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
        flip = (u < 0.04 * v).astype(np.uint8)
        out[v] = np.packbits(base ^ flip, axis=-1, bitorder="little")
    return out


def _alpha(V, R, seed, per_matrix):
    a = np.abs(synth.normal_f32((V, R), 1e-3, seed, 7203)).astype(np.float32) + np.float32(1e-5)
    return a[:, 0].copy() if per_matrix else a


def _check(bd, sb, alpha, per_matrix, what):
    g, c = bd.similarity(u8_dev(sb), f32_dev(alpha), per_matrix=per_matrix)
    g, c = host(g), host(c)
    g64, c64 = oracle.similarity(sb, alpha, per_matrix=per_matrix)
    assert np.array_equal(g, g64), (what, np.abs(g - g64).max())
    assert np.all(np.abs(c - c64) <= np.spacing(np.abs(c64))), (what, np.abs(c - c64).max())
    return g, c


SIM_CASES = [(1, 5, 64), (2, 17, 32), (3, 300, 1024), (14, 300, 1024), (16, 40, 224), (5, 1000, 8192),
             (14, 64, 28672), (7, 257, 96)]


@pytest.mark.parametrize("per_matrix", [False, True], ids=["alpha_row", "alpha_matrix"])
@pytest.mark.parametrize("case", SIM_CASES, ids=lambda c: f"v{c[0]}_{c[1]}x{c[2]}")
def test_similarity_matches_oracle(bd, case, per_matrix):
    V, R, C = case
    for correlated in (False, True):
        sb = _signs(V, R, C, seed=V + R, correlated=correlated)
        alpha = _alpha(V, R, seed=V + C, per_matrix=per_matrix)
        _check(bd, sb, alpha, per_matrix, f"{case} correlated={correlated}")


def test_similarity_known_patterns(bd):
    """Identical variants: cosine 1; complementary sign patterns with the same
    alpha: gram = -gram_aa and cosine -1; repeated calls give the same bits."""
    V, R, C = 4, 130, 512
    sb = _signs(V, R, C, seed=3, correlated=False)
    sb[1] = sb[0]
    sb[2] = ~sb[0]
    alpha = _alpha(V, R, seed=3, per_matrix=False)
    alpha[1] = alpha[0]
    alpha[2] = alpha[0]
    g, c = _check(bd, sb, alpha, False, "patterns")
    assert c[0, 1] == 1.0 and g[0, 1] == g[0, 0]
    assert g[0, 2] == -g[0, 0] and c[0, 2] == -1.0
    g2, c2 = bd.similarity(u8_dev(sb), f32_dev(alpha))
    assert np.array_equal(host(g2), g) and np.array_equal(host(c2), c)


def test_similarity_14_variants_8192(bd):
    """The multi-tenant layer's size: 14 variants of an 8192 x 8192 matrix,
    correlated signs, the whole Gram matrix bit for bit."""
    V, R, C = 14, 8192, 8192
    sb = _signs(V, R, C, seed=14, correlated=True)
    alpha = _alpha(V, R, seed=14, per_matrix=False)
    g, c = _check(bd, sb, alpha, False, "14 x 8192^2")
    # the flip probabilities 0.04 v set the sign correlation (1 - 0.08 a)(1 - 0.08 b);
    # the independent per-row alphas scale it by sum(a_a a_b) / sqrt(sum a_a^2 sum a_b^2)
    a64 = alpha.astype(np.float64)
    f = (a64 @ a64.T) / np.sqrt(np.outer((a64 ** 2).sum(1), (a64 ** 2).sum(1)))
    exp = f * np.outer(1 - 0.08 * np.arange(V), 1 - 0.08 * np.arange(V))
    np.fill_diagonal(exp, 1.0)
    assert np.allclose(c, exp, atol=5e-3)
