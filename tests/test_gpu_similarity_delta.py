"""GPU tier: K-Merge similarity over the full task vectors Delta = W_ft -
W_base against the oracle, through the C ABI.  The Gram matrix must match bit
for bit (its summation order is fixed); the cosines, one fp64 multiply,
square root and divide on top of it, to within 1 ulp.  Inputs: a shared
N(0, 0.02) bf16 base and per-variant Laplace deltas, independent or sharing a
common component (so the cosines span (0, 1)), fp32 or bf16 W_ft; shapes with
ragged 512-column steps, row counts past 256 and 1..16 variants (every tile
count of the kernel)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tenant_fine_tune_amd as bd

    return bd


def _weights(V, R, C, seed, shared):
    wb = synth.to_bf16_bits(synth.normal_f32((R, C), 0.02, seed, 7301))
    base = synth.bf16_bits_to_f32(wb)
    common = synth.laplace_f32((R, C), 1e-3, seed, 7302)
    ft = np.empty((V, R, C), dtype=np.float32)
    for v in range(V):
        own = synth.laplace_f32((R, C), 1e-3 * (1 + 0.3 * v), seed, 7310 + v)
        d = (np.float32(0.25 * (v % 4)) * common + own).astype(np.float32) if shared else own
        ft[v] = (base + d).astype(np.float32)
    return wb, ft


def _check(bd, wb, ft, what):
    if ft.dtype == np.uint16:
        fd = bf16_dev(ft)
    else:
        fd = f32_dev(ft)
    g, c = bd.similarity_delta(bf16_dev(wb), fd)
    g, c = host(g), host(c)
    g64, c64 = oracle.similarity_delta(wb, ft)
    assert np.array_equal(g, g64), (what, np.abs(g - g64).max())
    assert np.all(np.abs(c - c64) <= np.spacing(np.abs(c64))), (what, np.abs(c - c64).max())
    return g, c


CASES = [(1, 5, 64), (2, 17, 8), (3, 300, 1032), (4, 64, 512), (5, 33, 4096), (8, 257, 520), (12, 20, 2056),
         (14, 300, 1024), (16, 40, 224), (14, 128, 8192)]


@pytest.mark.parametrize("ft_bf16", [False, True], ids=["ft_f32", "ft_bf16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"v{c[0]}_{c[1]}x{c[2]}")
def test_similarity_delta_matches_oracle(bd, case, ft_bf16):
    V, R, C = case
    wb, ft = _weights(V, R, C, seed=V + R % 7, shared=True)
    if ft_bf16:
        ft = synth.to_bf16_bits(ft)
    g, c = _check(bd, wb, ft, f"{case} bf16={ft_bf16}")
    assert np.array_equal(g, g.T)
    assert np.all(np.abs(np.diag(c) - 1.0) <= 2.0 ** -52)


def test_similarity_delta_exact_cases(bd):
    """A variant with the negated delta and one with the doubled delta
    (dyadic inputs, exact): cosines -1 and +1, Gram entries -G_00 and 2 G_00;
    an all-zero delta gives a zero row and column."""
    R, C = 40, 1032
    kb = (synth.u64((R, C), 5, 7320) % np.uint64(17)).astype(np.int64) - 8
    base = (kb * 2.0 ** -8).astype(np.float32)
    wb = synth.to_bf16_bits(base)
    d0 = ((synth.u64((R, C), 5, 7321) % np.uint64(17)).astype(np.int64) - 8) * 2.0 ** -10
    ft = np.stack([base + d0, base - d0, base + 2 * d0, base]).astype(np.float32)
    g, c = _check(bd, wb, ft, "exact")
    assert g[0, 1] == -g[0, 0] and c[0, 1] == -1.0
    assert g[0, 2] == 2 * g[0, 0] and g[2, 2] == 4 * g[0, 0] and c[0, 2] == 1.0
    assert np.all(g[3] == 0) and np.all(c[3] == 0)


def test_similarity_delta_deterministic_and_consistent_with_code(bd):
    """Repeated calls give the same bits; a delta of one magnitude per row
    (what the 1-bit code stores exactly) gives the same Gram matrix as the
    similarity of its compressed code."""
    V, R, C = 3, 64, 2048
    kb = (synth.u64((R, C), 6, 7330) % np.uint64(17)).astype(np.int64) - 8
    base = (kb * 2.0 ** -8).astype(np.float32)
    wb = synth.to_bf16_bits(base)
    alpha = ((1 + synth.u64((V, R), 6, 7331) % np.uint64(8)).astype(np.float64) * 2.0 ** -11).astype(np.float32)
    s = 2.0 * (synth.u64((V, R, C), 6, 7332) % np.uint64(2)).astype(np.float64) - 1.0
    ft = (base[None] + alpha[:, :, None] * s).astype(np.float32)
    wbd, fd = bf16_dev(wb), f32_dev(ft)
    g1, c1 = bd.similarity_delta(wbd, fd)
    g2, c2 = bd.similarity_delta(wbd, fd)
    assert torch.equal(g1, g2) and torch.equal(c1, c2)
    signs, alphas = [], []
    for v in range(V):
        sg, ag = bd.compress(wbd, fd[v])
        signs.append(sg)
        alphas.append(ag)
    gc, _ = bd.similarity(torch.stack(signs), torch.stack(alphas))
    assert torch.equal(gc, g1)
