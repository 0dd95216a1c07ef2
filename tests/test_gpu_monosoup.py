"""GPU tier: MonoSoup merge (section "MonoSoup" of "BitDelta: Serving 14 Zen
Models from One GPU Cluster") through the C ABI, against the oracle's exact
truncated SVD.

The GPU path finds each task vector's rank-r truncation with a 64-column
randomized range finder; the oracle takes the exact one (one-sided Jacobi).
Tolerances:
  - the merge is compared as rel = ||(M_gpu - W_base) - (M_ref - W_base)||_F /
    ||M_ref - W_base||_F and as the largest element error over the largest
    |M_ref - W_base|;
  - with power_iters >= 1 on task vectors whose spectrum drops by a factor of
    about 50 after the r-th singular value (the synthetic recipe: rank-r
    signal, entry RMS 1e-3, plus N(0, 1e-5^2) noise), the range finder's own
    error is below 2e-7 (fp64 emulation), so what is left is fp32 arithmetic:
    the passes accumulate up to a few hundred fp32 products per output
    (relative error about sqrt(n) 2^-24 < 1e-6) and the result is rounded to
    fp32.  Bar: rel <= 2e-5, element <= 5e-5;
  - with power_iters = 0 the range finder's error (Halko, Martinsson and Tropp
    2011, the oversampled Gaussian bound) dominates: 3e-3 on these inputs in
    fp64 emulation.  Bar: rel <= 2e-2;
  - task vectors of rank <= 64 are captured exactly by the sketch, so their
    truncation matches to the fp32 bar even without power iterations when
    the sketch is oversampled (r < 64; see the r = 64 case below);
  - zero task vectors and rank 0 give f32(W_base) bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import bf16_dev, f32_dev, host

pytestmark = pytest.mark.gpu

TIGHT_REL, TIGHT_ELEM, LOOSE_REL = 2e-5, 5e-5, 2e-2


@pytest.fixture(scope="module")
def bd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tenant_fine_tune_amd as bd

    return bd


def _run(bd, wb, wf, om, rank, q):
    out, sig = bd.monosoup(bf16_dev(wb), f32_dev(wf), f32_dev(om), rank, power_iters=q)
    torch.cuda.synchronize()
    return host(out).astype(np.float64), (host(sig) if sig is not None else None)


def _errors(got, ref, base):
    d_ref = ref - base
    rel = np.linalg.norm((got - base) - d_ref) / max(np.linalg.norm(d_ref), 1e-300)
    elem = np.abs(got - ref).max() / max(np.abs(d_ref).max(), 1e-300)
    return rel, elem


_CASES = {
    # name: (R, C, k, signal rank, merge rank, noise)
    "ragged_tall": (200, 332, 3, 8, 8, 1e-5),
    "ragged_small": (130, 68, 2, 6, 6, 1e-5),
    "wide": (70, 260, 1, 10, 10, 1e-5),
    "rank_40_of_64": (300, 256, 2, 64, 40, 0.0),
    "many_checkpoints": (96, 72, 64, 8, 8, 1e-5),   # the largest k the entry point takes
}
_ORACLE = {}


def _case(name):
    if name not in _ORACLE:
        R, C, k, rho, r, noise = _CASES[name]
        wb, wf = synth.checkpoints(R, C, k, rho, noise, seed=71)
        om = synth.omega(C, seed=71)
        ref, sig = oracle.monosoup(wb, wf, r)
        _ORACLE[name] = (wb, wf, om, r, ref, sig)
    return _ORACLE[name]


@pytest.mark.parametrize("name", sorted(_CASES))
@pytest.mark.parametrize("q", [0, 1, 2])
def test_monosoup_vs_oracle(bd, name, q):
    wb, wf, om, r, ref, sig = _case(name)
    base = synth.bf16_bits_to_f32(wb).astype(np.float64)
    got, gsig = _run(bd, wb, wf, om, r, q)
    rel, elem = _errors(got, ref, base)
    exact_range = _CASES[name][3] <= 64 and _CASES[name][5] == 0.0
    if q >= 1 or exact_range:
        assert rel <= TIGHT_REL and elem <= TIGHT_ELEM, (name, q, rel, elem)
        assert np.allclose(gsig, sig[:, :r], rtol=1e-5, atol=0), (name, q)
    else:
        assert rel <= LOOSE_REL, (name, q, rel)
    assert np.all(np.diff(gsig, axis=1) <= 0)


def test_monosoup_exact_low_rank_is_the_mean(bd):
    """Task vectors of rank 5 (no noise) kept at rank 8: every tau_i is Delta_i,
    so the merge is the mean of the checkpoints; the sketch's Gram matrix is
    singular (rank 5 of 64), which the solver must drop, not invert."""
    R, C, k = 1000, 700, 2
    wb, wf = synth.checkpoints(R, C, k, 5, 0.0, seed=72)
    om = synth.omega(C, seed=72)
    base = synth.bf16_bits_to_f32(wb).astype(np.float64)
    delta = wf.astype(np.float64) - base[None]
    # the task vector is the fp32 difference; it equals W_i - W_base exactly here
    # up to the fp32 rounding of W_i, far below the bar
    ref = base + delta.mean(axis=0)
    for q in (0, 1):
        got, _ = _run(bd, wb, wf, om, 8, q)
        rel, elem = _errors(got, ref, base)
        assert rel <= TIGHT_REL and elem <= TIGHT_ELEM, (q, rel, elem)


def test_monosoup_degenerate_cases(bd):
    """Rank 0 and zero task vectors give f32(W_base) bit for bit; rank r = 64
    (the sketch width) on a rank-64 task vector gives it back whole.  With
    r = 64 there is no oversampling: the sketch Delta Omega then carries the
    condition number of a square 64 x 64 Gaussian block (often 1e2 to 1e3) on
    top of Delta's, which fp32 rounding turns into about 1e-4 relative error;
    one power iteration (re-orthonormalised) removes that factor, so this case
    runs with power_iters = 1."""
    R, C = 96, 200
    wb, wf = synth.checkpoints(R, C, 2, 64, 0.0, seed=73)
    om = synth.omega(C, seed=73)
    base = synth.bf16_bits_to_f32(wb)
    got, sig = _run(bd, wb, wf, om, 0, 1)
    assert sig is None and np.array_equal(got.astype(np.float32), base)
    zero = np.stack([base, base])
    got, sig = _run(bd, wb, zero, om, 16, 1)
    assert np.array_equal(got.astype(np.float32), base) and np.all(sig == 0.0)
    got, _ = _run(bd, wb, wf, om, 64, 1)
    ref = base.astype(np.float64) + (wf.astype(np.float64) - base[None]).mean(axis=0)
    rel, elem = _errors(got, ref, base.astype(np.float64))
    assert rel <= TIGHT_REL and elem <= TIGHT_ELEM, (rel, elem)


@pytest.mark.parametrize("R,C", [(1, 260), (300, 4), (5, 8)])
def test_monosoup_full_rank_thin_shapes(bd, R, C):
    """A single row, four columns, a 5 x 8 matrix: at rank min(R, C) every
    task vector is kept whole, so the merge is the mean of the checkpoints
    (the sketch is wider than the matrix's rank: the solver must drop the
    empty directions)."""
    r = min(R, C)
    wb = synth.to_bf16_bits(synth.normal_f32((R, C), 0.02, 75, synth.tag(synth.TAG_WBASE, C)))
    base = synth.bf16_bits_to_f32(wb)
    wf = base[None] + synth.normal_f32((3, R, C), 1e-3, 75, synth.tag(synth.TAG_NOISE, C))
    om = synth.omega(C, seed=75)
    got, _ = _run(bd, wb, wf, om, r, 1)
    ref = base.astype(np.float64) + (wf.astype(np.float64) - base[None]).mean(axis=0)
    rel, elem = _errors(got, ref, base.astype(np.float64))
    assert rel <= TIGHT_REL and elem <= TIGHT_ELEM, (rel, elem)


def test_monosoup_maximum_rows_and_power_iterations(bd):
    """The largest row count the entry point takes (2^21) on four columns,
    rank 4 (the whole task vector), with the largest power_iters (4): the
    merge is the mean of the checkpoints."""
    R, C, r = 1 << 21, 4, 4
    wb = synth.to_bf16_bits(synth.normal_f32((R, C), 0.02, 76, synth.tag(synth.TAG_WBASE, 1)))
    base = synth.bf16_bits_to_f32(wb)
    wf = base[None] + synth.normal_f32((2, R, C), 1e-3, 76, synth.tag(synth.TAG_NOISE, 1))
    om = synth.omega(C, seed=76)
    got, _ = _run(bd, wb, wf, om, r, 4)
    ref = base.astype(np.float64) + (wf.astype(np.float64) - base[None]).mean(axis=0)
    rel, elem = _errors(got, ref, base.astype(np.float64))
    assert rel <= TIGHT_REL and elem <= TIGHT_ELEM, (rel, elem)


def test_monosoup_identical_checkpoints_merge_as_one(bd):
    wb, wf, om, r, _, _ = _case("ragged_tall")
    one, _ = _run(bd, wb, wf[:1], om, r, 1)
    three, _ = _run(bd, wb, np.stack([wf[0]] * 3), om, r, 1)
    base = synth.bf16_bits_to_f32(wb).astype(np.float64)
    rel, _ = _errors(three, one, base)
    assert rel <= 1e-6, rel


def test_monosoup_full_size_property_and_determinism(bd):
    """8192 x 8192, two checkpoints with rank-32 task vectors, merged at rank 32
    with one power iteration (the benchmarked configuration): each truncation
    is the whole task vector, so the merge is the mean of the checkpoints; two
    calls give the same bits."""
    R = C = 8192
    k, r = 2, 32
    print(f"monosoup full size: generating [{k}, {R}, {C}]", flush=True)
    wb, wf = synth.checkpoints(R, C, k, r, 0.0, seed=74)
    om = synth.omega(C, seed=74)
    base = synth.bf16_bits_to_f32(wb).astype(np.float64)
    ref = base + (wf.astype(np.float64) - base[None]).mean(axis=0)
    wb_d, wf_d, om_d = bf16_dev(wb), f32_dev(wf), f32_dev(om)
    print("monosoup full size: running", flush=True)
    out1, _ = bd.monosoup(wb_d, wf_d, om_d, r, power_iters=1)
    out2, _ = bd.monosoup(wb_d, wf_d, om_d, r, power_iters=1)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    rel, elem = _errors(host(out1).astype(np.float64), ref, base)
    assert rel <= TIGHT_REL and elem <= TIGHT_ELEM, (rel, elem)
