"""CPU tier: the pins catch plausible mistakes in the oracle.

Each case plants one mistake in a private copy of the oracle source (a flipped
sign convention, a reversed bit order, a dropped term, a wrong divisor, index
or stride), compiles it into a temporary library, and requires at least one
pin of tests/pins.py to fail on it.  Mutants only ever run on the CPU; every
planted index stays in bounds.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

from tests import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "bitdelta_oracle.c")

MUTANTS = {
    "msb_first_bits": ("byte |= (uint8_t)(1u << i);", "byte |= (uint8_t)(1u << (7 - i));"),
    "strict_sign": ("if (d >= 0.0f)", "if (d > 0.0f)"),
    "delta_reversed": ("float d = w_ft_at(w_ft, ft_is_f32, idx) - oracle_f32_from_bf16(w_base[idx]);",
                       "float d = oracle_f32_from_bf16(w_base[idx]) - w_ft_at(w_ft, ft_is_f32, idx);"),
    "no_abs": ("(double)fabsf(d);", "(double)d;"),
    "row_divisor": ("alpha[r] = (float)(S[r] / (double)C);", "alpha[r] = (float)(S[r] / (double)(C - 8));"),
    "matrix_divisor": ("alpha[0] = (float)(T / ((double)R * (double)C));", "alpha[0] = (float)(T / (double)C);"),
    "tree_drops_last": ("for (int s = 128; s >= 1; s >>= 1)", "for (int s = 128; s >= 2; s >>= 1)"),
    "sum_in_fp32": ("p[g % 256] = p[g % 256] + (double)fabsf(d);",
                    "p[g % 256] = (double)(float)(p[g % 256] + (double)fabsf(d));"),
    "sign_flipped_scale": ("return bit ? a : -a;", "return bit ? -a : a;"),
    "round_half_up": ("u += 0x7FFFu + lsb;", "u += 0x8000u;"),
    "truncate": ("u += 0x7FFFu + lsb;", "u += 0u * lsb;"),
    "always_first_alpha": ("float a = per_matrix ? alpha[0] : alpha[r];", "float a = alpha[0];"),
    "reversed_k": ("acc += xv * we[j];", "acc += xv * we[C - 1 - j];"),
    "signed_scale": ("sc += fabs(xv) * fabs(we[j]);", "sc += xv * we[j];"),
    "variant_alpha_stride": ("per_matrix ? alpha + v : alpha + (int64_t)v * R;",
                             "per_matrix ? alpha + v : alpha + (int64_t)v;"),
    "variant_ignored": ("const uint8_t *sv = signs + (int64_t)v * R * (C / 8);", "const uint8_t *sv = signs;"),
    "similarity_agreements_only": ("c += sa * sb;", "c += (sa == sb);"),
    "similarity_alpha_twice": ("double term = ((double)fa * (double)fb) * (double)c;",
                               "double term = ((double)fa * (double)fa) * (double)c;"),
    "similarity_no_sqrt": ("double d = sqrt(na * nb);", "double d = na * nb;"),
    "monosoup_no_mean": ("out[i] = (double)oracle_f32_from_bf16(w_base[i]) + acc / (double)k;",
                         "out[i] = (double)oracle_f32_from_bf16(w_base[i]) + acc;"),
    "monosoup_smallest_first": ("while (b > 0 && norm[order[b - 1]] < norm[v])",
                                "while (b > 0 && norm[order[b - 1]] > norm[v])"),
    "monosoup_no_base": ("double d = (double)(wi[i * C + c] - oracle_f32_from_bf16(w_base[i * C + c]));",
                         "double d = (double)wi[i * C + c];"),
    "monosoup_v_transposed": ("s += A[j * m + i] * V[j * n + c];", "s += A[j * m + i] * V[c * n + j];"),
    "monosoup_rotation_sign": ("cp[i] = c * ap - s * aq;", "cp[i] = c * ap + s * aq;"),
    "monosoup_sigma_of_first_column": ("sigma[(int64_t)ck * n + j] = norm[order[j]];",
                                       "sigma[(int64_t)ck * n + j] = norm[order[0]];"),
    "monosoup_first_checkpoint": ("const float *wi = w_ft + (int64_t)ck * R * C;", "const float *wi = w_ft;"),
    "monosoup_rank_minus_one": ("for (int32_t t = 0; t < r; ++t)", "for (int32_t t = 1; t < r; ++t)"),
    "simdelta_base_kept_in_b": ("float db = w_ft_at(w_ft, ft_is_f32, ((int64_t)b * R + r) * C + j) - base;",
                                "float db = w_ft_at(w_ft, ft_is_f32, ((int64_t)b * R + r) * C + j);"),
    "simdelta_row_of_a_twice": ("float db = w_ft_at(w_ft, ft_is_f32, ((int64_t)b * R + r) * C + j) - base;",
                                "float db = w_ft_at(w_ft, ft_is_f32, ((int64_t)a * R + r) * C + j) - base;"),
    "simdelta_fp32_products": ("double prod = (double)da * (double)db;", "double prod = (double)(da * db);"),
    "simdelta_tree_drops_last": ("for (int s = 32; s >= 1; s >>= 1)", "for (int s = 32; s >= 2; s >>= 1)"),
    "simdelta_rows_tree_skipped": ("double total = halving_tree_256(q);", "double total = q[0];"),
    "simdelta_no_sqrt": ("double den = sqrt(norm2);", "double den = norm2;"),
    "similarity_row_of_b": ("const uint8_t *rb = signs + ((int64_t)b * R + r) * G;",
                            "const uint8_t *rb = signs + ((int64_t)a * R + r) * G;"),
}


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(workdir, name):
    import oracle

    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique/found: {old}"
    mpath = os.path.join(workdir, f"{name}.c")
    with open(mpath, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(workdir, f"lib{name}.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-std=c11", "-shared", "-fPIC",
                    mpath, "-o", lib, "-lm"], check=True)
    mutant = oracle.Oracle(lib)
    for pin in pins.ALL:
        try:
            pin(mutant)
        except AssertionError:
            return
    pytest.fail(f"no pin caught mutant {name}")
