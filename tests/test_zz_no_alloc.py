"""GPU tier: bitdelta_linear_grouped_noalloc (the grouped linear with the
library's device-resident bucketing table, for callers that cannot allocate)
against bitdelta_linear_grouped (the caller's workspace), through the C ABI.
Outputs must be equal bit for bit on calls in a row whose later calls are
smaller (fewer tokens and variants, another shape), so a table left over from
an earlier call cannot leak into a later one; some ids are out of range (zero
rows)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import bf16_dev, f32_dev, i32_dev, u8_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tenant_fine_tune_amd as bd

    return bd


def _case(m, V, R, C, seed):
    wb = synth.to_bf16_bits(synth.normal_f32((R, C), 0.02, seed, 7601))
    signs = synth.u64((V, R, C // 8), seed, 7602).astype(np.uint8)
    alpha = (np.abs(synth.normal_f32((V, R), 1e-3, seed, 7603)) + np.float32(1e-5)).astype(np.float32)
    ids = (synth.u64(m, seed, 7604) % np.uint64(V + 1)).astype(np.int32)   # id V is out of range: a zero row
    x = synth.activations(m, C, seed=seed, index=7)
    return bf16_dev(x), i32_dev(ids), bf16_dev(wb), u8_dev(signs), f32_dev(alpha)


def _noalloc(bd, x, ids, wb, sg, al, per_matrix):
    m, (R, C), V = x.shape[0], wb.shape, sg.shape[0]
    y = torch.empty((m, R), dtype=torch.bfloat16, device="cuda")
    P = ctypes.c_void_p
    rc = bd.lib.bitdelta_linear_grouped_noalloc(P(x.data_ptr()), m, P(ids.data_ptr()), V, P(wb.data_ptr()),
                                                P(sg.data_ptr()), P(al.data_ptr()), 1 if per_matrix else 0, R, C,
                                                P(y.data_ptr()), P(torch.cuda.current_stream().cuda_stream))
    assert rc == bd.BD_OK, bd.lib.bitdelta_last_error().decode()
    return y


CALLS = [(3000, 9, 768, 1024, False), (700, 3, 512, 512, True), (65, 2, 96, 520, False)]


def test_noalloc_grouped_equals_workspace_grouped(bd):
    for m, V, R, C, per_matrix in CALLS:
        print(f"noalloc grouped: m={m} V={V} {R}x{C} per_matrix={per_matrix}", flush=True)
        x, ids, wb, sg, al = _case(m, V, R, C, seed=m % 13)
        if per_matrix:
            al = al[:, 0].contiguous()
        ref = bd.linear_grouped(x, ids, wb, sg, al, per_matrix=per_matrix)
        got = _noalloc(bd, x, ids, wb, sg, al, per_matrix)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (m, V, R, C)
        zero = (ids.cpu().numpy() == V)
        assert zero.any() and torch.all(got[torch.from_numpy(zero).cuda()] == 0)
