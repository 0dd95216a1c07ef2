"""GPU tier: the measurement probes do the work they report.  The read probe
must read every byte (the XOR of its sink words equals the XOR of the
buffer's 32-bit words, including ragged sizes whose last 1 KB run is
partial); the MFMA probe's words equal the closed form 128 * iters * a * b."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tenant_fine_tune_amd as bd

    return bd


@pytest.mark.parametrize("nbytes", [16, 1040, 32 * 1024, 32 * 1024 + 16, 34 * 2 ** 20, 64 * 2 ** 20 + 48])
def test_probe_read_reads_every_word(bd, nbytes):
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes)
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda", generator=g)
    sink = bd.probe_read(buf)
    torch.cuda.synchronize()
    assert sink.numel() == bd.lib.bitdelta_probe_read_sink_words(nbytes)
    want = np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want, (nbytes, hex(got), hex(want))


@pytest.mark.parametrize("blocks,iters,a,b", [(1, 1, 1.0, 1.0), (8, 100, 1.5, -0.5), (300, 7, 0.25, 3.0)])
def test_probe_mfma_closed_form(bd, blocks, iters, a, b):
    sink = bd.probe_mfma(blocks, iters, a, b)
    torch.cuda.synchronize()
    assert sink.numel() == 4 * blocks
    assert torch.all(sink == 128.0 * iters * a * b), sink[:8]
