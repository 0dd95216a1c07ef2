"""GPU tier: the measurement probes do the work they report.  The read probe
must read every byte (the XOR of its sink words equals the XOR of the
buffer's 32-bit words, including ragged sizes whose last 1 KB run is
partial); the MFMA probe's words equal the closed form 128 * iters * a * b;
the LDS probe's words equal a host model of every block each wave read,
wrote or copied (include/bitdelta.h gives the access pattern)."""
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


M32 = 0xFFFFFFFF


def _xor(words):
    return int(np.bitwise_xor.reduce(np.asarray(words, dtype=np.uint64) & M32))


def _lds_model(mode, iters, stride, src_words=None):
    """The 16 sink words of one workgroup, from the access pattern alone."""
    fill = (np.arange(16384, dtype=np.uint64) * 0x9E3779B1) & M32
    n = 8 * iters
    out = []
    for w in range(16):
        if mode in (0, 1):
            bw = 256 if mode == 0 else 128          # words per block
            nblk = 16384 // bw
            odd = np.zeros(nblk, dtype=bool)
            for u in range(n):
                odd[(u * stride + w) & (nblk - 1)] ^= True
            out.append(_xor([_xor(fill[b * bw:(b + 1) * bw]) for b in np.nonzero(odd)[0]] or [0]))
        elif mode == 2:
            acc = 0
            for c in range(4):
                u = n - 4 + c
                for l in range(64):
                    acc ^= ((u * 0x9E3779B1 + l) & M32) ^ (((u << 8) ^ l) & M32) ^ ((u + l * 0x01000193) & M32) \
                        ^ (~(u ^ (l << 16)) & M32)
            out.append(acc)
        else:
            nb = src_words.size // 256
            acc = 0
            for c in range(4):
                u = n - 4 + c
                sb = (u * stride + w) & (nb - 1)
                acc ^= _xor(src_words[sb * 256:(sb + 1) * 256])
            out.append(acc)
    return out


@pytest.mark.parametrize("mode,iters,stride", [(0, 3, 17), (0, 8, 1), (1, 5, 33), (2, 2, 17), (2, 7, 3),
                                               (3, 3, 5), (3, 6, 1)])
def test_probe_lds_moves_every_block(bd, mode, iters, stride):
    src = None
    src_words = None
    if mode == 3:
        g = torch.Generator(device="cuda")
        g.manual_seed(iters)
        src = torch.randint(-2 ** 31, 2 ** 31 - 1, (16 * 256,), dtype=torch.int32, device="cuda", generator=g)
        src_words = src.cpu().numpy().view(np.uint32).astype(np.uint64)
    blocks = 3
    sink, cycles = bd.probe_lds(blocks, iters, mode, stride, src)
    torch.cuda.synchronize()
    want = _lds_model(mode, iters, stride, src_words)
    got = sink.cpu().numpy().view(np.uint32).reshape(blocks, 16)
    for b in range(blocks):
        assert [int(v) for v in got[b]] == want, (mode, b)
    assert torch.all(cycles > 0)
