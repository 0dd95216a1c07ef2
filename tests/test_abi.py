"""CPU tier: the C-ABI library loads, exports every declared symbol, and
rejects bad arguments on the host before any launch (no GPU needed).

Only invalid argument sets are passed here: every call below must return
before reaching the HIP runtime.  The one exception (BD_EDEVICE) is run only
where no GPU is visible.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "bitdelta.h")


@pytest.fixture(scope="module")
def bd():
    import tenant_fine_tune_amd as bd

    return bd


def declared_functions():
    inc = os.path.dirname(HDR)
    src = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(bitdelta_\w+)\s*\(", src))


def test_exports_match_header(bd):
    decl = declared_functions()
    assert decl == set(bd.EXPORTS), decl ^ set(bd.EXPORTS)
    handle = ctypes.CDLL(bd.lib_path)
    for name in decl:
        assert hasattr(handle, name), name


def test_version_and_strings(bd):
    assert bd.lib.bitdelta_version() >= 100
    for s in range(7):
        assert bd.lib.bitdelta_status_string(s).decode().startswith("BD_")
    assert b"unknown" in bd.lib.bitdelta_status_string(99)


def test_no_torch_in_header():
    src = open(HDR).read()
    assert "torch" not in src.lower().replace("//", "") or "torch" not in re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    assert "extern \"C\"" in src


FAKE = ctypes.c_void_p(4096)       # aligned, never dereferenced: every call below fails validation
FAKE_ODD = ctypes.c_void_p(4098)   # misaligned


def err(bd):
    return bd.lib.bitdelta_last_error().decode()


def test_compress_validation(bd):
    L = bd.lib
    c = lambda *a: L.bitdelta_compress(*a)  # noqa: E731
    assert c(FAKE, FAKE, 1, 4, 12, 0, FAKE, FAKE, None, 0, None) == bd.BD_ESHAPE  # d_in % 8
    assert "multiple of 8" in err(bd)
    assert c(FAKE, FAKE, 1, 0, 16, 0, FAKE, FAKE, None, 0, None) == bd.BD_ESHAPE   # d_out = 0
    assert c(FAKE, FAKE, 1, 4, -8, 0, FAKE, FAKE, None, 0, None) == bd.BD_ESHAPE   # d_in < 0
    assert c(FAKE, FAKE, 1, 4, 16, 2, FAKE, FAKE, None, 0, None) == bd.BD_EINVAL   # bad mode
    assert c(FAKE, FAKE, 7, 4, 16, 0, FAKE, FAKE, None, 0, None) == bd.BD_EINVAL   # bad dtype
    assert c(None, FAKE, 1, 4, 16, 0, FAKE, FAKE, None, 0, None) == bd.BD_EINVAL   # null
    assert c(FAKE, FAKE, 1, 4, 16, 0, None, FAKE, None, 0, None) == bd.BD_EINVAL
    assert c(FAKE_ODD, FAKE, 1, 4, 16, 0, FAKE, FAKE, None, 0, None) == bd.BD_EALIGN
    assert c(FAKE, FAKE_ODD, 1, 4, 16, 0, FAKE, FAKE, None, 0, None) == bd.BD_EALIGN
    assert c(FAKE, FAKE, 1, 4, 16, 0, FAKE, ctypes.c_void_p(4097), None, 0, None) == bd.BD_EALIGN
    # per-matrix alpha needs 8 * d_out bytes of workspace
    assert L.bitdelta_compress_workspace(4, 16, 1) == 32
    assert L.bitdelta_compress_workspace(4, 16, 0) == 0
    assert c(FAKE, FAKE, 1, 4, 16, 1, FAKE, FAKE, FAKE, 31, None) == bd.BD_EWORKSPACE
    assert c(FAKE, FAKE, 1, 4, 16, 1, FAKE, FAKE, None, 32, None) == bd.BD_EINVAL


def test_reconstruct_validation(bd):
    r = bd.lib.bitdelta_reconstruct
    assert r(FAKE, FAKE, FAKE, 0, 4, 20, FAKE, None) == bd.BD_ESHAPE
    assert r(FAKE, FAKE, FAKE, 5, 4, 16, FAKE, None) == bd.BD_EINVAL
    assert r(FAKE, None, FAKE, 0, 4, 16, FAKE, None) == bd.BD_EINVAL
    assert r(FAKE, FAKE, FAKE, 0, 4, 16, FAKE_ODD, None) == bd.BD_EALIGN


def test_linear_validation(bd):
    f = bd.lib.bitdelta_linear
    assert f(FAKE, 4, FAKE, FAKE, FAKE, 0, 8, 12, FAKE, None, 0, None) == bd.BD_ESHAPE
    assert f(FAKE, -1, FAKE, FAKE, FAKE, 0, 8, 16, FAKE, None, 0, None) == bd.BD_ESHAPE
    assert f(FAKE, 4, FAKE, FAKE, FAKE, 3, 8, 16, FAKE, None, 0, None) == bd.BD_EINVAL
    assert f(None, 4, FAKE, FAKE, FAKE, 0, 8, 16, FAKE, None, 0, None) == bd.BD_EINVAL
    assert f(FAKE, 4, FAKE, FAKE, FAKE, 0, 8, 16, None, None, 0, None) == bd.BD_EINVAL
    assert f(FAKE_ODD, 4, FAKE, FAKE, FAKE, 0, 8, 16, FAKE, None, 0, None) == bd.BD_EALIGN
    assert f(FAKE, 40, FAKE, FAKE, FAKE, 0, 8, 16, FAKE_ODD, None, 0, None) == bd.BD_EALIGN
    # m = 0 is a no-op, whatever the (unused) pointers are
    assert f(None, 0, None, None, None, 0, 8, 16, None, None, 0, None) == bd.BD_OK
    assert bd.lib.bitdelta_linear_workspace(4096, 4096, 4096) == 0


def test_decode_rejects_rows_past_32bit_offsets(bd):
    """The decode kernels address W_base in chunks of at least 16 rows (and x)
    through 32-bit buffer offsets: a d_in whose 16 rows reach 2 GiB is a shape
    error, not a silent wrap.  The boundary itself still validates further."""
    f = bd.lib.bitdelta_linear
    lim = (1 << 31) // (16 * 2)            # 16 rows of bf16 reach 2 GiB at d_in = 2^26
    for m in (1, 4, 16):
        assert f(FAKE, m, FAKE, FAKE, FAKE, 0, 1, lim, FAKE, None, 0, None) == bd.BD_ESHAPE, m
        assert "2 GiB" in err(bd)
        assert f(FAKE, m, FAKE, FAKE, FAKE, 0, 1, 1 << 27, FAKE, None, 0, None) == bd.BD_ESHAPE
    # one step below the limit passes the shape check and fails only on the
    # (deliberately misaligned) output pointer, so nothing is launched
    assert f(FAKE, 16, FAKE, FAKE, FAKE, 0, 1, lim - 8, FAKE_ODD, None, 0, None) == bd.BD_EALIGN


def test_linear_split_k_workspace(bd):
    """Prefill with few 256 x 256 output tiles splits K, and so does a last
    partial wave of at most 128 tiles; the workspace holds one fp32 partial
    tile per split tile and range.  With at most 128 tiles of 256 x 256 the
    tiles are 256 x 128 (twice as many, half the K ranges) where the wide
    plan's K ranges are at most 1024 columns or narrow tiles need no split."""
    W = bd.lib.bitdelta_linear_workspace
    tile = 256 * 256 * 4
    narrow = 256 * 128 * 4
    assert W(16, 64, 4096) == 0                    # decode path: few rows of short width
    # decode on 512..2048 rows of at least 8192 columns: the row's steps in parts, fp32 sums per part
    assert W(16, 1024, 8192) == 4 * 16 * 1024 * 4
    assert W(8, 2048, 8192) == 2 * 8 * 2048 * 4
    assert W(16, 1000, 28672) == 7 * 16 * 1000 * 4
    assert W(3, 1024, 28672) == 7 * 3 * 1024 * 4   # m = 3 with x above 64 KB: the whole-row kernel
    assert W(4, 1024, 8192) == 0 and W(2, 1024, 8192) == 0 and W(1, 1024, 8192) == 0   # stream kernels
    assert W(16, 511, 8192) == 0 and W(16, 2049, 8192) == 0 and W(16, 1024, 4096) == 0
    f = bd.lib.bitdelta_linear
    assert f(FAKE, 16, FAKE, FAKE, FAKE, 0, 1024, 8192, FAKE, None, 0, None) == bd.BD_EWORKSPACE
    assert W(2048, 8192, 8192) == 0                # 256 tiles fill the chip
    assert W(2048, 8192, 28672) == 0
    assert W(2048, 28672, 8192) == 2 * 128 * tile  # 896 tiles: last 128 in 2 K ranges
    assert W(4000, 4128, 4096) == 2 * 16 * tile    # 272 tiles: K/2 = 2048 is the floor
    assert W(256, 256 * 264, 15872) == 4 * 8 * tile   # 264 tiles: last 8 in 4 K ranges (K/8 < 2048)
    assert W(256, 256 * 264, 16384) == 0           # W_base of 2 GiB or more: rejected, no workspace
    assert W(4096, 6400, 8192) == 0                # last wave of 144 tiles: over half the CUs
    assert W(4096, 4352, 2048) == 0                # K/2 = 1024: too short to repay the sum
    assert W(512, 28672, 8192) == 0                # 224 tiles: one wave
    assert W(600, 64, 4096) == 8 * 3 * narrow      # 3 narrow tiles, K/8 = 512 per split
    assert W(2048, 1024, 8192) == 4 * 64 * narrow  # 64 narrow tiles x 4 splits = 256
    assert W(40, 1024, 8192) == 16 * 8 * narrow    # 8 narrow tiles, capped at 16 splits
    assert W(512, 8192, 28672) == 4 * 64 * tile    # wide ranges of 7168 columns: stays 256 wide
    assert W(512, 8192, 8192) == 4 * 64 * tile      # wide ranges of 2048 columns: stays 256 wide
    assert W(1024, 4096, 4096) == 2 * 128 * narrow  # wide ranges of 1024 columns: narrow, K in 2
    assert W(512, 256 * 80, 8192) == 2 * 160 * tile  # 160 tiles (over 128): 256 wide, K in 2
    assert W(256, 256 * 128, 4096) == 0            # 256 narrow tiles fill the chip unsplit
    assert W(600, 64, 1032) == 0                   # d_in not a multiple of 64: general kernel
    assert W(600, 80, 4096) == 0                   # d_out not a multiple of 32: general kernel
    assert W(600, 64, 960) == 0                    # K too short to split
    f = bd.lib.bitdelta_linear
    need = W(600, 64, 4096)
    assert f(FAKE, 600, FAKE, FAKE, FAKE, 0, 64, 4096, FAKE, FAKE, need - 1, None) == bd.BD_EWORKSPACE
    assert f(FAKE, 600, FAKE, FAKE, FAKE, 0, 64, 4096, FAKE, None, need, None) == bd.BD_EINVAL
    assert f(FAKE, 600, FAKE, FAKE, FAKE, 0, 64, 4096, FAKE, FAKE_ODD, need, None) == bd.BD_EALIGN


def test_grouped_validation(bd):
    g = bd.lib.bitdelta_linear_grouped
    W = bd.lib.bitdelta_linear_grouped_workspace
    need = W(100, 3, 64, 64)
    assert need >= 4 * (100 + 4)
    assert g(FAKE, 100, FAKE, 0, FAKE, FAKE, FAKE, 0, 64, 64, FAKE, FAKE, need, None) == bd.BD_EINVAL
    assert g(FAKE, 100, FAKE, 5000, FAKE, FAKE, FAKE, 0, 64, 64, FAKE, FAKE, 1 << 30, None) == bd.BD_EINVAL
    assert g(FAKE, 100, FAKE, 3, FAKE, FAKE, FAKE, 0, 64, 60, FAKE, FAKE, need, None) == bd.BD_ESHAPE
    assert g(FAKE, 100, FAKE, 3, FAKE, FAKE, FAKE, 0, 64, 64, FAKE, FAKE, need - 1, None) == bd.BD_EWORKSPACE
    assert g(FAKE, 100, None, 3, FAKE, FAKE, FAKE, 0, 64, 64, FAKE, FAKE, need, None) == bd.BD_EINVAL
    assert g(FAKE, 100, ctypes.c_void_p(4098), 3, FAKE, FAKE, FAKE, 0, 64, 64, FAKE, FAKE, need, None) == bd.BD_EALIGN
    assert g(None, 0, None, 3, None, None, None, 0, 64, 64, None, None, W(0, 3, 64, 64), None) == bd.BD_OK


def test_grouped_noalloc_validation(bd):
    """bitdelta_linear_grouped_noalloc: the grouped checks, plus its token limit
    (the size of the library's table); every call below fails before any
    device call, and m = 0 is a no-op."""
    g = bd.lib.bitdelta_linear_grouped_noalloc
    assert g(FAKE, 100, FAKE, 0, FAKE, FAKE, FAKE, 0, 64, 64, FAKE, None) == bd.BD_EINVAL
    assert g(FAKE, 100, FAKE, 4097, FAKE, FAKE, FAKE, 0, 64, 64, FAKE, None) == bd.BD_EINVAL
    assert g(FAKE, 100, FAKE, 3, FAKE, FAKE, FAKE, 0, 64, 60, FAKE, None) == bd.BD_ESHAPE
    assert g(FAKE, 65537, FAKE, 3, FAKE, FAKE, FAKE, 0, 64, 64, FAKE, None) == bd.BD_ESHAPE
    assert "65536" in err(bd)
    assert g(FAKE, 100, None, 3, FAKE, FAKE, FAKE, 0, 64, 64, FAKE, None) == bd.BD_EINVAL
    assert g(FAKE, 100, FAKE, 3, FAKE, FAKE, FAKE, 0, 64, 64, FAKE_ODD, None) == bd.BD_EALIGN
    assert g(FAKE, 100, FAKE, 3, FAKE, FAKE, FAKE, 2, 64, 64, FAKE, None) == bd.BD_EINVAL
    assert g(None, 0, None, 3, None, None, None, 0, 64, 64, None, None) == bd.BD_OK


def test_python_binding_rejects_host_tensors(bd):
    import torch

    w = torch.zeros(8, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        bd.compress(w, w.float())
    with pytest.raises(ValueError):
        bd.linear(torch.zeros(2, 16, dtype=torch.bfloat16), w, torch.zeros(8, 2, dtype=torch.uint8),
                  torch.zeros(8))


def test_launch_without_device_reports_edevice(bd):
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: this case is only for hosts without one")
    # Valid arguments: validation passes and the launch itself fails (no device),
    # so no memory is ever touched.
    st = bd.lib.bitdelta_reconstruct(FAKE, FAKE, FAKE, 0, 4, 16, FAKE, None)
    assert st == bd.BD_EDEVICE, st
    assert "bitdelta_reconstruct" in err(bd)


def test_monosoup_validation(bd):
    """Host-side checks of bitdelta_monosoup (FAKE pointers never touched) and
    the workspace formula: split partials, the two sketches, the whitened
    copy, fp64 partial and summed Grams, the two 64 x 64 factors and the
    merge factors."""
    W = bd.lib.bitdelta_monosoup_workspace
    f = bd.lib.bitdelta_monosoup
    assert W(8192, 8192, 2, 0) == 0                      # rank 0: a copy of W_base, no scratch
    assert W(0, 64, 1, 8) == 0 and W(64, 2, 1, 8) == 0 and W(64, 64, 0, 8) == 0 and W(64, 64, 1, 65) == 0

    def a256(x):
        return (x + 255) // 256 * 256

    # 8192 x 8192, k = 2, r = 32: 256 blocks of 64 per pass -> 4 splits of 32 steps
    R = C = 8192
    expect = (a256(2 * 64 * 4 * R * 4) + a256(2 * R * 64 * 4) + a256(2 * C * 64 * 4) + a256(2 * R * 64 * 4)
              + 2 * a256(2 * 64 * 64 * 64 * 8) + 4 * a256(2 * 64 * 64 * 8) + a256(R * 64 * 4) + a256(C * 64 * 4))
    assert W(R, C, 2, 32) == expect
    need = W(100, 96, 2, 8)
    ok = (FAKE, FAKE, FAKE, 2, 100, 96, 8, 1, FAKE, FAKE, FAKE, need, None)

    def call(**kw):
        a = list(ok)
        names = ["wb", "wf", "om", "k", "R", "C", "r", "q", "out", "sig", "ws", "nws", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(C=98) == bd.BD_ESHAPE and call(C=0) == bd.BD_ESHAPE and call(R=0) == bd.BD_ESHAPE
    assert call(R=(1 << 21) + 1) == bd.BD_ESHAPE
    assert call(k=0) == bd.BD_EINVAL and call(k=65) == bd.BD_EINVAL
    assert call(r=-1) == bd.BD_EINVAL and call(r=65) == bd.BD_EINVAL
    assert call(R=20, r=21) == bd.BD_EINVAL                # rank above min(rows, cols)
    assert call(q=-1) == bd.BD_EINVAL and call(q=257) == bd.BD_EINVAL
    assert call(nws=need - 1) == bd.BD_EWORKSPACE
    assert call(wb=None) == bd.BD_EINVAL and call(out=None) == bd.BD_EINVAL and call(om=None) == bd.BD_EINVAL
    assert call(ws=None) == bd.BD_EINVAL
    assert call(wf=ctypes.c_void_p(4104)) == bd.BD_EALIGN
    assert call(om=ctypes.c_void_p(4104)) == bd.BD_EALIGN
    assert call(wb=ctypes.c_void_p(4100)) == bd.BD_EALIGN
    assert call(sig=ctypes.c_void_p(4100)) == bd.BD_EALIGN
    assert call(out=ctypes.c_void_p(4100)) == bd.BD_EALIGN
    assert call(ws=ctypes.c_void_p(4096 + 128)) == bd.BD_EALIGN


def test_similarity_validation(bd):
    """Host-side checks of bitdelta_similarity: every failing call returns
    before a launch (FAKE pointers are never dereferenced)."""
    W = bd.lib.bitdelta_similarity_workspace
    f = bd.lib.bitdelta_similarity
    assert W(14, 8192, 8192) == 4 * 8192 * 91        # int32 per row and pair
    assert W(2, 100, 64) == 4 * 100 * 1
    assert W(1, 100, 64) == 0                        # one variant: no pairs
    assert W(17, 100, 64) == 0 and W(0, 100, 64) == 0
    need = W(4, 64, 256)
    ok = (FAKE, FAKE, 0, 4, 64, 256, FAKE, FAKE, FAKE, need, None)

    def call(**kw):
        a = list(ok)
        names = ["signs", "alpha", "mode", "V", "d_out", "d_in", "gram", "cos", "ws", "nws", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(mode=2) == bd.BD_EINVAL
    assert call(V=0) == bd.BD_EINVAL and call(V=17) == bd.BD_EINVAL
    assert call(d_in=200) == bd.BD_ESHAPE              # multiple of 8, not of 32
    assert call(d_in=12) == bd.BD_ESHAPE and call(d_out=0) == bd.BD_ESHAPE
    assert call(V=16, d_out=1 << 20, d_in=1024) == bd.BD_ESHAPE  # signs of 2 GiB
    assert call(nws=need - 1) == bd.BD_EWORKSPACE
    assert call(signs=None) == bd.BD_EINVAL and call(gram=None) == bd.BD_EINVAL
    assert call(ws=None) == bd.BD_EINVAL
    assert call(signs=FAKE_ODD) == bd.BD_EALIGN
    assert call(gram=ctypes.c_void_p(4100)) == bd.BD_EALIGN
    assert call(ws=FAKE_ODD) == bd.BD_EALIGN


def test_similarity_delta_validation(bd):
    """Host-side checks of bitdelta_similarity_delta (FAKE pointers are never
    dereferenced: every call below fails before a launch)."""
    W = bd.lib.bitdelta_similarity_delta_workspace
    f = bd.lib.bitdelta_similarity_delta
    assert W(14, 8192, 8192) == 8 * 8192 * 105       # fp64 per row and pair, diagonal included
    assert W(1, 100, 64) == 8 * 100
    assert W(17, 100, 64) == 0 and W(0, 100, 64) == 0
    need = W(4, 64, 256)
    ok = (FAKE, FAKE, 1, 4, 64, 256, FAKE, FAKE, FAKE, need, None)

    def call(**kw):
        a = list(ok)
        names = ["wb", "wft", "ft", "V", "d_out", "d_in", "gram", "cos", "ws", "nws", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(ft=2) == bd.BD_EINVAL
    assert call(V=0) == bd.BD_EINVAL and call(V=17) == bd.BD_EINVAL
    assert call(d_in=12) == bd.BD_ESHAPE and call(d_out=0) == bd.BD_ESHAPE and call(d_in=0) == bd.BD_ESHAPE
    assert call(nws=need - 1) == bd.BD_EWORKSPACE
    assert call(wb=None) == bd.BD_EINVAL and call(wft=None) == bd.BD_EINVAL
    assert call(gram=None) == bd.BD_EINVAL and call(cos=None) == bd.BD_EINVAL and call(ws=None) == bd.BD_EINVAL
    assert call(wb=FAKE_ODD) == bd.BD_EALIGN and call(wft=ctypes.c_void_p(4104)) == bd.BD_EALIGN
    assert call(gram=ctypes.c_void_p(4100)) == bd.BD_EALIGN and call(ws=ctypes.c_void_p(4100)) == bd.BD_EALIGN


def test_probe_validation(bd):
    """The measurement probes check their sizes, pointers and alignment on the
    host; the read probe's sink holds one word per wave of 8 runs of 1 KB."""
    L = bd.lib
    words = L.bitdelta_probe_read_sink_words
    assert words(16) == 4 and words(32 * 1024) == 4 and words(32 * 1024 + 16) == 8
    assert words(34 * 2 ** 20) == 4 * -(-34 * 1024 // 32)
    for bad in (0, 8, 24, -16, 2 ** 31):
        assert words(bad) == 0
        assert L.bitdelta_probe_read(FAKE, bad, FAKE, None) == bd.BD_ESHAPE
    assert L.bitdelta_probe_read(None, 1024, FAKE, None) == bd.BD_EINVAL
    assert L.bitdelta_probe_read(FAKE, 1024, None, None) == bd.BD_EINVAL
    assert L.bitdelta_probe_read(FAKE_ODD, 1024, FAKE, None) == bd.BD_EALIGN
    assert L.bitdelta_probe_read(FAKE, 1024, FAKE_ODD, None) == bd.BD_EALIGN
    m = L.bitdelta_probe_mfma
    for blocks, iters in ((0, 1), (1, 0), (2 ** 20 + 1, 1), (1, 2 ** 20 + 1), (-1, 5)):
        assert m(blocks, iters, 1.0, 1.0, FAKE, None) == bd.BD_ESHAPE
    assert m(1, 1, 1.0, 1.0, None, None) == bd.BD_EINVAL
    assert m(1, 1, 1.0, 1.0, FAKE_ODD, None) == bd.BD_EALIGN
    p = L.bitdelta_probe_lds
    for mode in (-1, 4):
        assert p(1, 1, mode, 1, FAKE, 1024, FAKE, FAKE, None) == bd.BD_EINVAL
    for blocks, iters, stride in ((0, 1, 1), (2 ** 20 + 1, 1, 1), (1, 0, 1), (1, 2 ** 16 + 1, 1), (1, 1, 0),
                                  (1, 1, 2 ** 20 + 1)):
        assert p(blocks, iters, 0, stride, None, 0, FAKE, FAKE, None) == bd.BD_ESHAPE
    for nbytes in (0, 512, 1536, 3 * 1024, 2 ** 31):
        assert p(1, 1, 3, 1, FAKE, nbytes, FAKE, FAKE, None) == bd.BD_ESHAPE
    assert p(1, 1, 3, 1, None, 1024, FAKE, FAKE, None) == bd.BD_EINVAL
    assert p(1, 1, 3, 1, ctypes.c_void_p(4104), 1024, FAKE, FAKE, None) == bd.BD_EALIGN
    assert p(1, 1, 0, 1, None, 0, None, FAKE, None) == bd.BD_EINVAL
    assert p(1, 1, 0, 1, None, 0, FAKE, None, None) == bd.BD_EINVAL
    assert p(1, 1, 0, 1, None, 0, FAKE_ODD, FAKE, None) == bd.BD_EALIGN
    assert p(1, 1, 0, 1, None, 0, FAKE, ctypes.c_void_p(4100), None) == bd.BD_EALIGN
