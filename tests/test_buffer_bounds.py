"""CPU tier: a model of the buffer addressing of the decode, prefill and
similarity kernels, checked against the raw-buffer range-check rule.

A raw buffer access on this GPU checks only its lane (VGPR) offset against
the resource's size; the scalar (SGPR) offset is added after the check.  An
access whose lane offset is in range therefore touches bytes
[lane + scalar, lane + scalar + width) whatever they are, and those must lie
inside the tensor.  Each function below restates, in numpy, the (lane offset,
scalar offset, width) of every load a kernel issues, for every workgroup,
wave, lane and step of a launch, and the tests assert that no in-range access
reaches past its tensor, on ragged and even shapes.  A model of the earlier
prefill addressing (16 activation rows further in the scalar offset) is
checked to fail, so the check can see the mistake it guards against.

The formulas follow the kernels in tenant_fine_tune_amd/csrc (gemv.hip,
gemm.hip, similarity.hip); a change of a kernel's addressing needs the same
change here.
"""
import numpy as np
import pytest

INV = 0x80000000


def _violations(vo, so, width, tensor_bytes):
    """Accesses whose lane offset passes the range check but whose bytes end
    past the tensor (numpy arrays broadcast together)."""
    vo = np.asarray(vo, dtype=np.int64)
    so = np.asarray(so, dtype=np.int64)
    vo, so = np.broadcast_arrays(vo, so)
    checked = vo < tensor_bytes
    end = vo + so + width
    return int(np.count_nonzero(checked & (end > tensor_bytes)))


# ------------------------------------------------------------------ decode

def gemv_stream_accesses(R, K, m, MT, RW, waves, even, mask_weights=True):
    G = K // 8
    S = (G + 63) // 64
    blocks = -(-R // (waves * RW))
    b, w, l, r, s = np.meshgrid(np.arange(blocks), np.arange(waves), np.arange(64), np.arange(RW), np.arange(S),
                                indexing="ij")
    row0 = (b * waves + w) * RW
    ok = row0 + r < R
    wrow = np.where(ok, (row0 + r) * K * 2 + 16 * l, INV)
    srow = np.where(ok, (row0 + r) * G + l, INV)
    live = np.ones_like(ok) if even else (s * 64 + l < G)
    wlive = live if mask_weights else np.ones_like(live)
    out = [("W_base", np.where(wlive, wrow, INV), s * 1024, 16, R * K * 2),
           ("signs", np.where(wlive, srow, INV), s * 64, 1, R * G)]
    for t in range(MT):
        xrow = t * K * 2 + 16 * l if t < m else np.full_like(l, INV)
        out.append((f"x[{t}]", np.where(live, xrow, INV), s * 1024, 16, m * K * 2))
    return out


def gemv_mfma_accesses(R, K, m, even):
    G = K // 8
    T = -(-K // 128)
    KW = 8
    blocks = -(-R // 16)
    out = []
    b, w, l = np.meshgrid(np.arange(blocks), np.arange(KW), np.arange(64), indexing="ij")
    j, q = l % 16, l // 16
    n0 = b * 16
    row_ok = n0 + j < R
    wrow = np.where(row_ok, (n0 + j) * K * 2 + 16 * q, INV)
    srow = np.where(row_ok, (n0 + j) * G, INV)
    xrow = np.where(j < m, j * K * 2 + 16 * q, INV)
    nt = np.where(T > w, (T - 1 - w) // KW + 1, 0)
    for t in range(int(nt.max()) + 2):  # two dead stages past the last live one
        live = t < nt
        sb = w + t * KW
        so = sb * 256
        wv = np.where(live, wrow, INV)
        sv = np.where(live, srow, INV)
        if even:
            out.append(("signs", sv, sb * 16, 16, R * G))
        for jj in range(4):
            ok = live if even else live & (sb * 16 + 4 * jj + q < G)
            if not even:
                out.append(("signs", np.where(ok, sv + 4 * jj + q, INV), sb * 16, 1, R * G))
            out.append(("W_base", np.where(ok, wv + 64 * jj, INV), so, 16, R * K * 2))
            out.append(("x", np.where(ok, xrow + 64 * jj, INV), so, 16, m * K * 2))
    return out


def gemv_rows_accesses(R, K, m, RW=1, splits=1):
    """gemv_rows (d_in a multiple of 4096): 16 waves per workgroup of 16 RW
    rows, wave w streams rows n0 + w + 16 k (k < RW) in 512-column steps (1 KB
    per instruction), starting at step b mod S (RW = 1) or (b + b // 8) mod S
    (RW = 2); lane (j, q) reads x[j][32 w + 8 q ..] of the step's columns.
    With splits > 1, workgroup (block b, part p) walks steps
    p S' .. p S' + S' - 1 (S' = S / splits) starting at p S' + b mod S'."""
    assert K % 4096 == 0
    G, S = K // 8, K // 512
    assert S % splits == 0
    Sp = S // splits
    blocks = -(-R // (16 * RW))
    b, w, l = np.meshgrid(np.arange(blocks), np.arange(16), np.arange(64), indexing="ij")
    j, q = l & 15, l >> 4
    xoff = np.where(j < m, j * K * 2 + (32 * w + 8 * q) * 2, INV)
    out = []
    for p in range(splits):
        rot = b % Sp if RW == 1 else (b + (b >> 3)) % Sp
        steps = [p * Sp + (s + rot) % Sp for s in range(Sp)]
        # every workgroup visits each of its part's steps once
        assert np.array_equal(np.sort(np.stack([st[:, 0, 0] for st in steps]), axis=0),
                              np.broadcast_to(p * Sp + np.arange(Sp)[:, None], (Sp, blocks)))
        for k in range(RW):
            row = b * 16 * RW + w + 16 * k
            ok = row < R
            wrow = np.where(ok, row * K * 2 + 16 * l, INV)
            srow = np.where(ok, row * G + l, INV)
            for c in steps:
                out.append(("W_base", wrow, c * 1024, 16, R * K * 2))
                out.append(("signs", srow, c * 64, 1, R * G))
        for c in steps:
            out.append(("x", xoff, c * 1024, 16, m * K * 2))
    return out


def gemv_splits(m, R, K):
    """The launcher's split count for few rows of long width (1 = none)."""
    if not (m > 4 or (m > 2 and m * K * 2 > 64 * 1024)) or K % 4096 or K < 8192:
        return 1
    blocks = -(-R // 16)
    if R < 512 or blocks > 128 or R * K * 2 >= 1 << 30:
        return 1
    S, target, best = K // 512, -(-256 // blocks), 1
    for sp in range(2, S // 4 + 1):
        if S % sp or (S // sp) % 4:
            continue
        best = sp
        if sp >= target:
            break
    return best


def gemv_rows_plan(R, K):
    """Rows per wave the launcher picks: 2 for rows longer than one ring (4096)
    when there are at least 8192 of them, else 1."""
    return 2 if K > 4096 and R >= 32 * 256 else 1


@pytest.mark.parametrize("R,K", [(1000, 4096), (33, 8192), (24, 4096), (7, 12288), (16, 4096), (1, 4096),
                                 (8208, 8192), (8192, 12288), (8200, 8192)])
@pytest.mark.parametrize("m", [3, 5, 13, 16])
def test_gemv_rows_stays_in_bounds(R, K, m):
    RW = gemv_rows_plan(R, K)
    for name, vo, so, width, size in gemv_rows_accesses(R, K, m, RW):
        assert _violations(vo, so, width, size) == 0, (name, R, K, m, RW)


@pytest.mark.parametrize("R,K,m,splits", [(1024, 8192, 16, 4), (1000, 28672, 16, 7), (512, 8192, 5, 4),
                                          (2048, 8192, 8, 2), (1000, 28672, 3, 7), (1025, 12288, 16, 6)])
def test_gemv_rows_split_stays_in_bounds(R, K, m, splits):
    """Few rows: the row's steps in parts of whole rings, every part's scalar
    offsets inside the row; the plan's split count is the one modelled."""
    assert gemv_splits(m, R, K) == splits
    for name, vo, so, width, size in gemv_rows_accesses(R, K, m, 1, splits):
        assert _violations(vo, so, width, size) == 0, (name, R, K, m, splits)


@pytest.mark.parametrize("R,K", [(33, 8192), (7, 12288), (17, 8192), (1, 8192)])
def test_gemv_rows_two_row_plan_stays_in_bounds_on_ragged_rows(R, K):
    """The two-row addressing on row counts that leave partial 32-row blocks."""
    for name, vo, so, width, size in gemv_rows_accesses(R, K, 16, 2):
        assert _violations(vo, so, width, size) == 0, (name, R, K)


@pytest.mark.parametrize("R,K", [(1, 8), (3, 520), (17, 1032), (5, 4096), (33, 1544), (64, 4104), (7, 24)])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_gemv_stream_stays_in_bounds(R, K, m):
    MT, RW, waves = {1: (1, 1, 4), 2: (2, 2, 8), 3: (4, 1, 8), 4: (4, 1, 8)}[m]
    even = (K // 8) % 64 == 0
    if m == 2 and even and m * K * 2 <= 64 * 1024:
        RW = 1  # x in LDS: one row per wave
    for name, vo, so, width, size in gemv_stream_accesses(R, K, m, MT, RW, waves, even):
        assert _violations(vo, so, width, size) == 0, (name, R, K, m)


def test_gemv_model_sees_unmasked_ragged_steps():
    """Without the per-lane mask on W_base in a ragged last step (the earlier
    kernel), the last row's lanes past the row read past W_base."""
    acc = gemv_stream_accesses(3, 520, 1, 1, 1, 4, False, mask_weights=False)
    assert sum(_violations(vo, so, w, sz) for name, vo, so, w, sz in acc if name == "W_base") > 0


@pytest.mark.parametrize("R,K", [(1, 8), (3, 136), (17, 1032), (16, 4096), (33, 1544), (20, 4104), (7, 24)])
@pytest.mark.parametrize("m", [5, 16])
def test_gemv_mfma_stays_in_bounds(R, K, m):
    even = K % 128 == 0
    for name, vo, so, width, size in gemv_mfma_accesses(R, K, m, even):
        assert _violations(vo, so, width, size) == 0, (name, R, K, m)


# ----------------------------------------------------------------- prefill

def w8_accesses(M, N, K, splits=1, old_x=False, tn=256):
    """gemm_tiles_w8, dense: 256 x tn tiles (tn = 256 or 128), K steps of 64,
    8 waves, each loading tn / 8 rows of W_base in groups of 8."""
    assert K % 64 == 0 and tn in (256, 128)
    G = K // 8
    ng = tn // 64
    m_tiles, n_tiles = -(-M // 256), -(-N // tn)
    ks = K if splits == 1 else -(-(-(-K // splits)) // 64) * 64
    out = []
    mt, nt, wave, l = np.meshgrid(np.arange(m_tiles), np.arange(n_tiles), np.arange(8), np.arange(64),
                                  indexing="ij")
    m0, n0 = mt * 256, nt * tn
    p = l & 7
    for ky in range(-(-K // ks)):
        k_begin = ky * ks
        T = (min(K, k_begin + ks) - k_begin) // 64
        kx0, ks0 = k_begin * 2, k_begin // 8
        for t in range(T):
            kb = kx0 + t * 128
            for j in range(4):
                jj = (j & 1) if old_x else j
                row = wave * 32 + jj * 8 + (l >> 3)
                c = p ^ (((jj & 1) * 4 + (l >> 4)) & 7)
                tok = m0 + row
                vo = np.where(tok < M, (tok * K + c * 8) * 2, INV)
                so = kb + ((j >> 1) * 16 * K * 2 if old_x else 0)
                out.append(("x", vo, so, 16, M * K * 2))
            nw = n0 + wave * (8 * ng) + (l >> 3)
            woff = np.where(nw < N, (nw * K + p * 8) * 2, INV)
            soff = np.where(nw < N, nw * G + p, INV)
            for i in range(ng):
                out.append(("W_base", woff, kb + i * 8 * K * 2, 16, N * K * 2))
                out.append(("signs", soff, ks0 + t * 8 + i * 8 * G, 1, N * G))
    return out


def w8_shape(N, K):
    return K % 64 == 0 and N % 32 == 0


@pytest.mark.parametrize("M,N,K", [(17, 32, 64), (300, 96, 128), (257, 288, 192), (40, 1024, 512),
                                   (600, 64, 4096), (513, 544, 256), (1000, 320, 64)])
def test_prefill_stays_in_bounds(M, N, K):
    assert w8_shape(N, K)
    for tn in (256, 128):
        for splits in (1, 2):
            for name, vo, so, width, size in w8_accesses(M, N, K, splits, tn=tn):
                assert _violations(vo, so, width, size) == 0, (name, M, N, K, splits, tn)


def test_prefill_model_sees_rows_in_the_scalar_offset():
    """The earlier addressing (rows 16 further in the scalar offset) reads past
    x when M is not a multiple of 32: the model must flag it."""
    bad = sum(_violations(vo, so, w, sz) for name, vo, so, w, sz in w8_accesses(300, 96, 128, old_x=True)
              if name == "x")
    assert bad > 0
    ok = sum(_violations(vo, so, w, sz) for name, vo, so, w, sz in w8_accesses(320, 96, 128, old_x=True)
             if name == "x")
    assert ok == 0


def test_prefill_w_rows_need_whole_32_row_blocks():
    """W_base rows 8, 16, 24 further go in the scalar offset; with N not a
    multiple of 32 that reads past W_base, which is why such shapes run on the
    general kernel (all offsets in the lane offset)."""
    for tn, n in ((256, 80), (128, 72)):  # a wave's 32 (16) rows straddle N
        bad = sum(_violations(vo, so, w, sz) for name, vo, so, w, sz in w8_accesses(64, n, 64, tn=tn)
                  if name in ("W_base", "signs"))
        assert bad > 0
    assert not w8_shape(80, 64)


# -------------------------------------------------------------- similarity

def similarity_accesses(V, R, K):
    G = K // 8
    even = G % 64 == 0
    nk = (G + 63) // 64
    blocks = -(-R // 16)
    out = []
    b, w, l = np.meshgrid(np.arange(blocks), np.arange(4), np.arange(64), indexing="ij")
    j, q = l & 15, l >> 4
    row = b * 16 + j
    row_ok = row < R
    base = np.where(row_ok, row * G + 16 * q, INV)
    size = V * R * G
    for k in range(nk + 4):
        wave_has = (k % 4) == w  # wave w takes chunks w, w + 4, ...
        if even:
            vo = np.where(wave_has & (k < nk), base, INV)
            for v in range(V):
                out.append(("signs", vo, k * 64 + v * R * G, 16, size))
        else:
            start = k * 64 + 16 * q
            for i in range(4):
                vo = np.where(wave_has & row_ok & (start + 4 * i < G), base + k * 64 + 4 * i, INV)
                for v in range(V):
                    out.append(("signs", vo, v * R * G, 4, size))
    return out


@pytest.mark.parametrize("V,R,K", [(2, 17, 32), (3, 5, 544), (14, 33, 4128), (4, 16, 4096), (2, 1, 4096)])
def test_similarity_stays_in_bounds(V, R, K):
    for name, vo, so, width, size in similarity_accesses(V, R, K):
        assert _violations(vo, so, width, size) == 0, (name, V, R, K)
