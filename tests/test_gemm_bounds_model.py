"""Host-side model of the W4A4 GEMM's global -> LDS loads: where the hardware may fetch.

The kernel loads 16 bytes per lane through raw buffer resources over each tile's rows.  The
range check of a raw resource covers the VGPR offset only (row and 16-byte chunk here); the
SGPR offset is added to the address after it.  The model mirrors the kernel's offset
arithmetic (tile rows, the K walk's starting buffer by tile column parity, the XOR chunk
swizzle, the scale groups, every issue including those past the end of K with their
out-of-range sentinel), assumes the check admits a dword when VGPR offset + 4 <=
num_records, and compares the admitted dwords' addresses with the operand's size.

* The scale loads carry their column in the VGPR offset, so the range check covers it: a
  half last scale group (K % 512 != 0) reads zeros past the operand's last row.
* The code loads carry their column in the SGPR offset, except for the half last buffer
  of a ragged K (K % 256 == 128), whose column goes into the VGPR offset.
* As built, nothing is fetched outside any operand.  With every code column in the SGPR
  offset (the earlier form) a ragged K reads up to 64 bytes past the codes' last row; with
  the scale column there, a half last scale group reads past the scales' last row.  The
  model checks both, so a change of either placement is caught.
* A withdrawn form moved the code column into the resource base and subtracted it from
  the record count; the model shows that a count which wraps round admits the sentinel
  offset (2 GiB past the operand), and a saturating one does not.
"""
import numpy as np
import pytest

BM = BN = 256
BKP, ROWB = 256, 128
NW, QW, SW = 8, 4, 1
KSCALE_ROW = 16


def _swz(row):
    return (row >> 1) & 7


def _lane_offsets(rowbytes, rowscales):
    """Per wave, per issue index: VGPR offsets of the 64 lanes (codes: QW x 64; scales:
    SW x 64), as the kernel builds them."""
    lane = np.arange(64)
    codes, scales = [], []
    for wave in range(NW):
        cq = []
        for q in range(QW):
            qq = q & 1
            row = 8 * (QW * wave + qq) + (lane >> 3)
            base = row * rowbytes + 16 * ((lane & 7) ^ _swz(row))
            cq.append(base + (q & ~1) * 8 * rowbytes)
        codes.append(cq)
        sq = []
        for q in range(SW):
            t = SW * wave + q
            sq.append((64 * (t & 3) + lane) * rowscales)
        scales.append(sq)
    return codes, scales


KOOB = 1 << 31          # the kernel's offset for an issue past the end of K


def _issues(np_):
    """(code buffer index or scale group, valid) in the kernel's issue order: the prologue
    (scale group 0, buffers 0 and 1, the latter out of range when np == 1), then at step p
    buffer p + 2 and, on even steps, scale group (p + 2) / 2, valid only below np."""
    codes = [(0, True), (1, np_ > 1)] + [(p + 2, p + 2 < np_) for p in range(np_)]
    scales = [(0, True)] + [((p + 2) >> 1, p + 2 < np_) for p in range(0, np_, 2)]
    return codes, scales


def _fetched_max(M, N, K, code_col_in_voff=True, scale_col_in_voff=True, base_shift=False, wrap=False):
    """Largest byte offset + 1 fetched from each operand (A codes, B codes, A scales,
    B scales) over every tile and issued load, or -1 if none.  `code_col_in_voff`: the
    ragged last code buffer's column in the VGPR offset (as built); `scale_col_in_voff`:
    the scale loads' column in the VGPR offset (as built).  `base_shift` models a withdrawn
    form of the code loads: the column moved into the resource base and subtracted from
    the record count, which saturates at zero, or wraps round with `wrap`."""
    rowbytes, rowscales = K // 2, K // 32
    np_ = (K + BKP - 1) // BKP
    ragged = K % BKP != 0
    tiles_m, tiles_n = (M + BM - 1) // BM, (N + BN - 1) // BN
    codes_off, scale_off = _lane_offsets(rowbytes, rowscales)
    code_issues, scale_issues = _issues(np_)
    top = {"a": -1, "b": -1, "sa": -1, "sb": -1}

    def admit(key, base, nrec, col, voff, valid, col_in_voff, shift=False):
        voff = np.asarray(voff, dtype=np.int64) if valid else np.full(64, KOOB, dtype=np.int64)
        vcol, scol = (col, 0) if col_in_voff else (0, col)
        if shift:
            base, scol = base + col, 0
            nrec = (nrec - col) % (1 << 32) if wrap else max(nrec - col, 0)
        voff = voff + vcol
        assert voff.max() < 1 << 32                 # the 32-bit offset never wraps
        for d in range(4):                          # the four dwords of a 16-byte load
            ok = voff + 4 * d + 4 <= nrec
            if ok.any():
                top[key] = max(top[key], int(base + scol + voff[ok].max() + 4 * d + 4))

    for tm in range(tiles_m):
        for tn in range(tiles_n):
            m0, n0 = tm * BM, tn * BN
            rows_a, rows_b = min(BM, M - m0), min(BN, N - n0)
            ne = 0 if ragged else np_ & ~1
            rot = 2 * (tn & 1) if ne >= 4 else 0
            vcol_buf = np_ - 1 if ragged and code_col_in_voff and not base_shift else -1

            def rotated(q):
                if q >= ne:
                    return q
                q += rot
                return q - ne if q >= ne else q

            for q, valid in code_issues:
                buf = rotated(q)
                col = buf * ROWB
                for key, r0, rows in (("a", m0, rows_a), ("b", n0, rows_b)):
                    for wave in range(NW):
                        for i in range(QW):
                            admit(key, r0 * rowbytes, rows * rowbytes, col, codes_off[wave][i], valid,
                                  buf == vcol_buf, base_shift)
            for h, valid in scale_issues:
                col = (rotated(2 * h) >> 1) * KSCALE_ROW
                for wave in range(NW):
                    for i in range(SW):
                        t = SW * wave + i
                        key, r0, rows = ("sb", n0, rows_b) if t >> 2 else ("sa", m0, rows_a)
                        admit(key, r0 * rowscales, rows * rowscales, col, scale_off[wave][i], valid,
                              scale_col_in_voff)
    return top


def _sizes(M, N, K):
    return {"a": M * K // 2, "b": N * K // 2, "sa": M * K // 32, "sb": N * K // 32}


# the GPU test shapes, plus the W4A4 configuration's K with small M, N
SHAPES = [(1, 1, 128), (64, 96, 256), (300, 260, 384), (256, 512, 1024), (1100, 1300, 1536), (777, 392, 512),
          (513, 257, 8192), (130, 70, 640), (200, 300, 1408), (300, 600, 8192), (300, 600, 768), (513, 520, 4352),
          (300, 1100, 1280)]


@pytest.mark.parametrize("M,N,K", SHAPES + [(256, 256, 4352), (300, 260, 4352), (1, 1, 384), (2, 3, 128)])
def test_fetches_of_the_kernel_as_built(M, N, K):
    """The kernel as built: every fetch stays inside its operand, and the last row of codes
    is read whole."""
    top = _fetched_max(M, N, K)
    size = _sizes(M, N, K)
    for key in top:
        assert top[key] <= size[key], (key, top[key], size[key])
    assert top["a"] == size["a"] and top["b"] == size["b"]


@pytest.mark.parametrize("K", [384, 640, 1408, 4224])
def test_code_column_in_the_sgpr_offset_would_read_past(K):
    """With every code column in the SGPR offset (the earlier form), a ragged K's last row
    of codes is followed by 64 fetched bytes past the operand; a K % 256 == 0 is not.
    (K = 128 has a single buffer, at column 0, where the two forms coincide.)"""
    for M, N in ((256, 256), (300, 260)):
        top = _fetched_max(M, N, K, code_col_in_voff=False)
        size = _sizes(M, N, K)
        assert top["a"] - size["a"] == 64 and top["b"] - size["b"] == 64
    top = _fetched_max(256, 256, K + 128, code_col_in_voff=False)
    assert top["a"] == _sizes(256, 256, K + 128)["a"]
    top = _fetched_max(256, 256, 128, code_col_in_voff=False)
    assert top["a"] == _sizes(256, 256, 128)["a"]


def test_scale_column_in_the_sgpr_offset_would_read_past():
    """With the column in the SGPR offset (the earlier form), a half last scale group reads
    8 bytes past the last row's scales at K = 4352 and 12 at K = 640."""
    for K, want in ((4352, 8), (640, 12)):
        top = _fetched_max(256, 256, K, scale_col_in_voff=False)
        assert top["sa"] - _sizes(256, 256, K)["sa"] == want


def test_the_sentinel_stays_out_of_range_with_a_column_added():
    """An issue past the end of K carries the sentinel offset 2^31; on the ragged last
    buffer the column is added to it.  The library admits M K / 2 < 2^31 only, so the
    sum still exceeds every resource's record count, and stays below 2^32."""
    for K in (128, 384):
        np_ = (K + BKP - 1) // BKP
        col = (np_ - 1) * ROWB
        rows_max = ((1 << 31) - 1) // (K // 2)
        nrec = min(BM, rows_max) * (K // 2)
        assert KOOB + col + 16 > nrec and KOOB + col + 16 <= 1 << 32


def test_a_wrapping_resource_count_would_admit_the_sentinel():
    """The withdrawn base-shift form at M = N = 1, K = 128: past the end, step 0's refill
    (q = 2) has a column beyond the operand's 64 bytes (128 in the walk of that time, which
    wrapped it to buffer 1; 256 now).  A count that wraps round to about 4 GiB admits the
    out-of-range offset and fetches 2 GiB past the operand (the cause of a GPU fault); a
    saturating count admits nothing beyond it."""
    top = _fetched_max(1, 1, 128, base_shift=True, wrap=True)
    assert top["a"] > (1 << 31)
    top = _fetched_max(1, 1, 128, base_shift=True)
    assert top["a"] == 64 and top["b"] == 64
