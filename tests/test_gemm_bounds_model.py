"""Host-side model of the W4A4 GEMM's global -> LDS loads: where the hardware may fetch.

The kernel loads 16 bytes per lane through raw buffer resources over each tile's rows.  The
range check of a raw resource covers the VGPR offset only (row and 16-byte chunk here); the
SGPR offset (the K column) is added to the address after it.  The model mirrors the
kernel's offset arithmetic (tile rows, the K walk's starting buffer, the XOR chunk swizzle,
the scale groups, every issue including those past the end of K with their out-of-range
sentinel), assumes the check admits a dword when VGPR offset + 4 <= num_records, and
compares the admitted dwords' addresses with the operand's size.

* The scale loads carry their column in the VGPR offset, so the range check covers it: a
  half last scale group (K % 512 != 0) reads zeros past the operand's last row.
* K % 256 == 0: every code buffer ends by column K / 2, so nothing leaves the operand.
* K % 256 == 128 (a half last buffer): the last buffer's chunks past a row's end are
  admitted and read the next row, and at the operand's last row up to 64 code bytes past
  its end.  Those bytes only feed products whose scales are zeroed, but they must be
  mapped: this is an open bound, not a guarantee.
* The planned fix moves the column offset into the resource base and out of num_records,
  saturating at zero; the model checks it keeps every fetch inside, and that a count
  which wraps round instead admits the sentinel offset (2 GiB past the operand).
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


def _fetched_max(M, N, K, tail, wrap=False, scale_col_in_voff=True):
    """Largest byte offset + 1 fetched from each operand (A codes, B codes, A scales,
    B scales) over every tile and issued load, or -1 if none.  `wrap` models a resource
    count that wraps round instead of saturating when the column exceeds it;
    `scale_col_in_voff` the scale loads' column in the VGPR offset (as built)."""
    rowbytes, rowscales = K // 2, K // 32
    np_ = (K + BKP - 1) // BKP
    tiles_m, tiles_n = (M + BM - 1) // BM, (N + BN - 1) // BN
    codes_off, scale_off = _lane_offsets(rowbytes, rowscales)
    code_issues, scale_issues = _issues(np_)
    top = {"a": -1, "b": -1, "sa": -1, "sb": -1}

    def admit(key, base, nrec, col, voff, valid, col_in_voff=False):
        if col_in_voff:
            voff = (np.asarray(voff, dtype=np.int64) if valid else np.full(64, KOOB, dtype=np.int64)) + col
            for d in range(4):
                ok = voff + 4 * d + 4 <= nrec
                if ok.any():
                    top[key] = max(top[key], int(base + voff[ok].max() + 4 * d + 4))
            return
        if tail:
            base, soff = base + col, 0
            nrec = (nrec - col) % (1 << 32) if wrap else max(nrec - col, 0)
        else:
            soff = col
        voff = np.asarray(voff, dtype=np.int64) if valid else np.full(64, KOOB, dtype=np.int64)
        for d in range(4):                      # the four dwords of a 16-byte load
            ok = voff + 4 * d + 4 <= nrec
            if ok.any():
                top[key] = max(top[key], int(base + soff + voff[ok].max() + 4 * d + 4))

    for tm in range(tiles_m):
        for tn in range(tiles_n):
            m0, n0 = tm * BM, tn * BN
            rows_a, rows_b = min(BM, M - m0), min(BN, N - n0)
            rot = (2 * tm) % np_ if K % (2 * BKP) == 0 else 0

            def rotated(q):
                q += rot
                return q - np_ if q >= np_ else q

            for q, valid in code_issues:
                col = rotated(q) * ROWB
                for key, r0, rows in (("a", m0, rows_a), ("b", n0, rows_b)):
                    for wave in range(NW):
                        for i in range(QW):
                            admit(key, r0 * rowbytes, rows * rowbytes, col, codes_off[wave][i], valid)
            for h, valid in scale_issues:
                col = (rotated(2 * h) >> 1) * KSCALE_ROW
                for wave in range(NW):
                    for i in range(SW):
                        t = SW * wave + i
                        key, r0, rows = ("sb", n0, rows_b) if t >> 2 else ("sa", m0, rows_a)
                        admit(key, r0 * rowscales, rows * rowscales, col, scale_off[wave][i], valid,
                              col_in_voff=scale_col_in_voff and not tail)
    return top


def _sizes(M, N, K):
    return {"a": M * K // 2, "b": N * K // 2, "sa": M * K // 32, "sb": N * K // 32}


# the GPU test shapes, plus the W4A4 configuration's K with small M, N
SHAPES = [(1, 1, 128), (64, 96, 256), (300, 260, 384), (256, 512, 1024), (1100, 1300, 1536), (777, 392, 512),
          (513, 257, 8192), (130, 70, 640), (200, 300, 1408), (300, 600, 8192)]


@pytest.mark.parametrize("M,N,K", SHAPES + [(256, 256, 4352), (300, 260, 4352)])
def test_fetches_of_the_kernel_as_built(M, N, K):
    """The kernel as built: code loads with the column in the SGPR offset, scale loads with
    it in the VGPR offset."""
    top = _fetched_max(M, N, K, tail=False)
    size = _sizes(M, N, K)
    assert top["a"] >= size["a"] and top["b"] >= size["b"]   # the last row is read whole
    assert top["sa"] <= size["sa"] and top["sb"] <= size["sb"], (top, size)
    if K % BKP == 0:
        assert top["a"] <= size["a"] and top["b"] <= size["b"], (top, size)
    else:
        over = {k: top[k] - size[k] for k in ("a", "b")}
        assert max(over.values()) <= 64, over


def test_scale_column_in_the_sgpr_offset_would_read_past():
    """With the column in the SGPR offset (the earlier form), a half last scale group reads
    8 bytes past the last row's scales at K = 4352 and 12 at K = 640."""
    for K, want in ((4352, 8), (640, 12)):
        top = _fetched_max(256, 256, K, tail=False, scale_col_in_voff=False)
        assert top["sa"] - _sizes(256, 256, K)["sa"] == want


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_planned_fix_keeps_every_fetch_inside(M, N, K):
    top = _fetched_max(M, N, K, tail=K % (2 * BKP) != 0)
    size = _sizes(M, N, K)
    for key in top:
        assert top[key] <= size[key], (key, top[key], size[key])


def test_a_wrapping_resource_count_would_admit_the_sentinel():
    """M = N = 1, K = 128: past the end, rotated() wraps step 0's refill (q = 2) to buffer
    1, whose column (128) exceeds the operand's 64 bytes.  A count that wraps round to
    4 GiB admits the out-of-range offset and fetches 2 GiB past the operand; the
    saturating count admits nothing beyond it."""
    top = _fetched_max(1, 1, 128, tail=True, wrap=True)
    assert top["a"] > (1 << 31)
    top = _fetched_max(1, 1, 128, tail=True)
    assert top["a"] == 64 and top["b"] == 64


def test_ragged_k_overrun_of_the_kernel_as_built():
    """K = 384 (a half last buffer): the last row's second half-buffer of codes is admitted
    by the VGPR check and fetched past the end of the operand; the planned fix does not."""
    M, N, K = 300, 260, 384
    top = _fetched_max(M, N, K, tail=False)
    size = _sizes(M, N, K)
    assert top["a"] > size["a"] and top["b"] > size["b"]
    assert _fetched_max(M, N, K, tail=True)["a"] <= size["a"]
