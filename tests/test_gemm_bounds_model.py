"""Host-side model of the W4A4 GEMM's global -> LDS loads: every byte the hardware may
fetch lies inside its operand.

The kernel loads 16 bytes per lane through raw buffer resources.  The range check of a
raw resource covers the VGPR offset only; an SGPR offset is added to the address after
it.  The model mirrors the kernel's offset arithmetic (tile rows, the K walk's starting
buffer, the XOR chunk swizzle, the scale groups), assumes the check admits a dword when
VGPR offset + 4 (dword end) <= num_records, and checks the admitted dwords' addresses
against the operand's size:

* K % 512 == 0: the K-column offset rides in the SGPR offset; every code buffer ends by
  column K / 2 and every scale group by K / 32, so nothing leaves its row.
* otherwise (a half last buffer, or a half last scale group): the column offset moves into
  the resource base and out of num_records, so the check covers it.

The same model with the first scheme on a ragged K shows the overrun the second prevents.
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


def _fetched_max(M, N, K, tail):
    """Largest byte offset + 1 fetched from each operand (A codes, B codes, A scales,
    B scales) over every tile and load, or -1 if none."""
    rowbytes, rowscales = K // 2, K // 32
    np_ = (K + BKP - 1) // BKP
    tiles_m, tiles_n = (M + BM - 1) // BM, (N + BN - 1) // BN
    codes_off, scale_off = _lane_offsets(rowbytes, rowscales)
    top = {"a": -1, "b": -1, "sa": -1, "sb": -1}

    def admit(key, base, nrec, voff, soff):
        voff = np.asarray(voff, dtype=np.int64)
        for d in range(4):                      # the four dwords of a 16-byte load
            ok = voff + 4 * d + 4 <= nrec
            if ok.any():
                top[key] = max(top[key], int(base + soff + voff[ok].max() + 4 * d + 4))

    for tm in range(tiles_m):
        for tn in range(tiles_n):
            m0, n0 = tm * BM, tn * BN
            rows_a, rows_b = min(BM, M - m0), min(BN, N - n0)
            rot = (2 * tm) % np_ if K % (2 * BKP) == 0 else 0
            for p in range(np_):
                col = ((p + rot) % np_) * ROWB
                for key, r0, rows in (("a", m0, rows_a), ("b", n0, rows_b)):
                    base, nrec = r0 * rowbytes, rows * rowbytes
                    if tail:
                        base, nrec, soff = base + col, nrec - col, 0
                    else:
                        soff = col
                    for wave in range(NW):
                        for q in range(QW):
                            admit(key, base, nrec, codes_off[wave][q], soff)
            for h in range((np_ + 1) // 2):
                col = (((2 * h + rot) % np_) >> 1) * KSCALE_ROW
                for wave in range(NW):
                    for q in range(SW):
                        t = SW * wave + q
                        key, r0, rows = ("sb", n0, rows_b) if t >> 2 else ("sa", m0, rows_a)
                        base, nrec = r0 * rowscales, rows * rowscales
                        if tail:
                            base, nrec, soff = base + col, nrec - col, 0
                        else:
                            soff = col
                        admit(key, base, nrec, scale_off[wave][q], soff)
    return top


def _sizes(M, N, K):
    return {"a": M * K // 2, "b": N * K // 2, "sa": M * K // 32, "sb": N * K // 32}


# the GPU test shapes, plus the W4A4 configuration's K with small M, N
SHAPES = [(1, 1, 128), (64, 96, 256), (300, 260, 384), (256, 512, 1024), (1100, 1300, 1536), (777, 392, 512),
          (513, 257, 8192), (130, 70, 640), (200, 300, 1408), (300, 600, 8192)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_every_fetched_byte_is_inside_its_operand(M, N, K):
    tail = K % (2 * BKP) != 0                   # the launcher's choice of path
    top = _fetched_max(M, N, K, tail)
    size = _sizes(M, N, K)
    for key in top:
        assert top[key] <= size[key], (key, top[key], size[key])
    assert top["a"] == size["a"] and top["b"] == size["b"]   # and the last row is read whole


def test_sgpr_column_offset_would_overrun_on_a_ragged_k():
    """The first scheme on K = 384 (a half last buffer): the last row's second half-buffer
    is admitted by the VGPR check and fetched past the end of the operand."""
    M, N, K = 300, 260, 384
    top = _fetched_max(M, N, K, tail=False)
    size = _sizes(M, N, K)
    assert top["a"] > size["a"] and top["b"] > size["b"]
    assert _fetched_max(M, N, K, tail=True)["a"] <= size["a"]
