"""Element and scale formats of micro-scaled FP4, written out from their definitions.

TEST INFRASTRUCTURE: part of the CPU oracle. Only tests, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never does.

Sources
-------
* E2M1 elements ("mantisse E2M1"): ARCQuant summary (gist.science, Méthodologie,
  item 1) and the MR-GPTQ abstract (hyper.ai, Résumé) name 4-bit E2M1 elements for
  NVFP4 and MXFP4.  The pages give no bit layout; the layout used here is the OCP
  Microscaling (MX) v1.0 one: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa,
  magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* E4M3 block scales for NVFP4 (block 16: ARCQuant summary, Énoncé du Problème, second
  bullet).  Layout from OCP FP8 E4M3 ("FN" variant): bias 7, 3 mantissa bits,
  subnormal step 2^-9, largest finite 448, 0x7F/0xFF are NaN (never produced here).
* E8M0 power-of-two scales for MXFP4 ("quantification à échelle à puissance de deux",
  MR-GPTQ abstract, Résumé).  Layout from OCP MX v1.0: 8-bit biased exponent, bias 127,
  value 2^(code-127), 0xFF is NaN (never produced here).

Rounding is round-to-nearest with ties to the even code for E2M1 and E4M3, saturating
at the largest finite magnitude (6 and 448); the pages do not fix a rounding rule.
"""
import numpy as np

# ---------------------------------------------------------------------------
# E2M1
# ---------------------------------------------------------------------------
#: magnitude of the 3-bit code 0..7 (code bit 3 is the sign)
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0


def _e2m1_magnitude_from_bits(code3):
    """Magnitude of a 3-bit E2M1 code from its exponent/mantissa fields (bias 1)."""
    e = (code3 >> 1) & 3
    m = code3 & 1
    if e == 0:                       # subnormal: m * 2^(1-1) * 0.5
        return m * 0.5
    return (1.0 + 0.5 * m) * 2.0 ** (e - 1)


def e2m1_decode(codes):
    """Signed real value of 4-bit E2M1 codes (uint8 array with values 0..15)."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[codes & 7]
    return np.where(codes & 8, -mag, mag)


def _nearest_code_ties_even(a, grid):
    """Index of the grid value nearest to each a >= 0, ties to the even index.

    `grid` is sorted ascending.  Values above the last grid point map to the last
    index (saturation).  The midpoints are formed from the grid itself; every
    comparison is exact because grid values and their midpoints are short binary
    fractions and `a` is an fp64 value.
    """
    a = np.asarray(a, dtype=np.float64)
    mids = (grid[:-1] + grid[1:]) / 2.0
    idx = np.searchsorted(mids, a, side="left")          # number of midpoints < a
    on_mid = np.zeros(a.shape, dtype=bool)
    inside = idx < len(mids)
    on_mid[inside] = a[inside] == mids[idx[inside]]
    idx = idx + (on_mid & (idx % 2 == 1))               # tie: step to the even code
    return idx.astype(np.uint8)


def e2m1_rne(u):
    """E2M1 code of real values u: nearest magnitude, ties to even, saturating at 6.

    The sign bit is the IEEE sign of u, so negative values (and -0.0) that round to
    magnitude 0 keep code 8.  u must be finite.
    """
    u = np.asarray(u, dtype=np.float64)
    mag = _nearest_code_ties_even(np.abs(u), E2M1_MAGNITUDES)
    return (mag | (np.signbit(u).astype(np.uint8) << 3)).astype(np.uint8)


def e2m1_boundary_distance(u):
    """Relative distance of |u| to the nearest E2M1 rounding boundary.

    The boundaries of the magnitude decision are the midpoints of the grid (above 6
    everything saturates, so there is no boundary there).  Used by the tests to accept
    a differing code only where an fp32 evaluation may legitimately fall on the other
    side; returns |a - m| / max(m, tiny) for the nearest midpoint m.
    """
    a = np.abs(np.asarray(u, dtype=np.float64))
    mids = (E2M1_MAGNITUDES[:-1] + E2M1_MAGNITUDES[1:]) / 2.0
    d = np.abs(a[..., None] - mids) / mids
    return d.min(axis=-1)


def pack_nibbles(codes):
    """Two 4-bit codes per byte along the last axis: element 2j in bits 0-3, 2j+1 in bits 4-7."""
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape[-1] % 2 == 0
    return (codes[..., 0::2] & 15) | ((codes[..., 1::2] & 15) << 4)


def unpack_nibbles(packed):
    """Inverse of pack_nibbles."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 15
    out[..., 1::2] = packed >> 4
    return out


# ---------------------------------------------------------------------------
# E4M3 (OCP FP8, "FN": no infinities, NaN = S.1111.111)
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0


def _e4m3_value_from_bits(b):
    e = (b >> 3) & 15
    m = b & 7
    if e == 15 and m == 7:
        return np.nan
    if e == 0:
        return m * 2.0 ** -9                  # subnormal: (m/8) * 2^(1-7)
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_TABLE = np.array([_e4m3_value_from_bits(b) for b in range(128)])
#: finite non-negative E4M3 values, index = code 0..126, strictly increasing
E4M3_FINITE = _E4M3_TABLE[:127].copy()


def e4m3_decode(bits):
    """Real value of E4M3 bit patterns (uint8); 0x7F / 0xFF decode to NaN."""
    bits = np.asarray(bits, dtype=np.uint8)
    mag = _E4M3_TABLE[bits & 127]
    return np.where(bits & 128, -mag, mag)


def e4m3_rne(r):
    """E4M3 code of real r >= 0: nearest finite value, ties to even, saturating at 448."""
    r = np.asarray(r, dtype=np.float64)
    assert np.all(r >= 0), "scale arguments are non-negative"
    return _nearest_code_ties_even(r, E4M3_FINITE)


def e4m3_boundary_distance(r):
    """Relative distance of r to the nearest E4M3 rounding midpoint (for tolerance checks)."""
    r = np.asarray(r, dtype=np.float64)
    mids = (E4M3_FINITE[:-1] + E4M3_FINITE[1:]) / 2.0
    idx = np.clip(np.searchsorted(mids, r), 1, len(mids) - 1)
    d = np.minimum(np.abs(r - mids[idx - 1]) / mids[idx - 1], np.abs(r - mids[idx]) / mids[idx])
    return np.where(r > E4M3_MAX, np.inf, d)


# ---------------------------------------------------------------------------
# E8M0 (power-of-two scale)
# ---------------------------------------------------------------------------
E8M0_BIAS = 127
#: largest power of two in the E2M1 grid: 6 = 1.5 * 2^2, so emax = 2
E2M1_EMAX = 2


def e8m0_decode(code):
    """2^(code - 127) as fp64; 0xFF is the format's NaN (OCP MX v1.0), never produced by
    e8m0_from_amax, only met when decoding foreign scale bytes."""
    code = np.asarray(code, dtype=np.int64)
    return np.where(code == 255, np.nan, np.ldexp(1.0, code - E8M0_BIAS))


def e8m0_from_amax(amax):
    """Shared MX scale of a block with absolute maximum `amax` (OCP MX v1.0 rule).

    X = 2^(floor(log2 amax) - emax_elem) with emax_elem = 2 for E2M1, clamped to the
    representable exponents [-127, 127].  An all-zero block (amax = 0) gets code 0.
    floor(log2 a) is read exactly from frexp: a = f * 2^E with f in [0.5, 1).
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, E = np.frexp(amax)
    e = (E.astype(np.int64) - 1) - E2M1_EMAX
    e = np.clip(e, -E8M0_BIAS, E8M0_BIAS)
    code = np.where(amax > 0, e + E8M0_BIAS, 0)
    return code.astype(np.uint8)


# ---------------------------------------------------------------------------
# storage types of the surrounding tensors
# ---------------------------------------------------------------------------

def to_f32(v):
    """Round to IEEE binary32, nearest-even (numpy's conversion)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(v32):
    """bfloat16 bit pattern of fp32 values, round-to-nearest-even (finite inputs)."""
    b = np.asarray(v32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits):
    """Exact value of bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
