"""NVFP4 number format, written from its definition (oracle; test infrastructure only).

Follows "Replay the Curvature" (arXiv 2609.36654), Abstract: every 16 E2M1
weights share one E4M3 block scale.  The element and scale types are the OCP
8-bit (E4M3, "FN" variant: no infinities, S.1111.111 is NaN, largest finite
value 448) and 4-bit (E2M1: 1 sign, 2 exponent bits with bias 1, 1 mantissa
bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) floating-point formats.

Readings taken where the pages are silent (each pinned by a CPU test):
  * a per-tensor fp32 second-level scale g multiplies every block scale:
    g = fl32(max|W| / (6 * 448)), or 1 when W is all zero;
  * rounding is to the nearest representable value of the real quotient
    |w| / (scale), ties to the even mantissa (even code index);
  * a magnitude that rounds to zero is stored as +0 (code 0x0);
  * element magnitudes above the largest E2M1 value clip to 6; block scales
    above 448 saturate to 448 (code 0x7E), never NaN;
  * storage: two 4-bit codes per byte, the even column in the low nibble;
    code = sign << 3 | magnitude index; scales are E4M3 bytes, row-major
    [rows, cols / 16].

Exactness: every decision compares a magnitude against a midpoint times a
scale.  The midpoint products used here have at most 31 significant bits
(scale g: 24 bits, E4M3 value: 4 bits, E2M1 midpoint: 3 bits), so they are
exact in fp64, and fp64 comparisons of such products with fp32 or fp64 inputs
are exact.  The decisions are therefore those of exact real arithmetic.
"""

import numpy as np

BLOCK = 16

# E2M1 magnitudes by index: exponent field e (bias 1), mantissa bit m;
# e = 0 is subnormal (m * 0.5), otherwise 2**(e-1) * (1 + m/2).
def _e2m1_magnitudes():
    out = []
    for idx in range(8):
        e, m = idx >> 1, idx & 1
        out.append(m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0))
    return np.array(out, dtype=np.float64)


E2M1_MAG = _e2m1_magnitudes()
E2M1_MAX = float(E2M1_MAG[-1])          # 6
E4M3_MAX_CODE = 0x7E                    # 448, largest finite
E4M3_MAX = 448.0


def e4m3_decode(code):
    """Value of E4M3 (FN) byte(s): sign, 4-bit exponent (bias 7), 3-bit mantissa.

    Exponent field 0 is subnormal: mantissa * 2**-9.  0x7F / 0xFF are NaN.
    """
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


# Non-negative finite E4M3 values in code order (code 0..126), strictly increasing.
E4M3_POS = e4m3_decode(np.arange(E4M3_MAX_CODE + 1))


def _round_to_grid_index(mag, grid, scale):
    """Index of the nearest value of grid*scale to mag, ties to the even index.

    mag: array of non-negative reals.  grid: increasing 1-D array.  scale:
    scalar or array broadcastable to mag.  Values beyond the last midpoint map
    to the last index (saturation).  Exact when mids*scale is exact in fp64.
    """
    mag = np.asarray(mag, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    mids = (grid[:-1] + grid[1:]) / 2.0
    below = np.zeros(np.broadcast(mag, scale).shape, dtype=np.int64)
    tie = np.zeros(below.shape, dtype=bool)
    for i, mid in enumerate(mids):
        thr = mid * scale
        below += (mag > thr)
        tie |= (mag == thr)
    # On an exact tie the tied midpoint is mids[below]; its neighbours are
    # indices below and below+1: pick the even one.
    return below + (tie & (below % 2 == 1))


def e4m3_rne(x):
    """Round non-negative reals x to the nearest E4M3 code, ties to even; saturating."""
    return _round_to_grid_index(x, E4M3_POS, 1.0)


def e4m3_rne_ratio(num, den):
    """E4M3 code nearest to the real quotient num/den (num >= 0, den > 0), ties to even.

    Decided by comparing num with midpoint*den, so no quotient is rounded.
    """
    return _round_to_grid_index(num, E4M3_POS, den)


def e2m1_encode(v, block_scale_value, g):
    """4-bit E2M1 code of v under the real scale block_scale_value * g.

    The magnitude index is the nearest E2M1 magnitude to |v| / (s * g), ties to
    even; magnitudes past 6 clip to 6.  A zero index is stored as +0.
    """
    v = np.asarray(v, dtype=np.float64)
    scale = np.asarray(block_scale_value, dtype=np.float64) * np.float64(g)
    idx = _round_to_grid_index(np.abs(v), E2M1_MAG, scale)
    sign = ((v < 0) & (idx > 0)).astype(np.int64)
    return (sign << 3) | idx


def e2m1_value(code):
    """Signed E2M1 value of 4-bit code(s)."""
    c = np.asarray(code, dtype=np.int64)
    mag = E2M1_MAG[c & 7]
    return np.where((c >> 3) & 1, -mag, mag)


def dequant_exact(code4, scale_code, g):
    """Exact real value element_value * block_scale * g (fp64 holds it exactly)."""
    return e2m1_value(code4) * e4m3_decode(scale_code) * np.float64(g)


def dequant_f32(code4, scale_code, g):
    """The dequantized weight as fp32: the exact product rounded once to fp32."""
    return dequant_exact(code4, scale_code, g).astype(np.float32)


def global_scale(W):
    """Per-tensor fp32 second-level scale: fl32(max|W| / (6*448)); 1 for an all-zero W.

    With this g the block holding the largest magnitude needs a block scale of
    at most 448, the top of the E4M3 range.
    """
    amax = float(np.max(np.abs(np.asarray(W, dtype=np.float64)))) if np.size(W) else 0.0
    if amax == 0.0:
        return np.float32(1.0)
    return np.float32(amax / (E2M1_MAX * E4M3_MAX))


def pack_codes(codes4):
    """[rows, cols] 4-bit codes -> [rows, cols/2] bytes, even column in the low nibble."""
    c = np.asarray(codes4, dtype=np.uint8)
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)


def unpack_codes(packed):
    """Inverse of pack_codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def dequantize(packed, scales, g, out_dtype=np.float32):
    """Packed codes [m, k/2] + scale bytes [m, k/16] + g -> fp32 weights [m, k]."""
    codes = unpack_codes(packed)
    sc = np.repeat(np.asarray(scales, dtype=np.uint8), BLOCK, axis=1)
    return dequant_f32(codes, sc, g).astype(out_dtype)
