"""FP4 KV-cache format — oracle (test infrastructure only).

[MTP] ¶4: the main KV cache is stored as E2M1 values with one E4M3 scale for
every 16 channels, the NVFP4 layout without its global (per-tensor) scale.
The element formats are the OCP ones:

  E2M1  1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
        {0, 0.5, 1, 1.5, 2, 3, 4, 6}; no inf/NaN.
  E4M3  (FN variant) 1 sign, 4 exponent (bias 7), 3 mantissa bits; subnormals
        m * 2^-9; exponent 15 with mantissa 7 is NaN; largest finite 448.

Readings where the pages are silent (each listed in the design notes):
  * the block scale is the E4M3 value nearest to amax/6 (ties to even code),
    saturating at 448 -- the plain reading of the NVFP4 layout the page names;
  * an element is the E2M1 value nearest to x/scale (ties to even code),
    clamped at 6, with the sign bit copied from x (so a small negative value
    encodes as 0x8, "negative zero");
  * a block whose scale encodes to zero gets magnitude code 0 throughout;
  * byte j of a packed row holds channel 2j in its low nibble and channel 2j+1
    in its high nibble; scale byte b covers channels [16b, 16b+16).
"""
import numpy as np

BLOCK = 16                     # channels per E4M3 scale ([MTP] ¶4)
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # [OCP] E2M1 magnitudes
E4M3_MAX = 448.0


def e2m1_decode(codes) -> np.ndarray:
    """float64 value of each 4-bit E2M1 code (low 4 bits of each entry)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    mag = E2M1_MAG[c & 7]
    return np.where(c & 8, -mag, mag)


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each E4M3FN byte; NaN for 0x7F / 0xFF."""
    b = np.asarray(codes).astype(np.int64) & 0xFF
    s = b >> 7
    e = (b >> 3) & 0xF
    m = b & 7
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0 ** -9
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return np.where(s == 1, -v, v)


# The 127 finite non-negative E4M3 values, indexed by code 0..126 (increasing).
_E4M3_POS = e4m3_decode(np.arange(127))


def e4m3_encode(x) -> np.ndarray:
    """Round float64 values to E4M3FN codes: nearest, ties to the even code,
    finite values beyond 448 saturate to 448 (0x7E), NaN -> 0x7F.  The sign bit
    is copied from x (so -0.0 and tiny negatives give 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    # index of the first representable value >= |x|
    hi = np.searchsorted(_E4M3_POS, np.minimum(ax, E4M3_MAX), side="left")
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    v_hi = _E4M3_POS[hi]
    v_lo = _E4M3_POS[lo]
    d_hi = v_hi - ax
    d_lo = ax - v_lo
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(ax >= v_hi, hi, np.where(pick_hi, hi, lo))
    code = np.where(ax >= E4M3_MAX, 126, code)
    sign = np.signbit(x).astype(np.int64) << 7
    out = (code | sign).astype(np.int64)
    out = np.where(np.isnan(x), 0x7F, out)
    return out.astype(np.uint8)


# E2M1 rounding midpoints between consecutive magnitudes, and whether a value
# exactly at the midpoint rounds up (the upper neighbour has the even code).
_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
_TIE_UP = np.array([False, True, False, True, False, True, False])


def block_scales(x: np.ndarray) -> np.ndarray:
    """E4M3 scale codes, one per 16-channel block: RNE(amax / 6), saturating.

    x: float64 [..., C] holding bf16 values exactly.  amax/6 is formed in
    float64; a tie of the E4M3 grid has at most 5 significant bits, so a bf16
    amax divided by 6 either equals a tie exactly (and float64 holds it) or
    lies at least 2^-16 (relative) away from every tie -- float64 rounding
    cannot change the decision.
    """
    C = x.shape[-1]
    assert C % BLOCK == 0
    blocks = np.abs(x).reshape(x.shape[:-1] + (C // BLOCK, BLOCK))
    amax = blocks.max(axis=-1)
    return e4m3_encode(amax / 6.0)


def e2m1_encode_scaled(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """E2M1 code of x / s for every element: nearest, ties to even, clamp at 6.

    The comparison |x| vs midpoint * s is exact in float64 (x is bf16, s is
    E4M3, the midpoints have <= 3 significant bits).  s == 0 gives magnitude 0.
    """
    ax = np.abs(x)
    mag = np.zeros(x.shape, dtype=np.int64)
    for mid, up in zip(_MID, _TIE_UP):
        t = mid * s
        mag += (ax >= t) if up else (ax > t)
    mag = np.where(s == 0, 0, mag)
    sign = np.signbit(x).astype(np.int64) << 3
    return (mag | sign).astype(np.uint8)


def fp4_pack(x: np.ndarray):
    """Quantise rows of latent KV to the FP4 cache layout.

    x: float64 [N, C] (bf16 values).  Returns (codes uint8 [N, C/2],
    scales uint8 [N, C/16]).
    """
    x = np.asarray(x, dtype=np.float64)
    N, C = x.shape
    sc = block_scales(x)                                   # [N, C/16]
    s = np.repeat(e4m3_decode(sc), BLOCK, axis=-1)         # [N, C]
    nib = e2m1_encode_scaled(x, s).astype(np.uint8)        # [N, C]
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return codes, sc


def fp4_unpack(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 [N, C] dequantised rows: E2M1(code) * E4M3(scale) (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, half = codes.shape
    nib = np.empty((N, 2 * half), dtype=np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    s = np.repeat(e4m3_decode(scales), BLOCK, axis=-1)
    return e2m1_decode(nib) * s


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest bf16 value (ties to even), returned as uint16 bits.
    Values are first rounded to float32 (exact for anything already bf16)."""
    f = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (f >> 16) & 1
    r = ((f + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
