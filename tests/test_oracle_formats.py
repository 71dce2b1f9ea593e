"""Pins for the oracle's FP4 KV format (E2M1 elements, E4M3 scale per 16 channels).

The format is named in the KV-cache paragraph of the MarkTechPost retelling
(E2M1 with one E4M3 scale per 16 channels, NVFP4 without the global scale).
Pins: the OCP code tables, torch's own float8_e4m3fn cast, an exact-rational
brute-force nearest-value search, hand-derived blocks, round-trip and
idempotence, the rounding error bound and the storage ratio the page quotes.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


def _read_table(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            rows.append((int(a, 0), float(b)))
    return rows


def test_e2m1_table_matches_golden(golden_dir):
    for code, val in _read_table(os.path.join(golden_dir, "e2m1_codes.txt")):
        got = F.e2m1_decode(np.array([code]))[0]
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)


def test_e2m1_code_set_is_the_nvfp4_grid():
    vals = set(np.abs(F.e2m1_decode(np.arange(16))).tolist())
    assert vals == {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}


def test_e4m3_decode_exhaustive_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e4m3_special_values_golden(golden_dir):
    for code, val in _read_table(os.path.join(golden_dir, "e4m3_special.txt")):
        got = F.e4m3_decode(np.array([code]))[0]
        if np.isnan(val):
            assert np.isnan(got)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), (hex(code), got, val)


def _e4m3_ties():
    pos = F.e4m3_decode(np.arange(127))
    mids = (pos[:-1] + pos[1:]) / 2.0
    return np.concatenate([mids, -mids])


def test_e4m3_encode_vs_torch_in_range():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(20000) * np.exp2(rng.integers(-12, 8, 20000)),
        _e4m3_ties(),                                  # exact ties -> even code
        F.e4m3_decode(np.arange(256))[~np.isnan(F.e4m3_decode(np.arange(256)))],
        rng.uniform(-448, 448, 5000),
    ])
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(x)
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates_and_nan():
    # torch's cast does not saturate (values >= 464 become NaN); the oracle's
    # reading is satfinite: every finite value above 448 encodes as +-448.
    got = F.e4m3_encode(np.array([449.0, 463.9, 464.0, 1e6, -500.0, np.nan]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F]


def _brute_e4m3(q: Fraction) -> int:
    """Nearest non-negative finite E4M3 code to q (exact rationals), ties to even code."""
    best, best_d = None, None
    for c in range(127):
        v = Fraction(float(F.e4m3_decode(np.array([c]))[0]))
        d = abs(v - q)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best


def _brute_e2m1(ax: Fraction, s: Fraction) -> int:
    """Nearest E2M1 magnitude index to ax/s (exact), ties to the even index; s=0 -> 0."""
    if s == 0:
        return 0
    r = ax / s
    best, best_d = None, None
    for i, m in enumerate([0, Fraction(1, 2), 1, Fraction(3, 2), 2, 3, 4, 6]):
        d = abs(Fraction(m) - r)
        if best is None or d < best_d or (d == best_d and i % 2 == 0):
            best, best_d = i, d
    return best


def _bf16_values(rng, shape, scale=1.0):
    x = torch.from_numpy(rng.standard_normal(shape) * scale).to(torch.bfloat16)
    return x.to(torch.float64).numpy()


def test_pack_matches_exact_rational_brute_force():
    rng = np.random.default_rng(5)
    blocks = []
    blocks.append(_bf16_values(rng, (150, 16)))
    blocks.append(_bf16_values(rng, (40, 16), scale=1e-3))   # subnormal scales
    blocks.append(_bf16_values(rng, (20, 16), scale=300.0))  # saturating scales
    # blocks made of exact E2M1-grid ties times a representable scale
    s = F.e4m3_decode(rng.integers(8, 120, 30))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    e = rng.choice(mids, (30, 16)) * rng.choice([-1, 1], (30, 16))
    e[:, 0] = 6.0
    blocks.append(e * s[:, None])
    x = np.concatenate(blocks, axis=0)
    # ensure every value is a bf16 value
    x = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    codes, scales = F.fp4_pack(x)
    for r in range(x.shape[0]):
        amax = max(abs(Fraction(float(v))) for v in x[r])
        sc = _brute_e4m3(min(amax / 6, Fraction(448)))
        assert scales[r, 0] == sc, (r, scales[r, 0], sc)
        sv = Fraction(float(F.e4m3_decode(np.array([sc]))[0]))
        for c in range(16):
            mag = _brute_e2m1(abs(Fraction(float(x[r, c]))), sv)
            sign = 8 if np.signbit(x[r, c]) else 0
            nib = (codes[r, c // 2] >> (4 * (c % 2))) & 0xF
            assert nib == (mag | sign), (r, c, x[r, c], nib, mag | sign)


def test_amax_over_six_float64_decides_like_exact_rationals():
    rng = np.random.default_rng(9)
    amax = np.abs(_bf16_values(rng, 3000, scale=4.0))
    amax = np.concatenate([amax, 6 * F.e4m3_decode(np.arange(1, 127)), 3 * F.e4m3_decode(np.arange(1, 127))])
    amax = torch.from_numpy(amax).to(torch.bfloat16).to(torch.float64).numpy()
    got = F.e4m3_encode(amax / 6.0)
    for a, g in zip(amax[::7], got[::7]):
        assert g == _brute_e4m3(min(Fraction(float(a)) / 6, Fraction(448)))


def test_hand_derived_blocks():
    # Block 1: amax 6 -> scale RNE(1.0) = 0x38; values on the grid encode exactly.
    x = np.zeros((1, 16))
    x[0, :5] = [6.0, -3.0, 1.5, 0.5, -0.0]
    codes, sc = F.fp4_pack(x)
    assert sc[0, 0] == 0x38
    nib = [(codes[0, c // 2] >> (4 * (c % 2))) & 0xF for c in range(16)]
    assert nib[:5] == [0x7, 0xD, 0x3, 0x1, 0x8]
    assert nib[5:] == [0] * 11
    # Block 2: amax 12 -> scale 2.0 (0x40); every other value sits on an E2M1 tie.
    x = np.array([[12.0, 2.5, 3.5, 5.0, 7.0, 10.0, 0.5, 1.5, -0.25, -4.5, 0, 0, 0, 0, 0, 0]])
    codes, sc = F.fp4_pack(x)
    assert sc[0, 0] == 0x40
    nib = [(codes[0, c // 2] >> (4 * (c % 2))) & 0xF for c in range(16)]
    # 12/2=6 ->7; 1.25->1.0 (2); 1.75->2.0 (4); 2.5->2.0 (4); 3.5->4.0 (6); 5->4.0 (6);
    # 0.25->0 (0); 0.75->1.0 (2); -0.125->-0 (8); -2.25 -> -2.0 (0xC)
    assert nib[:10] == [7, 2, 4, 4, 6, 6, 0, 2, 8, 0xC]
    # Block 3: amax 4096 -> 4096/6 saturates to 448 (0x7E); 4096/448 > 6 clamps to 6.
    x = np.zeros((1, 16)); x[0, 0] = 4096.0; x[0, 1] = -2688.0
    codes, sc = F.fp4_pack(x)
    assert sc[0, 0] == 0x7E
    assert codes[0, 0] == (0x7 | (0xF << 4))
    # Block 4: amax/6 = 2^-10 is the tie between 0 and 2^-9: even code 0 -> scale 0,
    # so every magnitude code is 0 and only the signs survive.
    x = np.zeros((1, 16)); x[0, 0] = 6 * 2.0 ** -10; x[0, 1] = -3 * 2.0 ** -10
    codes, sc = F.fp4_pack(x)
    assert sc[0, 0] == 0
    assert codes[0, 0] == (0x0 | (0x8 << 4))
    # Block 5: amax/6 just above the tie rounds up to the smallest subnormal 2^-9.
    x = np.zeros((1, 16)); x[0, 0] = 6 * 2.0 ** -10 * (1 + 2.0 ** -7)
    codes, sc = F.fp4_pack(x)
    assert sc[0, 0] == 0x01


def test_representable_blocks_round_trip_bit_exactly():
    rng = np.random.default_rng(3)
    n = 500
    s_codes = rng.integers(1, 127, n).astype(np.uint8)       # any positive finite scale
    s = F.e4m3_decode(s_codes)
    e_codes = rng.integers(0, 16, (n, 16)).astype(np.uint8)
    for i in range(n):
        e_codes[i, rng.integers(0, 16)] = rng.choice([0x7, 0xF])   # |e| = 6 in each block
    x = F.e2m1_decode(e_codes) * s[:, None]
    codes, scales = F.fp4_pack(x)
    assert np.array_equal(scales[:, 0], s_codes)
    want = (e_codes[:, 0::2] | (e_codes[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(codes, want)
    back = F.fp4_unpack(codes, scales)
    assert np.array_equal(back, x)
    assert np.array_equal(np.signbit(back), np.signbit(x))


def test_idempotence_and_error_bound():
    rng = np.random.default_rng(4)
    x = _bf16_values(rng, (400, 512))
    x[:, [3, 77, 200]] *= 8
    x = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    codes, scales = F.fp4_pack(x)
    xh = F.fp4_unpack(codes, scales)
    c2, s2 = F.fp4_pack(xh)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    s = np.repeat(F.e4m3_decode(scales), 16, axis=1)
    r = np.abs(x) / s
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    gap = np.select([r < 2, r < 4], [0.5, 1.0], 2.0)
    bound = np.where(r > 6, np.abs(x) - 6 * s, 0.5 * gap * s)
    assert np.all(np.abs(x - xh) <= bound + 0.0)
    assert set(np.unique(np.abs(xh) / s)).issubset(set(grid.tolist()))


def test_storage_ratio_nearly_halves_fp8():
    # One FP8 byte per channel versus 4 bits per channel plus one byte per 16 channels.
    x = np.zeros((2, 512))
    codes, scales = F.fp4_pack(x)
    ratio = (codes.shape[1] + scales.shape[1]) / 512
    assert ratio == 0.5625 and 0.5 < ratio < 0.6


def test_all_zero_and_negative_zero_blocks():
    x = np.zeros((1, 32)); x[0, 16:] = -0.0
    codes, scales = F.fp4_pack(x)
    assert scales.tolist() == [[0, 0]]
    assert codes[0, :8].tolist() == [0] * 8 and codes[0, 8:].tolist() == [0x88] * 8
    back = F.fp4_unpack(codes, scales)
    assert np.all(back == 0) and np.all(np.signbit(back[0, 16:]))


def test_nibble_order_low_is_even_channel():
    x = np.zeros((1, 16)); x[0, 0] = 6.0; x[0, 1] = 1.0
    codes, _ = F.fp4_pack(x)
    assert codes[0, 0] == (0x7 | (0x2 << 4))


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(10000) * np.exp2(rng.integers(-20, 20, 10000))
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_round(x.astype(np.float32)), ref)
    assert np.array_equal(F.bf16_to_float(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy())


def test_non_finite_blocks():
    # Reading for non-finite latent values: E4M3 has no infinity, and the scale
    # rule already saturates finite values above 448, so an infinity behaves as
    # the largest finite value (same scale and codes as a huge finite entry);
    # a NaN makes the block's amax NaN, which encodes as the E4M3 NaN 0x7F, so
    # the whole block decodes to NaN while the row's other blocks are untouched.
    x = np.zeros((1, 48))
    x[0, 1], x[0, 2], x[0, 3] = 1.0, -3.0, 1500.0
    x[0, 16 + 1], x[0, 16 + 2] = 1.0, -3.0
    x[0, 32 + 5] = 0.75
    inf_row = x.copy(); inf_row[0, 3] = np.inf; inf_row[0, 4] = -np.inf
    big_row = x.copy(); big_row[0, 3] = 1e30; big_row[0, 4] = -1e30
    ci, si = F.fp4_pack(inf_row)
    cb, sb = F.fp4_pack(big_row)
    assert np.array_equal(ci, cb) and np.array_equal(si, sb)
    assert si[0, 0] == 0x7E                                 # 448: saturated
    assert (ci[0, 1] >> 4) == 0x7 and (ci[0, 2] & 0xF) == 0xF  # +6 / -6
    back = F.fp4_unpack(ci, si)
    assert back[0, 3] == 2688.0 and back[0, 4] == -2688.0
    nan_row = x.copy(); nan_row[0, 16] = np.nan
    cn, sn = F.fp4_pack(nan_row)
    assert sn[0, 1] == 0x7F
    assert np.all(cn[0, 8:16] & 0x77 == 0)                  # every magnitude code 0
    assert (cn[0, 9] & 0xF) == 0x8                           # the sign of -3 is kept
    back = F.fp4_unpack(cn, sn)
    assert np.all(np.isnan(back[0, 16:32]))
    ref_c, ref_s = F.fp4_pack(x)
    keep = np.r_[0:8, 16:24]
    assert np.array_equal(cn[0, keep], ref_c[0, keep]) and sn[0, 0] == ref_s[0, 0] and sn[0, 2] == ref_s[0, 2]
    assert np.array_equal(back[0, np.r_[0:16, 32:48]], F.fp4_unpack(ref_c, ref_s)[0, np.r_[0:16, 32:48]])
