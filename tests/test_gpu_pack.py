"""GPU parity: FP4 pack / unpack (csa2_fp4_pack, csa2_fp4_unpack) vs the oracle, bit-exact."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as OF
import fp4_sparse_attention_amd as F
from gpu_common import device, np_u8, bf16_to_f64

pytestmark = pytest.mark.gpu


def _gpu_pack(x):
    n, C = x.shape
    codes = torch.empty((n, C // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((n, C // 16), dtype=torch.uint8, device=x.device)
    F.csa2_fp4_pack(x, codes, scales)
    return codes, scales


def _special_rows():
    """bf16 rows with E2M1 ties, zero / negative-zero blocks, saturation and subnormal scales."""
    rng = np.random.default_rng(0)
    rows = []
    s = OF.e4m3_decode(rng.integers(1, 127, 64))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.0, 0.5, 1.0])
    for i in range(64):
        e = rng.choice(mids, 512) * rng.choice([-1.0, 1.0], 512)
        e[::16] = 6.0
        rows.append(e * s[i])
    z = np.zeros(512); z[16:32] = -0.0; z[40] = 6 * 2.0 ** -10; z[64] = 4096.0; z[65] = -1e30
    z[80] = 3e-5; z[96:112] = -1e-3 * np.arange(16)
    rows.append(z)
    # non-finite entries: a NaN block decodes to NaN, infinities saturate
    nf = rng.standard_normal(512)
    nf[3] = np.nan; nf[16 + 5] = -np.nan; nf[40] = np.inf; nf[41] = -np.inf; nf[64:80] = np.nan
    nf[96] = np.inf; nf[97] = np.nan; nf[130] = -np.inf
    rows.append(nf)
    x = np.stack(rows)
    return torch.from_numpy(x).to(torch.bfloat16)


@pytest.mark.parametrize("n_rows", [1, 3, 17, 4096])
def test_pack_unpack_bit_exact_small(n_rows):
    dev = device()
    x = W.latent_rows(0, n_rows, device="cpu", chunk_index=n_rows)
    codes, scales = _gpu_pack(x.to(dev))
    rc, rs = OF.fp4_pack(x.to(torch.float64).numpy())
    assert np.array_equal(np_u8(codes), rc) and np.array_equal(np_u8(scales), rs)
    out = torch.empty((n_rows, 512), dtype=torch.bfloat16, device=dev)
    F.csa2_fp4_unpack(codes, scales, out)
    ref = OF.fp4_unpack(rc, rs)
    got = bf16_to_f64(out)
    assert np.array_equal(got, ref) and np.array_equal(np.signbit(got), np.signbit(ref))


def test_pack_special_values_bit_exact():
    dev = device()
    x = _special_rows()
    codes, scales = _gpu_pack(x.to(dev))
    rc, rs = OF.fp4_pack(x.to(torch.float64).numpy())
    assert np.array_equal(np_u8(scales), rs)
    assert np.array_equal(np_u8(codes), rc)
    # the unpacked values, NaN blocks included (NaN compares by position; the
    # sign bit is checked on every other value)
    out = torch.empty_like(x.to(dev))
    F.csa2_fp4_unpack(codes, scales, out)
    got, ref = bf16_to_f64(out), OF.fp4_unpack(rc, rs)
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and int(np.isnan(ref).sum()) == 64
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin]) and np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_pack_strided_into_cache_rows():
    # the decode step writes one new row per sequence at position T-1 of the cache
    dev = device()
    B, T = 5, 40
    cache_c = torch.zeros((B, T, 256), dtype=torch.uint8, device=dev)
    cache_s = torch.zeros((B, T, 32), dtype=torch.uint8, device=dev)
    src = W.latent_rows(1, 2 * B, device="cpu")
    x = src.to(dev)[::2]                   # strided input rows
    F.csa2_fp4_pack(x, cache_c[:, T - 1, :], cache_s[:, T - 1, :])
    rc, rs = OF.fp4_pack(src[::2].to(torch.float64).numpy())
    assert np.array_equal(np_u8(cache_c[:, T - 1]), rc) and np.array_equal(np_u8(cache_s[:, T - 1]), rs)
    assert int(cache_c[:, :T - 1].abs().sum()) == 0 and int(cache_s[:, :T - 1].abs().sum()) == 0


def test_pack_stream_1m_rows_sampled_and_round_trip():
    """FP4 pack then unpack of 1,048,576 x 512 (the memory-bound stream workload):
    sampled rows against the oracle, and pack(unpack(pack(x))) == pack(x) on every row."""
    dev = device()
    cfg = W.PackStream()
    out = W.outlier_channels(cfg.seed)
    x = W.latent_rows(cfg.seed, cfg.rows, device=dev, outliers=out)
    codes, scales = _gpu_pack(x)
    xb = torch.empty_like(x)
    F.csa2_fp4_unpack(codes, scales, xb)
    c2, s2 = _gpu_pack(xb)
    assert torch.equal(c2, codes) and torch.equal(s2, scales)
    rng = np.random.default_rng(cfg.seed)
    rows = np.sort(rng.choice(cfg.rows, 2048, replace=False))
    rows = np.concatenate([[0, cfg.rows - 1], rows])
    rt = torch.from_numpy(rows).to(dev)
    xs = x[rt].to(torch.float64).cpu().numpy()
    rc, rs = OF.fp4_pack(xs)
    assert np.array_equal(np_u8(codes[rt]), rc) and np.array_equal(np_u8(scales[rt]), rs)
    assert np.array_equal(bf16_to_f64(xb[rt]), OF.fp4_unpack(rc, rs))


def _every_scale_rows():
    """Blocks for every finite E4M3 scale code c: the first element fixes the block maximum (6 s_c, or
    the largest bf16 value whose sixth still rounds to s_c, so that elements up to 6.4 s_c saturate),
    the others run through every bf16 magnitude from 2^-14 s_c up to that maximum, with alternating
    signs, plus zeros of both signs; every E2M1 midpoint times s_c (a bf16 value) is among them."""
    blocks = []
    all_bf16 = OF.bf16_to_float(np.arange(0, 0x7F80, dtype=np.uint16))        # every finite magnitude
    for c in range(1, 0x7F):
        s = float(OF.e4m3_decode(np.array([c]))[0])
        above = all_bf16[(all_bf16 > 6 * s) & (all_bf16 <= 6.5 * s)]
        codes = OF.block_scales(np.repeat(above[:, None], 16, axis=1))[:, 0] if above.size else np.array([])
        tops = [6 * s] + ([float(above[codes == c].max())] if np.any(codes == c) else [])
        for top in tops:
            vals = all_bf16[(all_bf16 >= s * 2.0 ** -14) & (all_bf16 <= top)]
            vals = np.concatenate([vals, [0.0, -0.0]])
            sign = np.where(np.arange(vals.size) % 2 == 0, 1.0, -1.0)
            vals = vals * sign
            n_blk = -(-vals.size // 15)
            pad = np.zeros(n_blk * 15)
            pad[:vals.size] = vals
            b = np.empty((n_blk, 16))
            b[:, 0] = top
            b[:, 1:] = pad.reshape(n_blk, 15)
            blocks.append(b)
    # scale code 0: every magnitude below half the smallest E4M3 step times 6
    tiny = all_bf16[all_bf16 < 6 * 2.0 ** -10][-15:]
    blocks.append(np.concatenate([[6 * 2.0 ** -11], tiny * np.where(np.arange(15) % 2, -1, 1)])[None, :])
    b = np.concatenate(blocks)
    n_rows = -(-b.shape[0] // 32)
    rows = np.zeros((n_rows * 32, 16))
    rows[:b.shape[0]] = b
    return rows.reshape(n_rows, 512)


def test_pack_every_scale_and_magnitude_bit_exact():
    """The pack's E2M1 rounding (hardware FP4 conversion of the snapped quotient) against the oracle's
    threshold rule on every finite scale code and every bf16 magnitude up to the block maximum:
    ties to even, saturation above 6, signed zeros, zero scale."""
    dev = device()
    x64 = _every_scale_rows()
    x = torch.from_numpy(x64).to(torch.bfloat16)
    assert np.array_equal(x.to(torch.float64).numpy(), x64)          # every value is a bf16 value
    codes, scales = _gpu_pack(x.to(dev))
    rc, rs = OF.fp4_pack(x64)
    assert np.array_equal(np_u8(scales), rs)
    gc = np_u8(codes)
    bad = np.argwhere(gc != rc)
    assert bad.size == 0, f"{bad.shape[0]} code bytes differ, first at {bad[:4].tolist()}"
