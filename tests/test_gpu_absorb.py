"""GPU parity: query absorption and output unabsorption (csa2_absorb_q,
csa2_unabsorb_o) against the oracle's absorb / unabsorb (fp64), at the
workloads' 64 heads x 128 on the 512-channel latent, on ragged row counts.

Bounds (from the arithmetic the header states):
  * absorb: exact bf16 products summed in fp32 and rounded once to bf16, so
    |gpu - ref| <= 2^-8 |ref| (half an ulp of an 8-bit significand) +
    2^-20 sum_d |q_d w_dc| (fp32 sum), and all but a few elements equal the
    fp64 sum rounded to bf16 (they differ only where the fp32 sum crosses a
    rounding boundary);
  * unabsorb: o_lat enters as bf16 hi + lo (about 2^-17 relative), exact
    products, fp32 sum of 1,024 terms: |gpu - ref| <= 2^-13 sum_c |w_dc o_c|.
The unabsorbed output also meets the attention bar (per row and head, max
error <= 2e-3 of the row's max); the absorbed query is a correctly rounded bf16
value, whose rounding alone can reach 2^-8 of the row's max, so it is held to
the half-ulp bound instead.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA, formats as OF
import fp4_sparse_attention_amd as F
from gpu_common import device, bf16_to_f64

pytestmark = pytest.mark.gpu


def _normwise(got, ref):
    return float((np.abs(got - ref).max(axis=-1) / np.abs(ref).max(axis=-1)).max())


@pytest.mark.parametrize("R,H", [(8, 64), (64, 64), (1, 64), (77, 16), (200, 64)])
def test_absorb_q_vs_oracle(R, H):
    dev = device()
    q = W.head_queries(11, R, R, H, device=dev)
    w_uk, _ = W.absorb_weights(11, R, H, device=dev)
    q_lat = torch.empty((R, H, 512), dtype=torch.bfloat16, device=dev)
    F.csa2_absorb_q(q, w_uk, q_lat)
    torch.cuda.synchronize()
    qh, wh = bf16_to_f64(q), bf16_to_f64(w_uk)
    ref = OA.absorb(qh, wh)
    mag = np.einsum("rhd,hdc->rhc", np.abs(qh), np.abs(wh))
    got = bf16_to_f64(q_lat)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -20 * mag)
    rne = OF.bf16_to_float(OF.bf16_round(ref))
    assert np.mean(got != rne) <= 1e-3


@pytest.mark.parametrize("R,H", [(8, 64), (64, 64), (1, 16), (77, 64), (130, 48)])
def test_unabsorb_o_vs_oracle(R, H):
    dev = device()
    g = torch.Generator(device=dev); g.manual_seed(12 + R)
    o_lat = torch.randn((R, H, 512), generator=g, device=dev) * 0.3
    o_lat[0, 0, :7] = torch.tensor([1e-30, -3e5, 1e-3, 7.0, -0.0, 2.0 ** -20, 65504.0], device=dev)
    _, w_uv = W.absorb_weights(12, R, H, device=dev)
    out = torch.empty((R, H, 128), dtype=torch.float32, device=dev)
    F.csa2_unabsorb_o(o_lat, w_uv, out)
    torch.cuda.synchronize()
    oh, wh = o_lat.to(torch.float64).cpu().numpy(), bf16_to_f64(w_uv)
    ref = OA.unabsorb(oh, wh)
    mag = np.einsum("rhc,hdc->rhd", np.abs(oh), np.abs(wh))
    got = out.to(torch.float64).cpu().numpy()
    assert np.all(np.abs(got - ref) <= 2.0 ** -13 * mag)
    assert _normwise(got, ref) <= 2e-3


def test_absorb_attend_unabsorb_chain_per_call():
    """q -> absorb -> sparse + window attention -> unabsorb on the GPU, each call
    checked on its own inputs, at the 64-head decode shape of one sequence."""
    import math
    from gpu_common import DecodeWorkload, assert_attention_close
    from oracle import formats as OF
    dev = device()
    B, T, H, K = 2, 4096, 64, 256
    wl = DecodeWorkload(B, T, H, 1, seed=13)
    q = W.head_queries(13, 0, B, H, device=dev)
    w_uk, w_uv = W.absorb_weights(13, 0, H, device=dev)
    q_lat = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    F.csa2_absorb_q(q, w_uk, q_lat)
    idx = torch.stack([torch.randperm(T, device=dev)[:K] for _ in range(B)]).sort(dim=1).values.to(torch.int32)
    io = wl.layers[0]
    o = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    sigma = 1.0 / math.sqrt(128)
    F.csa2_sparse_swa_decode(q_lat, wl.codes, wl.scales, idx, io.swa, io.swa_start, io.swa_len, sigma, o, lse)
    out = torch.empty((B, H, 128), dtype=torch.float32, device=dev)
    F.csa2_unabsorb_o(o, w_uv, out)
    torch.cuda.synchronize()
    for b in range(B):
        pos = idx[b].cpu().numpy()
        c, s = OF.fp4_pack(wl.latent_host(b, pos))
        rows = OF.fp4_unpack(c, s)
        ql = bf16_to_f64(q_lat[b])
        o_s, l_s = OA.attend(ql, rows, sigma)
        o_w, l_w = OA.attend(ql, OA.window_rows(bf16_to_f64(io.swa[b]), int(io.swa_start[b]), int(io.swa_len[b])),
                             sigma)
        o_ref, l_ref = OA.merge(o_s, l_s, o_w, l_w)
        assert_attention_close(o[b].cpu().numpy(), lse[b].cpu().numpy(), o_ref, l_ref, f"chain b={b}")
        ref = OA.unabsorb(o[b].to(torch.float64).cpu().numpy(), bf16_to_f64(w_uv))
        assert _normwise(out[b].to(torch.float64).cpu().numpy(), ref) <= 2e-3


def test_absorb_unabsorb_empty_rows():
    dev = device()
    q = torch.zeros((0, 4, 128), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((4, 128, 512), dtype=torch.bfloat16, device=dev)
    F.csa2_absorb_q(q, w, torch.zeros((0, 4, 512), dtype=torch.bfloat16, device=dev))       # R = 0: no-op
    F.csa2_unabsorb_o(torch.zeros((0, 4, 512), device=dev), w, torch.zeros((0, 4, 128), device=dev))
    torch.cuda.synchronize()
