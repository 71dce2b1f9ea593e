"""GPU parity: sparse attention over the FP4 cache and the sliding-window merge vs the oracle."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as OF, attention as OA
import fp4_sparse_attention_amd as F
from gpu_common import device, np_u8, bf16_to_f64, assert_attention_close

pytestmark = pytest.mark.gpu
SIGMA = 1.0 / math.sqrt(128)


def _cache(B, T, seed):
    lat = torch.stack([W.latent_rows(seed, T, chunk_index=b) for b in range(B)])      # bf16 [B,T,512] cpu
    codes, scales = [], []
    for b in range(B):
        c, s = OF.fp4_pack(lat[b].to(torch.float64).numpy())      # oracle side
        codes.append(c); scales.append(s)
    ref_rows = [OF.fp4_unpack(codes[b], scales[b]) for b in range(B)]
    return lat, ref_rows


def _gpu_cache(lat, dev):
    B, T, _ = lat.shape
    codes = torch.empty((B, T, 256), dtype=torch.uint8, device=dev)
    scales = torch.empty((B, T, 32), dtype=torch.uint8, device=dev)
    x = lat.to(dev)
    for b in range(B):
        F.csa2_fp4_pack(x[b], codes[b], scales[b])
    return codes, scales


@pytest.mark.parametrize("B,T,H,K", [(1, 4096, 16, 256), (2, 1000, 64, 300), (3, 700, 32, 33),
                                     (1, 300, 48, 512), (2, 5000, 64, 2048)])
def test_sparse_decode_vs_oracle(B, T, H, K):
    dev = device()
    rng = np.random.default_rng(B * 1000 + K)
    lat, ref_rows = _cache(B, T, seed=21)
    codes, scales = _gpu_cache(lat, dev)
    q = W.bf16_normal(22, (B, H, 512), std=0.5)
    idx = np.full((B, K), -1, dtype=np.int32)
    for b in range(B):
        n = min(K, T) - (b % 2) * 7                              # some -1 padding
        idx[b, :n] = np.sort(rng.choice(T, n, replace=False))
    if K > 40:
        idx[0, 5] = T + 3                                        # out of range: skipped
    o = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    F.csa2_sparse_decode(q.to(dev), codes, scales, torch.from_numpy(idx).to(dev), SIGMA, o, lse)
    qf = q.to(torch.float64).numpy()
    for b in range(B):
        valid = idx[b][(idx[b] >= 0) & (idx[b] < T)]
        o_ref, l_ref = OA.sparse_attend(qf[b], ref_rows[b], valid, SIGMA)
        assert_attention_close(o[b].cpu().numpy(), lse[b].cpu().numpy(), o_ref, l_ref, f"row {b}")


def test_sparse_decode_empty_rows_and_row_seq():
    dev = device()
    T, H = 500, 16
    lat, ref_rows = _cache(2, T, seed=23)
    codes, scales = _gpu_cache(lat, dev)
    R, K = 4, 64
    row_seq = np.array([1, 0, 1, 0], dtype=np.int32)
    q = W.bf16_normal(24, (R, H, 512), std=0.5)
    idx = np.full((R, K), -1, dtype=np.int32)
    idx[0, :10] = np.arange(10) * 7
    idx[2, :K] = np.arange(K) + 100                      # row 1 and row 3 stay empty
    o = torch.empty((R, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    F.csa2_sparse_decode(q.to(dev), codes, scales, torch.from_numpy(idx).to(dev), SIGMA, o, lse,
                         row_seq=torch.from_numpy(row_seq).to(dev))
    qf = q.to(torch.float64).numpy()
    for r in range(R):
        o_ref, l_ref = OA.sparse_attend(qf[r], ref_rows[row_seq[r]], idx[r], SIGMA)
        assert_attention_close(o[r].cpu().numpy(), lse[r].cpu().numpy(), o_ref, l_ref, f"row {r}")
    assert torch.all(o[1] == 0) and torch.all(torch.isneginf(lse[1]))


@pytest.mark.parametrize("with_sparse", [True, False])
def test_swa_merge_vs_oracle(with_sparse):
    dev = device()
    B, H, S = 4, 64, 160
    q = W.bf16_normal(25, (B, H, 512), std=0.5)
    swa = W.bf16_normal(26, (B, S, 512))
    start = np.array([0, 5, 32, 150], dtype=np.int32)
    length = np.array([128, 1, 77, 0], dtype=np.int32)
    qf = q.to(torch.float64).numpy()
    swf = swa.to(torch.float64).numpy()
    rng = np.random.default_rng(5)
    o_s = rng.standard_normal((B, H, 512)).astype(np.float32)
    l_s = (rng.standard_normal((B, H)) * 3).astype(np.float32)
    l_s[2, :5] = -np.inf
    o_s[2, :5] = 0
    o_out = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    lse_out = torch.empty((B, H), dtype=torch.float32, device=dev)
    kw = {}
    if with_sparse:
        kw = dict(o_sparse=torch.from_numpy(o_s).to(dev), lse_sparse=torch.from_numpy(l_s).to(dev))
    F.csa2_swa_merge(q.to(dev), swa.to(dev), torch.from_numpy(start).to(dev), torch.from_numpy(length).to(dev),
                     SIGMA, o_out, lse_out, **kw)
    for b in range(B):
        o_w, l_w = OA.attend(qf[b], OA.window_rows(swf[b], int(start[b]), int(length[b])), SIGMA)
        if with_sparse:
            o_ref, l_ref = OA.merge(o_s[b].astype(np.float64), l_s[b].astype(np.float64), o_w, l_w)
        else:
            o_ref, l_ref = o_w, l_w
        assert_attention_close(o_out[b].cpu().numpy(), lse_out[b].cpu().numpy(), o_ref, l_ref, f"row {b}")


def test_swa_merge_in_place_and_window_bound():
    # o_out aliases o_sparse; rows outside the window do not change the result
    dev = device()
    B, H, S = 2, 32, 300
    q = W.bf16_normal(27, (B, H, 512), std=0.5).to(dev)
    swa = W.bf16_normal(28, (B, S, 512)).to(dev)
    start = torch.tensor([172, 0], dtype=torch.int32, device=dev)
    length = torch.tensor([128, 128], dtype=torch.int32, device=dev)
    o1 = torch.randn((B, H, 512), device=dev)
    l1 = torch.randn((B, H), device=dev)
    o_keep, l_keep = o1.clone(), l1.clone()
    F.csa2_swa_merge(q, swa, start, length, SIGMA, o1, l1, o_sparse=o1, lse_sparse=l1)
    o2, l2 = o_keep.clone(), l_keep.clone()
    swa2 = swa.clone()
    swa2[0, :172] = torch.randn_like(swa2[0, :172]).to(torch.bfloat16) * 50
    swa2[1, 128:] = 1000
    F.csa2_swa_merge(q, swa2, start, length, SIGMA, o2, l2, o_sparse=o2, lse_sparse=l2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3 = torch.empty_like(o1); l3 = torch.empty_like(l1)
    F.csa2_swa_merge(q, swa, start, length, SIGMA, o3, l3, o_sparse=o_keep, lse_sparse=l_keep)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_sparse_decode_deterministic():
    dev = device()
    T, H, K = 3000, 64, 2048
    lat, _ = _cache(1, T, seed=29)
    codes, scales = _gpu_cache(lat, dev)
    q = W.bf16_normal(30, (1, H, 512), std=0.5).to(dev)
    idx = torch.from_numpy(np.sort(np.random.default_rng(0).choice(T, K, replace=False)).astype(np.int32)[None]).to(dev)
    outs = []
    for _ in range(2):
        o = torch.empty((1, H, 512), dtype=torch.float32, device=dev)
        lse = torch.empty((1, H), dtype=torch.float32, device=dev)
        F.csa2_sparse_decode(q, codes, scales, idx, SIGMA, o, lse)
        outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("B,T,H,K", [(2, 3000, 64, 2048), (3, 700, 16, 100)])
def test_fused_sparse_window_vs_oracle(B, T, H, K):
    """csa2_sparse_swa_decode = sparse attention over idx and the window rows in one softmax."""
    dev = device()
    rng = np.random.default_rng(T + K)
    lat, ref_rows = _cache(B, T, seed=31)
    codes, scales = _gpu_cache(lat, dev)
    q = W.bf16_normal(32, (B, H, 512), std=0.5)
    S = 140
    swa = W.bf16_normal(33, (B, S, 512))
    start = np.array([12, 0, 3][:B], dtype=np.int32)
    length = np.array([128, 0, 57][:B], dtype=np.int32)
    idx = np.full((B, K), -1, dtype=np.int32)
    for b in range(B):
        n = min(K, T) - 5 * b
        idx[b, :n] = np.sort(rng.choice(T, n, replace=False))
    o = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    F.csa2_sparse_swa_decode(q.to(dev), codes, scales, torch.from_numpy(idx).to(dev), swa.to(dev),
                             torch.from_numpy(start).to(dev), torch.from_numpy(length).to(dev), SIGMA, o, lse)
    qf = q.to(torch.float64).numpy()
    swf = swa.to(torch.float64).numpy()
    for b in range(B):
        o_s, l_s = OA.sparse_attend(qf[b], ref_rows[b], idx[b], SIGMA)
        o_w, l_w = OA.attend(qf[b], OA.window_rows(swf[b], int(start[b]), int(length[b])), SIGMA)
        o_ref, l_ref = OA.merge(o_s, l_s, o_w, l_w)
        assert_attention_close(o[b].cpu().numpy(), lse[b].cpu().numpy(), o_ref, l_ref, f"row {b}")


def test_layers_call_matches_oracle_per_layer():
    """csa2_sparse_swa_decode_layers: each layer = sparse attention over its idx
    slice plus its own window, one softmax; layers 1 and 2 share slice 1."""
    dev = device()
    L, B, T, H, K, S = 3, 3, 2500, 64, 300, 140
    rng = np.random.default_rng(41)
    lat, ref_rows = _cache(B, T, seed=43)
    codes, scales = _gpu_cache(lat, dev)
    q = W.bf16_normal(44, (L, B, H, 512), std=0.5)
    swa = W.bf16_normal(45, (L, B, S, 512))
    start = np.array([[12, 0, 3], [0, 5, 7], [2, 0, 11]], dtype=np.int32)
    length = np.array([[128, 0, 57], [1, 128, 33], [77, 128, 0]], dtype=np.int32)
    idx = np.full((2, B, K), -1, dtype=np.int32)
    for sl in range(2):
        for b in range(B):
            n = K - 7 * b - sl
            idx[sl, b, :n] = np.sort(rng.choice(T, n, replace=False))
    layer_idx = [0, 1, 1]
    o = torch.empty((L, B, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((L, B, H), dtype=torch.float32, device=dev)
    F.csa2_sparse_swa_decode_layers(q.to(dev), codes, scales, torch.from_numpy(idx).to(dev), layer_idx, swa.to(dev),
                                    torch.from_numpy(start).to(dev), torch.from_numpy(length).to(dev), SIGMA, o, lse)
    qf = q.to(torch.float64).numpy()
    swf = swa.to(torch.float64).numpy()
    for l in range(L):
        for b in range(B):
            o_s, l_s = OA.sparse_attend(qf[l, b], ref_rows[b], idx[layer_idx[l], b], SIGMA)
            o_w, l_w = OA.attend(qf[l, b], OA.window_rows(swf[l, b], int(start[l, b]), int(length[l, b])), SIGMA)
            o_ref, l_ref = OA.merge(o_s, l_s, o_w, l_w)
            assert_attention_close(o[l, b].cpu().numpy(), lse[l, b].cpu().numpy(), o_ref, l_ref, f"layer {l} row {b}")


def test_layers_call_equals_single_layer_calls():
    # the multi-layer launch and per-layer csa2_sparse_swa_decode give the same bits
    dev = device()
    L, B, T, H, K, S = 4, 8, 4096, 64, 2048, 128
    lat, _ = _cache(B, T, seed=47)
    codes, scales = _gpu_cache(lat, dev)
    q = W.bf16_normal(48, (L, B, H, 512), std=0.5).to(dev)
    swa = W.bf16_normal(49, (L, B, S, 512)).to(dev)
    st = torch.zeros((L, B), dtype=torch.int32, device=dev)
    ln = torch.full((L, B), 128, dtype=torch.int32, device=dev)
    g = torch.Generator(device=dev).manual_seed(50)
    idx = torch.sort(torch.randperm(T, device=dev, generator=g)[:K].repeat(2, B, 1).to(torch.int32), dim=2).values
    layer_idx = [0, 1, 1, 1]
    o = torch.empty((L, B, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((L, B, H), dtype=torch.float32, device=dev)
    F.csa2_sparse_swa_decode_layers(q, codes, scales, idx, layer_idx, swa, st, ln, SIGMA, o, lse)
    for l in range(L):
        o1 = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
        l1 = torch.empty((B, H), dtype=torch.float32, device=dev)
        F.csa2_sparse_swa_decode(q[l].contiguous(), codes, scales, idx[layer_idx[l]].contiguous(), swa[l].contiguous(),
                                 st[l].contiguous(), ln[l].contiguous(), SIGMA, o1, l1)
        # chunking differs between the two launches: compare to the attention tolerance
        ref_o = o1.cpu().numpy().astype(np.float64)
        ref_l = l1.cpu().numpy().astype(np.float64)
        for b in range(B):
            assert_attention_close(o[l, b].cpu().numpy(), lse[l, b].cpu().numpy(), ref_o[b], ref_l[b], f"layer {l} b {b}")


def test_many_rows_single_chunk_writes_outputs_directly():
    """With enough rows (here 300 over 2 sequences, 64 heads) each row is one chunk and the chunk
    kernel writes the normalised o and lse itself: against the oracle on sampled rows, including
    a row with no valid key and no window (o = 0, lse = -inf), a window-only row and a sparse-only
    row; the same rows through csa2_sparse_decode (one chunk, direct) and csa2_swa_merge (with a
    prior, through the combine) agree with the fused call within rounding."""
    dev = device()
    B, T, H, K, R = 2, 3000, 64, 256, 300
    rng = np.random.default_rng(41)
    lat, ref_rows = _cache(B, T, seed=43)
    codes, scales = _gpu_cache(lat, dev)
    row_seq = (np.arange(R) % B).astype(np.int32)
    q = W.bf16_normal(44, (R, H, 512), std=0.5)
    S = 400
    swa = W.bf16_normal(45, (B, S, 512))
    start = rng.integers(0, S - 128, R).astype(np.int32)
    length = np.full(R, 128, dtype=np.int32)
    idx = np.stack([np.sort(rng.choice(T, K, replace=False)) for _ in range(R)]).astype(np.int32)
    idx[0] = -1
    length[0] = 0                      # nothing at all
    idx[1] = -1                        # window only
    length[2] = 0                      # sparse only
    idx[3, 100:] = -1                  # short sparse list
    to = lambda a: torch.from_numpy(a).to(dev)
    o = torch.empty((R, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    F.csa2_sparse_swa_decode(q.to(dev), codes, scales, to(idx), swa.to(dev), to(start), to(length), SIGMA, o, lse,
                             row_seq=to(row_seq))
    o2 = torch.empty_like(o)
    lse2 = torch.empty_like(lse)
    F.csa2_sparse_decode(q.to(dev), codes, scales, to(idx), SIGMA, o2, lse2, row_seq=to(row_seq))
    F.csa2_swa_merge(q.to(dev), swa.to(dev), to(start), to(length), SIGMA, o2, lse2, o_sparse=o2, lse_sparse=lse2,
                     row_seq=to(row_seq))
    torch.cuda.synchronize()
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    qf = q.to(torch.float64).numpy()
    swf = swa.to(torch.float64).numpy()
    for r in (0, 1, 2, 3, 150, R - 1):
        b = int(row_seq[r])
        o_s, l_s = OA.sparse_attend(qf[r], ref_rows[b], idx[r], SIGMA)
        o_w, l_w = OA.attend(qf[r], OA.window_rows(swf[b], int(start[r]), int(length[r])), SIGMA)
        o_ref, l_ref = OA.merge(o_s, l_s, o_w, l_w)
        assert_attention_close(o[r].cpu().numpy(), lse[r].cpu().numpy(), o_ref, l_ref, f"row {r}")
        assert_attention_close(o2[r].cpu().numpy(), lse2[r].cpu().numpy(), o_ref, l_ref, f"row {r} two calls")


def test_attention_exact_for_wide_range_bf16_inputs():
    """Queries and window rows far outside the f16 range (bf16 magnitudes 2^-100 .. 2^80): each head's
    query is scaled by a power of two before the f16 products and window rows go through bf16
    products, so the result matches the oracle (fp64) as closely as for unit-scale inputs.  The lse of
    a huge score carries fp32 relative error, so it is held to 1e-4 + 2^-16 * sigma * max_j sum_c
    |q_c x_jc| (the fp32 rounding of the score sums) instead of the plain 1e-4."""
    dev = device()
    B, T, H, K = 3, 2000, 64, 256
    rng = np.random.default_rng(91)
    lat, ref_rows = _cache(B, T, seed=92)
    codes, scales = _gpu_cache(lat, dev)
    q = W.bf16_normal(93, (B, H, 512), std=0.5).to(torch.float32)
    q[:, 0:16] *= 2.0 ** 40          # huge: products far above the f16 range
    q[:, 16:32] *= 2.0 ** -60        # tiny: below the f16 subnormals
    q[:, 48:64] *= 2.0 ** 20
    q[1, 40, :7] = torch.tensor([1e30, -1e-38, 65504.0, 7e4, 2.0 ** -30, 0.0, -0.0])
    q = q.to(torch.bfloat16)
    S = 130
    swa = W.bf16_normal(94, (B, S, 512)).to(torch.float32)
    swa[0] *= 2.0 ** 80
    swa[1] *= 2.0 ** -100
    swa[2, 0::2] *= 2.0 ** 60
    swa[2, 1::2] *= 2.0 ** -60
    swa = swa.to(torch.bfloat16)
    start = np.array([0, 2, 1], dtype=np.int32)
    length = np.array([128, 128, 77], dtype=np.int32)
    idx = np.stack([np.sort(rng.choice(T, K, replace=False)) for _ in range(B)]).astype(np.int32)
    o = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    F.csa2_sparse_swa_decode(q.to(dev), codes, scales, torch.from_numpy(idx).to(dev), swa.to(dev),
                             torch.from_numpy(start).to(dev), torch.from_numpy(length).to(dev), SIGMA, o, lse)
    qf = q.to(torch.float64).numpy()
    swf = swa.to(torch.float64).numpy()
    for b in range(B):
        win = OA.window_rows(swf[b], int(start[b]), int(length[b]))
        o_s, l_s = OA.sparse_attend(qf[b], ref_rows[b], idx[b], SIGMA)
        o_w, l_w = OA.attend(qf[b], win, SIGMA)
        o_ref, l_ref = OA.merge(o_s, l_s, o_w, l_w)
        got_o, got_l = o[b].cpu().numpy().astype(np.float64), lse[b].cpu().numpy().astype(np.float64)
        err = np.abs(got_o - o_ref).max(axis=-1) / np.abs(o_ref).max(axis=-1)
        assert float(err.max()) <= 2e-3, f"row {b}: normwise error {float(err.max()):.3e}"
        rows = np.concatenate([ref_rows[b][idx[b]], win])
        mag = SIGMA * (np.abs(qf[b]) @ np.abs(rows).T).max(axis=1)
        assert np.all(np.abs(got_l - l_ref) <= 1e-4 + 2.0 ** -16 * mag), f"row {b}: lse"
