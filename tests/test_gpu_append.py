"""GPU parity for the decode-time append: the new token's FP4 cache row, its
indexer key and every layer's window row (mirrored ring) over many steps with
sequences of different lengths; the ring's window feeds the attention call and
matches the oracle over the last min(128, t + 1) appended rows."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA, formats as OF
import fp4_sparse_attention_amd as F
from gpu_common import device, assert_attention_close

pytestmark = pytest.mark.gpu
SIGMA = 1.0 / math.sqrt(128)


def test_decode_append_cache_keys_and_window_ring():
    dev = device()
    B, L, T, S = 3, 2, 320, 256
    n_tok = [300, 129, 5]                                      # tokens appended per sequence
    g = torch.Generator(device="cpu").manual_seed(131)
    codes = torch.full((B * T, 256), 0xA5, dtype=torch.uint8, device=dev)
    scales = torch.full((B * T, 32), 0x5A, dtype=torch.uint8, device=dev)
    k_idx = torch.full((B * T, 64), 0x11, dtype=torch.uint8, device=dev)
    swa = torch.zeros((L, B, S, 512), dtype=torch.bfloat16, device=dev)
    start = torch.full((L, B), -7, dtype=torch.int32, device=dev)
    length = torch.full((L, B), -7, dtype=torch.int32, device=dev)
    lat_hist, key_hist = [[] for _ in range(B)], [[] for _ in range(B)]
    win_hist = [[[] for _ in range(B)] for _ in range(L)]
    checks = {0, 1, 4, 126, 127, 128, 129, 200, 299}
    for step in range(max(n_tok)):
        lat = W.latent_rows(132, B, chunk_index=step)                        # bf16 [B, 512] cpu
        keys = torch.randint(0, 256, (B, 64), dtype=torch.uint8, generator=g)
        keys[(keys & 0x7F) == 0x7F] = 0                                       # no NaN codes
        win = W.bf16_normal(133, (L, B, 512), chunk_index=step)
        live = [step < n for n in n_tok]
        rows = torch.tensor([b * T + step if live[b] else -1 for b in range(B)], dtype=torch.int64)
        pos = torch.tensor([step if live[b] else -1 for b in range(B)], dtype=torch.int64)
        F.csa2_decode_append(lat.to(dev), rows.to(dev), codes, scales, new_keys=keys.to(dev), k_idx=k_idx,
                             new_window=win.to(dev), swa=swa, tok_pos=pos.to(dev), swa_start=start, swa_len=length)
        for b in range(B):
            if live[b]:
                lat_hist[b].append(lat[b])
                key_hist[b].append(keys[b])
                for l in range(L):
                    win_hist[l][b].append(win[l, b])
        if step in checks:
            torch.cuda.synchronize()
            st, ln, ring = start.cpu().numpy(), length.cpu().numpy(), swa.cpu()
            for l in range(L):
                for b in range(B):
                    t = min(step, n_tok[b] - 1)
                    want_len = min(128, t + 1)
                    assert ln[l, b] == want_len and st[l, b] == ((t + 1) % 128 if t >= 127 else 0), (step, l, b)
                    got = ring[l, b, st[l, b]:st[l, b] + ln[l, b]]
                    want = torch.stack(win_hist[l][b][-want_len:])
                    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (step, l, b)
    torch.cuda.synchronize()
    c_h, s_h, k_h = codes.cpu().numpy(), scales.cpu().numpy(), k_idx.cpu().numpy()
    for b in range(B):
        n = n_tok[b]
        x = torch.stack(lat_hist[b])
        dc = torch.empty((n, 256), dtype=torch.uint8, device=dev)
        ds = torch.empty((n, 32), dtype=torch.uint8, device=dev)
        F.csa2_fp4_pack(x.to(dev), dc, ds)
        assert np.array_equal(c_h[b * T:b * T + n], dc.cpu().numpy()), b
        assert np.array_equal(s_h[b * T:b * T + n], ds.cpu().numpy()), b
        oc, os_ = OF.fp4_pack(x[:3].to(torch.float64).numpy())
        assert np.array_equal(c_h[b * T:b * T + 3], oc) and np.array_equal(s_h[b * T:b * T + 3], os_), b
        assert np.array_equal(k_h[b * T:b * T + n], torch.stack(key_hist[b]).numpy()), b
        assert (c_h[b * T + n:(b + 1) * T] == 0xA5).all() and (k_h[b * T + n:(b + 1) * T] == 0x11).all(), b
    # the ring's window in an attention call: sparse keys from the cache plus the window, against the oracle
    H, K = 16, 64
    q = W.bf16_normal(134, (B, H, 512), std=0.5)
    idx = np.full((B, K), -1, dtype=np.int32)
    rng = np.random.default_rng(135)
    for b in range(B):
        m = min(K, n_tok[b])
        idx[b, :m] = np.sort(rng.choice(n_tok[b], m, replace=False))
    o = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    l = 1
    F.csa2_sparse_swa_decode(q.to(dev), codes.view(B, T, 256), scales.view(B, T, 32), torch.from_numpy(idx).to(dev),
                             swa[l].contiguous(), start[l].contiguous(), length[l].contiguous(), SIGMA, o, lse)
    qf = q.to(torch.float64).numpy()
    for b in range(B):
        rows = OF.fp4_unpack(*OF.fp4_pack(torch.stack(lat_hist[b]).to(torch.float64).numpy()))
        o_s, l_s = OA.sparse_attend(qf[b], rows, idx[b][idx[b] >= 0], SIGMA)
        t = n_tok[b] - 1
        wrows = torch.stack(win_hist[l][b][-min(128, t + 1):]).to(torch.float64).numpy()
        o_w, l_w = OA.attend(qf[b], wrows, SIGMA)
        o_ref, l_ref = OA.merge(o_s, l_s, o_w, l_w)
        assert_attention_close(o[b].cpu().numpy(), lse[b].cpu().numpy(), o_ref, l_ref, f"row {b}")
