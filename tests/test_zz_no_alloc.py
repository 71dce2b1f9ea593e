"""Allocation-free multi-layer attention: csa2_sparse_swa_decode_layers_noalloc
against csa2_sparse_swa_decode_layers (caller workspace) on the same inputs.

Both run the same kernels with the same chunk plan, so o and lse agree bit for
bit.  The calls run back to back, the second on a smaller input, so that the
second reads only what it wrote itself into the library's shared static array.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as OF, attention as OA
import fp4_sparse_attention_amd as F
from gpu_common import device, assert_attention_close

pytestmark = pytest.mark.gpu
SIGMA = 1.0 / math.sqrt(128)


def _inputs(dev, L, B, T, H, K, S, seed, ragged):
    lat = torch.stack([W.latent_rows(seed, T, chunk_index=b) for b in range(B)])
    codes = torch.empty((B, T, 256), dtype=torch.uint8, device=dev)
    scales = torch.empty((B, T, 32), dtype=torch.uint8, device=dev)
    x = lat.to(dev)
    for b in range(B):
        F.csa2_fp4_pack(x[b], codes[b], scales[b])
    q = W.bf16_normal(seed + 1, (L, B, H, 512), std=0.5).to(dev)
    swa = W.bf16_normal(seed + 2, (L, B, S, 512)).to(dev)
    rng = np.random.default_rng(seed)
    start = np.zeros((L, B), dtype=np.int32)
    length = np.full((L, B), min(128, S), dtype=np.int32)
    idx = np.full((2, B, K), -1, dtype=np.int32)
    for sl in range(2):
        for b in range(B):
            n = min(K, T) - (7 * b + sl if ragged else 0)
            idx[sl, b, :n] = np.sort(rng.choice(T, n, replace=False))
    if ragged:
        start[:, :] = rng.integers(0, S - 128 + 1, size=(L, B))
        length[:, :] = rng.integers(0, 129, size=(L, B))
        length[0, 0] = 0                               # a row with no window
    return (lat, codes, scales, q, torch.from_numpy(idx).to(dev), swa, torch.from_numpy(start).to(dev),
            torch.from_numpy(length).to(dev))


def _both(dev, L, B, T, H, K, S, seed, ragged=False, layer_idx=None):
    lat, codes, scales, q, idx, swa, st, ln = _inputs(dev, L, B, T, H, K, S, seed, ragged)
    layer_idx = layer_idx or [0] + [1] * (L - 1)
    o_ws = torch.empty((L, B, H, 512), dtype=torch.float32, device=dev)
    l_ws = torch.empty((L, B, H), dtype=torch.float32, device=dev)
    F.csa2_sparse_swa_decode_layers(q, codes, scales, idx, layer_idx, swa, st, ln, SIGMA, o_ws, l_ws)
    o_na = torch.full((L, B, H, 512), float("nan"), dtype=torch.float32, device=dev)
    l_na = torch.full((L, B, H), float("nan"), dtype=torch.float32, device=dev)
    F.csa2_sparse_swa_decode_layers_noalloc(q, codes, scales, idx, layer_idx, swa, st, ln, SIGMA, o_na, l_na)
    torch.cuda.synchronize()
    return (lat, q, idx, swa, st, ln, layer_idx), (o_ws, l_ws), (o_na, l_na)


def _bits_equal(a, b):
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_noalloc_equals_workspace_call_twice_second_smaller():
    dev = device()
    # large: 4 layers x 8 rows x 64 heads, K = 2048, 8 chunks per row (32 MiB of partials)
    need = F.csa2_sparse_swa_decode_layers_workspace_size(4, 8, 64, 2048)
    assert 16 << 20 < need <= F.NOALLOC_SCRATCH_BYTES
    _, (o1, l1), (o2, l2) = _both(dev, 4, 8, 8192, 64, 2048, 128, seed=61)
    assert _bits_equal(o1, o2) and _bits_equal(l1, l2)
    # smaller, ragged: 2 layers x 3 rows x 32 heads, K = 300, window bounds drawn per row
    inp, (o1, l1), (o2, l2) = _both(dev, 2, 3, 3000, 32, 300, 200, seed=62, ragged=True)
    assert _bits_equal(o1, o2) and _bits_equal(l1, l2)
    # and the smaller call against the oracle
    lat, q, idx, swa, st, ln, layer_idx = inp
    rows = [OF.fp4_unpack(*OF.fp4_pack(lat[b].to(torch.float64).numpy())) for b in range(lat.shape[0])]
    qf = q.cpu().to(torch.float64).numpy()
    swf = swa.cpu().to(torch.float64).numpy()
    idx_h, st_h, ln_h = idx.cpu().numpy(), st.cpu().numpy(), ln.cpu().numpy()
    for l in range(qf.shape[0]):
        for b in range(qf.shape[1]):
            sel = idx_h[layer_idx[l], b]
            o_s, s_s = OA.sparse_attend(qf[l, b], rows[b], sel[sel >= 0], SIGMA)
            o_w, s_w = OA.attend(qf[l, b], OA.window_rows(swf[l, b], int(st_h[l, b]), int(ln_h[l, b])), SIGMA)
            o_ref, l_ref = OA.merge(o_s, s_s, o_w, s_w)
            assert_attention_close(o2[l, b].cpu().numpy(), l2[l, b].cpu().numpy(), o_ref, l_ref, f"layer {l} row {b}")


def test_noalloc_one_chunk_rows_and_oversize_shape():
    dev = device()
    # 4 layers x 64 rows: each (layer, row) is one chunk, written without partials
    _, (o1, l1), (o2, l2) = _both(dev, 4, 64, 1024, 64, 2048, 128, seed=63)
    assert _bits_equal(o1, o2) and _bits_equal(l1, l2)
    # K = 8192 over 128 rows of one sequence: the partials need more than the array
    L, R, H, K, T = 1, 128, 64, 8192, 8192
    assert F.csa2_sparse_swa_decode_layers_workspace_size(L, R, H, K) > F.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((L, R, H, 512), dtype=torch.bfloat16, device=dev)
    codes = torch.zeros((1, T, 256), dtype=torch.uint8, device=dev)
    scales = torch.zeros((1, T, 32), dtype=torch.uint8, device=dev)
    idx = torch.zeros((1, R, K), dtype=torch.int32, device=dev)
    swa = torch.zeros((L, 1, 128, 512), dtype=torch.bfloat16, device=dev)
    st = torch.zeros((L, R), dtype=torch.int32, device=dev)
    ln = torch.zeros((L, R), dtype=torch.int32, device=dev)
    row_seq = torch.zeros((R,), dtype=torch.int32, device=dev)
    o = torch.full((L, R, H, 512), 7.0, dtype=torch.float32, device=dev)
    lse = torch.full((L, R, H), 7.0, dtype=torch.float32, device=dev)
    with pytest.raises(F.Csa2Error) as e:
        F.csa2_sparse_swa_decode_layers_noalloc(q, codes, scales, idx, [0], swa, st, ln, SIGMA, o, lse,
                                                row_seq=row_seq)
    assert e.value.status == 6
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())     # refused before any launch
