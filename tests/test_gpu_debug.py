"""GPU: the opt-in validation (CSA2_DEBUG) rejects bad device-side entries before any other launch.

Every bad entry below stays inside allocated memory even if it were not caught (the key and
window arrays have a spare sequence / rows behind the part passed), so a miss shows as a wrong
status, never as a fault."""
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
import fp4_sparse_attention_amd as F
from gpu_common import device

pytestmark = pytest.mark.gpu
SIGMA = 1.0 / math.sqrt(128)


@pytest.fixture
def debug_on():
    old = os.environ.get("CSA2_DEBUG")
    os.environ["CSA2_DEBUG"] = "1"
    yield
    if old is None:
        del os.environ["CSA2_DEBUG"]
    else:
        os.environ["CSA2_DEBUG"] = old


def _status(fn):
    try:
        fn()
        torch.cuda.synchronize()
        return 0
    except F.Csa2Error as e:
        return e.status


def test_debug_rejects_row_seq_outside_b(debug_on):
    dev = device()
    B, T, R = 3, 4096, 5
    # a spare sequence on both sides: row_seq -1 or B would still read allocated keys
    k_full = W.fp8_normal(3, (B + 2, T, 64), device=dev)
    k = k_full[1:B + 1]
    q = W.fp8_normal(4, (R, 64), device=dev)
    scores = torch.full((R, T), 7.0, device=dev)
    good = torch.tensor([0, 2, 1, 1, 0], dtype=torch.int32, device=dev)
    bad = torch.tensor([0, 2, 3, 1, 0], dtype=torch.int32, device=dev)
    assert _status(lambda: F.csa2_index_full(q, k, scores, row_seq=bad)) == 1
    assert bool((scores == 7.0).all())                       # nothing launched
    assert _status(lambda: F.csa2_index_full(q, k, scores, row_seq=good)) == 0
    ref = torch.empty_like(scores)
    os.environ["CSA2_DEBUG"] = "0"
    F.csa2_index_full(q, k, ref, row_seq=good)
    torch.cuda.synchronize()
    assert torch.equal(scores, ref)
    os.environ["CSA2_DEBUG"] = "1"
    # the pool call checks too
    pool = torch.empty((R, 256), dtype=torch.int32, device=dev)
    top = torch.empty((R, 64), dtype=torch.int32, device=dev)
    neg = torch.tensor([0, -1, 1, 1, 0], dtype=torch.int32, device=dev)
    assert _status(lambda: F.csa2_index_full_pool(q, k, None, 256, 64, pool, top, row_seq=neg)) == 1


def test_debug_rejects_attention_indices_and_window_bounds(debug_on):
    dev = device()
    B, T, H, K, S = 2, 3000, 32, 64, 200
    lat = W.latent_rows(5, B * T, device=dev)
    codes = torch.empty((B * T, 256), dtype=torch.uint8, device=dev)
    scales = torch.empty((B * T, 32), dtype=torch.uint8, device=dev)
    F.csa2_fp4_pack(lat, codes, scales)
    codes, scales = codes.view(B, T, 256), scales.view(B, T, 32)
    q = W.bf16_normal(6, (B, H, 512), std=0.5, device=dev)
    swa = W.bf16_normal(7, (B, S, 512), device=dev)
    g = torch.Generator(device=dev).manual_seed(8)
    idx = torch.sort(torch.randperm(T, device=dev, generator=g)[:K].repeat(B, 1).to(torch.int32), dim=1).values
    st = torch.tensor([0, 50], dtype=torch.int32, device=dev)
    ln = torch.tensor([128, 100], dtype=torch.int32, device=dev)
    o = torch.full((B, H, 512), 7.0, device=dev)
    lse = torch.empty((B, H), device=dev)
    call = lambda i, s_, l_: F.csa2_sparse_swa_decode(q, codes, scales, i, swa, s_, l_, SIGMA, o, lse)
    bad_idx = idx.clone()
    bad_idx[1, 5] = T + 5
    assert _status(lambda: call(bad_idx, st, ln)) == 1
    bad_ln = torch.tensor([128, 151], dtype=torch.int32, device=dev)      # 50 + 151 > S
    assert _status(lambda: call(idx, st, bad_ln)) == 1
    assert bool((o == 7.0).all())
    pad_idx = idx.clone()
    pad_idx[0, -3:] = -1                                                 # padding is valid
    assert _status(lambda: call(pad_idx, st, ln)) == 0
    ref_o, ref_l = torch.empty_like(o), torch.empty_like(lse)
    os.environ["CSA2_DEBUG"] = "0"
    F.csa2_sparse_swa_decode(q, codes, scales, pad_idx, swa, st, ln, SIGMA, ref_o, ref_l)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)
