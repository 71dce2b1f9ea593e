"""GPU parity: csa2_index_full_pool over more rows than one workspace batch holds.

The streaming selection keeps worst-case candidate storage (8 bytes per visible
position) for at most ~896 MiB of rows at a time and runs larger row counts in
batches, so its workspace stays below 1 GB at any R.  These tests run shapes
with several batches: every output must equal the separate csa2_index_full +
csa2_topk_pool calls (dense rows: each batch reads its own sequences' keys), and
the 4,096-row chunked prefill over 2^20 positions must match the oracle on
sampled rows, including the first and last row of a batch.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import indexer as OI, topk as OT
import fp4_sparse_attention_amd as F
from gpu_common import device, np_u8, assert_topk_swap_rule

pytestmark = pytest.mark.gpu


def _e4m3_bytes(shape, seed, dev):
    """Random finite E4M3 bytes (every code but the two NaN codes), generated on the device."""
    g = torch.Generator(device=dev).manual_seed(seed)
    mag = torch.randint(0, 0x7F, shape, dtype=torch.uint8, device=dev, generator=g)
    sign = torch.randint(0, 2, shape, dtype=torch.uint8, device=dev, generator=g) << 7
    return mag | sign


def test_dense_rows_in_two_batches_equal_separate_calls():
    dev = device()
    R, T, k_pool, k_top = 2200, 40000, 2048, 256
    # 2,148 rows of 40,000 positions fill one batch: two batches, the second of 52 rows
    assert F.csa2_index_full_pool_workspace_size(R, T, k_pool) < F.csa2_index_full_pool_workspace_size(1, T, k_pool) * R
    k = _e4m3_bytes((R, T, 64), 7, dev)
    q = _e4m3_bytes((R, 64), 8, dev)
    p1 = torch.empty((R, k_pool), dtype=torch.int32, device=dev)
    t1 = torch.empty((R, k_top), dtype=torch.int32, device=dev)
    ps1 = torch.empty((R, k_pool), dtype=torch.float32, device=dev)
    F.csa2_index_full_pool(q, k, None, k_pool, k_top, p1, t1, pool_scores=ps1)
    s2 = torch.empty((R, T), dtype=torch.float32, device=dev)
    F.csa2_index_full(q, k, s2)
    p2, t2, ps2 = torch.empty_like(p1), torch.empty_like(t1), torch.empty_like(ps1)
    F.csa2_topk_pool(s2, k_pool, k_top, p2, t2, pool_scores=ps2)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(t1, t2)
    assert torch.equal(torch.nan_to_num(ps1, nan=7.0), torch.nan_to_num(ps2, nan=7.0))
    # a row of the second batch against the oracle's exact scores
    r = 2190
    s_ref = OI.full_scores(np_u8(q[r]), np_u8(k[r]))
    ref = OT.topk(s_ref, k_top)
    assert_topk_swap_rule(t1[r].cpu().numpy(), ref, lambda j: float(s_ref[j]), f"row {r}")


def test_prefill_4096_rows_over_1m_positions_sampled():
    """4,096 causal query rows of one sequence over 2^20 positions (row i sees positions
    <= 2^20 - 4,096 + i), Top-2,048 (pool = Top-K): workspace below 1 GB, sampled rows against
    the oracle's exact scores under the swap rule."""
    dev = device()
    R, T, K = 4096, 1 << 20, 2048
    ws_bytes = F.csa2_index_full_pool_workspace_size(R, T, K)
    assert ws_bytes < 10 ** 9
    k = torch.stack([W.fp8_normal(131, (T, 64), device=dev, chunk_index=0)])
    q = W.fp8_normal(132, (R, 64), device=dev)
    row_seq = torch.zeros(R, dtype=torch.int32, device=dev)
    limit = torch.arange(T - R, T, dtype=torch.int64, device=dev)
    pool = torch.empty((R, K), dtype=torch.int32, device=dev)
    top = torch.empty((R, K), dtype=torch.int32, device=dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    F.csa2_index_full_pool(q, k, None, K, K, pool, top, row_seq=row_seq, row_limit=limit, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(pool, top)
    kh = np_u8(k[0])
    rb = 96          # rows per batch at 2^20 positions
    for r in (0, rb - 1, rb, 2048, R - 1):
        lim = T - R + r
        s_ref = OI.full_scores(np_u8(q[r]), kh, limit=lim)
        ref = OT.topk(s_ref, K)
        assert_topk_swap_rule(top[r].cpu().numpy(), ref, lambda j: float(s_ref[j]), f"row {r}")
        assert int(top[r].max()) <= lim
