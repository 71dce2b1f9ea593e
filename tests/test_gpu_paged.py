"""GPU parity for the paged global KV calls: each paged call computes, on
shuffled page pools with partial last pages, unmapped blocks and per-row
lengths, exactly what the dense call computes on the logical sequences that
the oracle's page map reads out of the pools."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import paging as OP, attention as OA, formats as OF, topk as OT
import fp4_sparse_attention_amd as F
from gpu_common import device, assert_attention_close

pytestmark = pytest.mark.gpu
SIGMA = 1.0 / math.sqrt(128)


def _page_table(rng, B, max_blocks, lengths=None, page=None, holes=(), spare=3):
    """Random distinct page ids for every block; blocks past a sequence's
    length and the listed (b, j) holes are unmapped (-1)."""
    n_pages = B * max_blocks + spare
    table = rng.permutation(n_pages)[:B * max_blocks].astype(np.int32).reshape(B, max_blocks)
    if lengths is not None:
        for b, n in enumerate(lengths):
            table[b, (n + page - 1) // page:] = -1
    for b, j in holes:
        table[b, j] = -1
    return table, n_pages


def _rows_of(table, page, T):
    """Physical row of every (b, p), -1 where unmapped (vectorised, written apart from the oracle's map)."""
    p = np.arange(T)
    pg = table[:, p // page]
    return np.where(pg >= 0, pg.astype(np.int64) * page + p % page, -1)


def _dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


@pytest.mark.parametrize("page", [128, 256])
def test_pack_rows_scatters_into_pages(page):
    dev = device()
    rng = np.random.default_rng(page)
    B, T, max_blocks = 3, 700, 6
    table, n_pages = _page_table(rng, B, max_blocks, lengths=[700, 513, 128], page=page)
    rows = _rows_of(table, page, T)
    lat = torch.stack([W.latent_rows(71, T, chunk_index=b) for b in range(B)])          # bf16 [B, T, 512]
    wide = torch.zeros((B * T, 640), dtype=torch.bfloat16, device=dev)                  # strided source rows
    wide[:, :512] = lat.reshape(B * T, 512).to(dev)
    codes = torch.full((n_pages * page, 256), 0xA5, dtype=torch.uint8, device=dev)
    scales = torch.full((n_pages * page, 32), 0x5A, dtype=torch.uint8, device=dev)
    out_rows = rows.reshape(-1).copy()
    out_rows[5] = -1                                                                    # skipped row
    F.csa2_fp4_pack_rows(wide[:, :512], _dev(out_rows, dev), codes, scales)
    dc = torch.empty((B * T, 256), dtype=torch.uint8, device=dev)
    ds = torch.empty((B * T, 32), dtype=torch.uint8, device=dev)
    F.csa2_fp4_pack(lat.reshape(B * T, 512).to(dev), dc, ds)
    codes_h, scales_h = codes.cpu().numpy(), scales.cpu().numpy()
    view_c, mapped = OP.logical_view(codes_h, table, page, T)
    view_s, _ = OP.logical_view(scales_h, table, page, T)
    take = (out_rows >= 0).reshape(B, T)
    assert np.array_equal(take, mapped & (np.arange(B * T) != 5).reshape(B, T))
    dc_h, ds_h = dc.cpu().numpy().reshape(B, T, 256), ds.cpu().numpy().reshape(B, T, 32)
    assert np.array_equal(view_c[take], dc_h[take]) and np.array_equal(view_s[take], ds_h[take])
    # the oracle's pack on a few rows
    for b, p in ((0, 0), (1, 512), (2, 127)):
        c, s = OF.fp4_pack(lat[b, p:p + 1].to(torch.float64).numpy())
        assert np.array_equal(view_c[b, p], c[0]) and np.array_equal(view_s[b, p], s[0])
    # every pool row not written keeps its fill
    written = np.zeros(n_pages * page, dtype=bool)
    written[out_rows[out_rows >= 0]] = True
    assert (codes_h[~written] == 0xA5).all() and (scales_h[~written] == 0x5A).all()


@pytest.mark.parametrize("page,T", [(128, 3000), (256, 4096), (512, 1000)])
def test_index_full_paged_equals_dense_on_logical_view(page, T):
    dev = device()
    rng = np.random.default_rng(T + page)
    B = 3
    max_blocks = (T + page - 1) // page + 1
    table, n_pages = _page_table(rng, B, max_blocks, holes=[(1, 1)])
    k_pool = W.fp8_normal(81, (n_pages * page, 64))
    q = W.fp8_normal(82, (B, 64))
    view, mapped = OP.logical_view(k_pool.numpy(), table, page, T)
    limit = np.array([T - 1, T - 37, T // 3], dtype=np.int64)
    s_paged = torch.empty((B, T), dtype=torch.float32, device=dev)
    F.csa2_index_full_paged(q.to(dev), k_pool.to(dev), _dev(table, dev), page, T, s_paged,
                            row_limit=_dev(limit, dev))
    s_dense = torch.empty_like(s_paged)
    F.csa2_index_full(q.to(dev), _dev(view, dev), s_dense, row_limit=_dev(limit, dev))
    got, ref = s_paged.cpu().numpy(), s_dense.cpu().numpy()
    assert np.isneginf(got[~mapped]).all()
    assert np.array_equal(got[mapped], ref[mapped])
    # against the oracle on one row
    from oracle import indexer as OI
    exact = OI.full_scores(q[0].numpy(), view[0], int(limit[0]))
    assert np.array_equal(got[0][mapped[0]].astype(np.float32), exact[mapped[0]].astype(np.float32))


def test_index_paged_rows_sharing_sequences_and_reindex():
    # 40 query rows over 2 sequences (row_seq) and a pool of logical positions
    dev = device()
    rng = np.random.default_rng(91)
    B, R, T, page, P = 2, 40, 5000, 256, 700
    max_blocks = 20
    table, n_pages = _page_table(rng, B, max_blocks, holes=[(0, 3)])
    k_pool = W.fp8_normal(92, (n_pages * page, 64))
    q = W.fp8_normal(93, (R, 64))
    view, mapped = OP.logical_view(k_pool.numpy(), table, page, T)
    row_seq = (np.arange(R) % B).astype(np.int32)
    limit = (T - 1 - 97 * np.arange(R)).astype(np.int64)
    s_paged = torch.empty((R, T), dtype=torch.float32, device=dev)
    F.csa2_index_full_paged(q.to(dev), k_pool.to(dev), _dev(table, dev), page, T, s_paged,
                            row_seq=_dev(row_seq, dev), row_limit=_dev(limit, dev))
    s_dense = torch.empty_like(s_paged)
    F.csa2_index_full(q.to(dev), _dev(view, dev), s_dense, row_seq=_dev(row_seq, dev), row_limit=_dev(limit, dev))
    got, ref = s_paged.cpu().numpy(), s_dense.cpu().numpy()
    m = mapped[row_seq]
    assert np.isneginf(got[~m]).all() and np.array_equal(got[m], ref[m])
    pool = np.sort(rng.choice(T, size=(R, P)), axis=1).astype(np.int32)
    pool[:, -3:] = [-1, T, T + 5]                                   # invalid entries
    r_paged = torch.empty((R, P), dtype=torch.float32, device=dev)
    F.csa2_index_reindex_paged(q.to(dev), k_pool.to(dev), _dev(table, dev), page, T, _dev(pool, dev), r_paged,
                               row_seq=_dev(row_seq, dev))
    r_dense = torch.empty_like(r_paged)
    F.csa2_index_reindex(q.to(dev), _dev(view, dev), _dev(pool, dev), r_dense, row_seq=_dev(row_seq, dev))
    got, ref = r_paged.cpu().numpy(), r_dense.cpu().numpy()
    ok = (pool >= 0) & (pool < T)
    pm = np.zeros_like(ok)
    pm[ok] = m[np.nonzero(ok)[0], pool[ok]]
    assert np.isneginf(got[~pm]).all() and np.array_equal(got[pm], ref[pm])


@pytest.mark.parametrize("R,T,page,k_pool,k_top", [(4, 65536, 256, 4096, 512), (3, 3000, 128, 1024, 100),
                                                    (2, 40960, 1024, 8192, 2048)])
def test_index_full_pool_paged_equals_dense(R, T, page, k_pool, k_top):
    """Sequences shorter than the capacity leave their tail blocks unmapped:
    the paged selection equals the dense one on the logical sequences."""
    dev = device()
    rng = np.random.default_rng(R * T)
    max_blocks = T // page + 1
    lengths = [T, T - 3 * page - 77, T // 2 + 5, T // 7][:R]
    table, n_pages = _page_table(rng, R, max_blocks, lengths=lengths, page=page)
    k_pool_t = W.fp8_normal(101, (n_pages * page, 64))
    q = W.fp8_normal(102, (R, 64))
    view, _ = OP.logical_view(k_pool_t.numpy(), table, page, T)
    limit = _dev(np.array(lengths, dtype=np.int64) - 1, dev)
    out = []
    for paged in (True, False):
        s = torch.empty((R, T), dtype=torch.float32, device=dev)
        p = torch.empty((R, k_pool), dtype=torch.int32, device=dev)
        ps = torch.empty((R, k_pool), dtype=torch.float32, device=dev)
        t = torch.empty((R, k_top), dtype=torch.int32, device=dev)
        p0, t0 = torch.empty_like(p), torch.empty_like(t)
        if paged:
            F.csa2_index_full_pool_paged(q.to(dev), k_pool_t.to(dev), _dev(table, dev), page, T, s, k_pool, k_top,
                                         p, t, pool_scores=ps, row_limit=limit)
            F.csa2_index_full_pool_paged(q.to(dev), k_pool_t.to(dev), _dev(table, dev), page, T, None, k_pool, k_top,
                                         p0, t0, row_limit=limit)
        else:
            F.csa2_index_full_pool(q.to(dev), _dev(view, dev), s, k_pool, k_top, p, t, pool_scores=ps, row_limit=limit)
            p0, t0 = p, t
        torch.cuda.synchronize()
        out.append((s.cpu().numpy(), p.cpu().numpy(), torch.nan_to_num(ps, nan=7.0).cpu().numpy(), t.cpu().numpy(),
                    p0.cpu().numpy(), t0.cpu().numpy()))
    (s1, p1, ps1, t1, p10, t10), (s2, p2, ps2, t2, _, _) = out
    assert np.array_equal(s1, s2)
    assert np.array_equal(p1, p2) and np.array_equal(t1, t2) and np.array_equal(ps1, ps2)
    assert np.array_equal(p10, p1) and np.array_equal(t10, t1)
    for r in (0, R - 1):
        sh = s1[r].astype(np.float64)
        assert np.array_equal(p1[r], OT.topk(sh, k_pool)) and np.array_equal(t1[r], OT.topk(sh, k_top))


def test_index_full_pool_paged_holes_equal_separate_calls():
    # an unmapped block inside a sequence: its positions are never selected
    dev = device()
    rng = np.random.default_rng(111)
    R, T, page, k_pool, k_top = 4, 65536, 256, 4096, 512
    table, n_pages = _page_table(rng, R, T // page, holes=[(0, 0), (1, 100), (2, 255), (3, 17), (3, 18)])
    k_pool_t = W.fp8_normal(112, (n_pages * page, 64)).to(dev)
    q = W.fp8_normal(113, (R, 64)).to(dev)
    tab = _dev(table, dev)
    p1 = torch.empty((R, k_pool), dtype=torch.int32, device=dev)
    t1 = torch.empty((R, k_top), dtype=torch.int32, device=dev)
    F.csa2_index_full_pool_paged(q, k_pool_t, tab, page, T, None, k_pool, k_top, p1, t1)
    s = torch.empty((R, T), dtype=torch.float32, device=dev)
    F.csa2_index_full_paged(q, k_pool_t, tab, page, T, s)
    p2, t2 = torch.empty_like(p1), torch.empty_like(t1)
    F.csa2_topk_pool(s, k_pool, k_top, p2, t2)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(t1, t2)
    rows = _rows_of(table, page, T)
    for r in range(R):
        sel = p1[r].cpu().numpy()
        assert (rows[r, sel[sel >= 0]] >= 0).all()


def test_index_full_pool_paged_query_blocks():
    """Chunked-prefill rows (row_seq, R >= 32) over paged keys: the query-block scan translates
    each tile through the table; scores, pool and Top-K equal csa2_index_full_paged +
    csa2_topk_pool, and no selected position lies in an unmapped block."""
    dev = device()
    rng = np.random.default_rng(131)
    B, R, T, page, k_pool, k_top = 2, 48, 40960, 256, 4096, 1024
    max_blocks = T // page
    lengths = [T, T - 5 * page - 31]
    table, n_pages = _page_table(rng, B, max_blocks, lengths=lengths, page=page, holes=[(0, 9), (1, 40)])
    k_pool_t = W.fp8_normal(132, (n_pages * page, 64)).to(dev)
    q = W.fp8_normal(133, (R, 64)).to(dev)
    tab = _dev(table, dev)
    row_seq = (np.arange(R) % B).astype(np.int32)
    limit = np.array([lengths[b] - 1 - int(rng.integers(0, 9000)) for b in row_seq], dtype=np.int64)
    limit[:2] = [-1, 700]
    rs, lm = _dev(row_seq, dev), _dev(limit, dev)
    s1 = torch.empty((R, T), dtype=torch.float32, device=dev)
    p1 = torch.empty((R, k_pool), dtype=torch.int32, device=dev)
    ps1 = torch.empty((R, k_pool), dtype=torch.float32, device=dev)
    t1 = torch.empty((R, k_top), dtype=torch.int32, device=dev)
    F.csa2_index_full_pool_paged(q, k_pool_t, tab, page, T, s1, k_pool, k_top, p1, t1, pool_scores=ps1,
                                 row_seq=rs, row_limit=lm)
    p3, t3 = torch.empty_like(p1), torch.empty_like(t1)
    F.csa2_index_full_pool_paged(q, k_pool_t, tab, page, T, None, k_pool, k_top, p3, t3, row_seq=rs, row_limit=lm)
    s2 = torch.empty_like(s1)
    F.csa2_index_full_paged(q, k_pool_t, tab, page, T, s2, row_seq=rs, row_limit=lm)
    p2, ps2, t2 = torch.empty_like(p1), torch.empty_like(ps1), torch.empty_like(t1)
    F.csa2_topk_pool(s2, k_pool, k_top, p2, t2, pool_scores=ps2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal(p1, p2) and torch.equal(t1, t2) and torch.equal(p3, p2) and torch.equal(t3, t2)
    assert torch.equal(torch.nan_to_num(ps1, nan=7.0), torch.nan_to_num(ps2, nan=7.0))
    rows = _rows_of(table, page, T)
    for r in range(R):
        sel = p1[r].cpu().numpy()
        assert (rows[row_seq[r], sel[sel >= 0]] >= 0).all(), r
    assert (p1[0] == -1).all()


def test_decode_layers_paged_equals_dense_and_oracle():
    """Paged attention over a cache written by the scattered pack equals the
    dense call bit for bit; entries that fall in unmapped blocks count as
    skipped (-1) entries; one layer is checked against the oracle."""
    dev = device()
    rng = np.random.default_rng(121)
    L, B, T, H, K, S, page = 2, 3, 2500, 64, 300, 140, 128
    max_blocks = T // page + 2
    lengths = [2500, 1801, 640]
    table, n_pages = _page_table(rng, B, max_blocks, lengths=lengths, page=page, holes=[(0, 7)])
    rows = _rows_of(table, page, T)
    lat = torch.stack([W.latent_rows(123, T, chunk_index=b) for b in range(B)])
    codes = torch.zeros((n_pages * page, 256), dtype=torch.uint8, device=dev)
    scales = torch.zeros((n_pages * page, 32), dtype=torch.uint8, device=dev)
    F.csa2_fp4_pack_rows(lat.reshape(B * T, 512).to(dev), _dev(rows.reshape(-1), dev), codes, scales)
    dcodes = torch.empty((B, T, 256), dtype=torch.uint8, device=dev)
    dscales = torch.empty((B, T, 32), dtype=torch.uint8, device=dev)
    for b in range(B):
        F.csa2_fp4_pack(lat[b].to(dev), dcodes[b], dscales[b])
    q = W.bf16_normal(124, (L, B, H, 512), std=0.5).to(dev)
    swa = W.bf16_normal(125, (L, B, S, 512)).to(dev)
    start = _dev(np.array([[0, 3, 9], [5, 0, 1]], dtype=np.int32), dev)
    length = _dev(np.array([[128, 40, 0], [128, 128, 77]], dtype=np.int32), dev)
    idx = np.full((2, B, K), -1, dtype=np.int32)
    in_hole = np.array([7 * page, 7 * page + 1, 7 * page + 50, 8 * page - 1])
    for sl in range(2):
        for b in range(B):
            n = K - 11 * b - sl
            pick = rng.choice(np.setdiff1d(np.arange(lengths[b]), in_hole), n - 4, replace=False)
            idx[sl, b, :n] = np.sort(np.concatenate([pick, in_hole]))
    layer_idx = [0, 1]
    o1 = torch.empty((L, B, H, 512), dtype=torch.float32, device=dev)
    l1 = torch.empty((L, B, H), dtype=torch.float32, device=dev)
    F.csa2_sparse_swa_decode_layers_paged(q, codes, scales, _dev(table, dev), page, T, _dev(idx, dev), layer_idx,
                                          swa, start, length, SIGMA, o1, l1)
    idx_d = idx.copy()
    bad = rows[np.arange(B)[None, :, None], np.maximum(idx_d, 0)] < 0
    idx_d[bad & (idx_d >= 0)] = -1
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    F.csa2_sparse_swa_decode_layers(q, dcodes, dscales, _dev(idx_d, dev), layer_idx, swa, start, length, SIGMA, o2, l2)
    torch.cuda.synchronize()
    assert bad[0, 0].sum() >= 4
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # oracle: layer 0, sequence 0 (sparse set without the hole, plus its window)
    ref_rows = OF.fp4_unpack(*OF.fp4_pack(lat[0].to(torch.float64).numpy()))
    valid = idx_d[0, 0][idx_d[0, 0] >= 0]
    qf = q.to(torch.float64).cpu().numpy()
    o_s, l_s = OA.sparse_attend(qf[0, 0], ref_rows, valid, SIGMA)
    o_w, l_w = OA.attend(qf[0, 0], OA.window_rows(swa[0, 0].to(torch.float64).cpu().numpy(), 0, 128), SIGMA)
    o_ref, l_ref = OA.merge(o_s, l_s, o_w, l_w)
    assert_attention_close(o1[0, 0].cpu().numpy(), l1[0, 0].cpu().numpy(), o_ref, l_ref, "paged layer 0 row 0")
