"""GPU parity: indexer scoring (Full / Reindex) and Top-K selection vs the oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import indexer as OI, topk as OT, formats as OF
import fp4_sparse_attention_amd as F
from gpu_common import device, np_u8, assert_topk_swap_rule

pytestmark = pytest.mark.gpu


def _score_bound(q, k):
    """fp32-accumulation bound per score: 64 * 2^-24 * sum |q_d k_d|."""
    qa = np.abs(OF.e4m3_decode(q))
    ka = np.abs(OF.e4m3_decode(k))
    return (ka @ qa.T if qa.ndim == 2 else ka @ qa) * 64 * 2.0 ** -24


@pytest.mark.parametrize("B,T", [(1, 4096), (3, 100), (2, 4), (1, 4100)])
def test_index_full_scores(B, T):
    dev = device()
    k = torch.stack([W.fp8_normal(7, (T, 64), chunk_index=b) for b in range(B)])
    q = W.fp8_normal(8, (B, 64))
    scores = torch.empty((B, T), dtype=torch.float32, device=dev)
    F.csa2_index_full(q.to(dev), k.to(dev), scores)
    got = scores.cpu().numpy().astype(np.float64)
    n_exact = 0
    for b in range(B):
        exact = OI.full_scores(q[b].numpy(), k[b].numpy())
        bound = _score_bound(q[b].numpy(), k[b].numpy())
        assert np.all(np.abs(got[b] - exact) <= bound + 1e-30), (b, np.max(np.abs(got[b] - exact)))
        # the f16 matrix path sums exactly and rounds once: bit-equal to fp32(exact)
        assert np.array_equal(got[b].astype(np.float32), exact.astype(np.float32)), b


def test_index_scores_bound_on_wide_range_keys():
    # keys spanning the whole E4M3 range (subnormals to 448): running sums need far
    # more than 24 bits; the two 32-channel steps round into fp32, and on this
    # distribution the error stays within 2^-22 * sum |q_d k_d|
    dev = device()
    g = torch.Generator().manual_seed(17)
    T = 8192
    x = torch.randn((1, T, 64), generator=g) * torch.exp2(torch.randint(-10, 8, (1, T, 64), generator=g).float())
    k = x.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    q = (torch.randn((1, 64), generator=g) * 4).to(torch.float8_e4m3fn).view(torch.uint8)
    scores = torch.empty((1, T), dtype=torch.float32, device=dev)
    F.csa2_index_full(q.to(dev), k.to(dev), scores)
    exact = OI.full_scores(q[0].numpy(), k[0].numpy())
    got = scores[0].cpu().numpy().astype(np.float64)
    bound = _score_bound(q[0].numpy(), k[0].numpy()) / 16       # 64 * 2^-24 / 16 = 2^-22
    err = np.abs(got - exact)
    assert np.all(err <= bound), float((err / bound).max())
    print(f"exactly rounded: {np.mean(got == exact.astype(np.float32)):.4f}")


def test_index_full_causal_rows_and_row_seq():
    # 70 query rows over 2 sequences: row r belongs to sequence r % 2 and sees positions <= limit[r]
    dev = device()
    T, R = 1000, 70
    k = torch.stack([W.fp8_normal(9, (T, 64), chunk_index=b) for b in range(2)])
    q = W.fp8_normal(10, (R, 64))
    row_seq = torch.arange(R, dtype=torch.int32) % 2
    limit = torch.from_numpy(np.random.default_rng(0).integers(-1, T + 5, R)).to(torch.int64)
    scores = torch.empty((R, T), dtype=torch.float32, device=dev)
    F.csa2_index_full(q.to(dev), k.to(dev), scores, row_seq=row_seq.to(dev), row_limit=limit.to(dev))
    got = scores.cpu().numpy()
    for r in range(R):
        b = int(row_seq[r])
        exact = OI.full_scores(q[r].numpy(), k[b].numpy(), limit=int(limit[r]))
        fin = np.isfinite(exact)
        assert np.array_equal(np.isneginf(got[r]), ~fin), r
        assert np.array_equal(got[r][fin], exact[fin].astype(np.float32)), r


def test_index_prefill_block_rows_same_sequence():
    # 64 causal query rows of one sequence (the chunked-prefill layout)
    dev = device()
    T, R = 2048, 64
    k = W.fp8_normal(11, (1, T, 64))
    q = W.fp8_normal(12, (R, 64))
    row_seq = torch.zeros(R, dtype=torch.int32)
    limit = torch.arange(T - R, T, dtype=torch.int64)
    scores = torch.empty((R, T), dtype=torch.float32, device=dev)
    F.csa2_index_full(q.to(dev), k.to(dev), scores, row_seq=row_seq.to(dev), row_limit=limit.to(dev))
    got = scores.cpu().numpy()
    for r in range(R):
        exact = OI.full_scores(q[r].numpy(), k[0].numpy(), limit=int(limit[r]))
        fin = np.isfinite(exact)
        assert np.array_equal(np.isneginf(got[r]), ~fin)
        assert np.array_equal(got[r][fin], exact[fin].astype(np.float32)), r


def test_reindex_matches_full_bitwise_on_pool():
    dev = device()
    B, T, P = 3, 3000, 520
    k = torch.stack([W.fp8_normal(13, (T, 64), chunk_index=b) for b in range(B)]).to(dev)
    q = W.fp8_normal(14, (B, 64)).to(dev)
    full = torch.empty((B, T), dtype=torch.float32, device=dev)
    F.csa2_index_full(q, k, full)
    rng = np.random.default_rng(1)
    pool = np.stack([np.sort(rng.choice(T, P, replace=False)) for _ in range(B)]).astype(np.int32)
    pool[:, -7:] = -1
    pool[1, 3] = T + 5                      # out of range -> -inf
    pt = torch.from_numpy(pool).to(dev)
    re = torch.empty((B, P), dtype=torch.float32, device=dev)
    F.csa2_index_reindex(q, k, pt, re)
    got = re.cpu().numpy()
    fullh = full.cpu().numpy()
    for b in range(B):
        for p in range(P):
            pos = pool[b, p]
            if 0 <= pos < T:
                assert got[b, p] == fullh[b, pos]
            else:
                assert np.isneginf(got[b, p])


def _synthetic_scores(rng, R, N, tie_frac=0.3, ninf_frac=0.05):
    s = rng.standard_normal((R, N)).astype(np.float32) * 8
    ties = rng.random((R, N)) < tie_frac
    s[ties] = np.round(s[ties])                     # many exact ties
    s[rng.random((R, N)) < ninf_frac] = -np.inf
    s[rng.random((R, N)) < 0.01] = np.nan
    return s


@pytest.mark.parametrize("R,N,k", [(1, 4096, 256), (5, 1000, 64), (3, 12, 20), (2, 65536, 16384),
                                   (4, 131072, 2048), (1, 8, 1)])
def test_topk_bit_exact(R, N, k):
    dev = device()
    rng = np.random.default_rng(N + k)
    s = _synthetic_scores(rng, R, N)
    st = torch.from_numpy(s).to(dev)
    idx = torch.empty((R, k), dtype=torch.int32, device=dev)
    so = torch.empty((R, k), dtype=torch.float32, device=dev)
    F.csa2_topk(st, k, idx, score_out=so)
    gi, gs = idx.cpu().numpy(), so.cpu().numpy()
    for r in range(R):
        ri, rs = OT.topk_with_scores(s[r].astype(np.float64), k)
        assert np.array_equal(gi[r], ri), r
        assert np.array_equal(np.isnan(gs[r]), np.isnan(rs))
        assert np.array_equal(gs[r][~np.isnan(rs)], rs[~np.isnan(rs)].astype(np.float32))


def test_topk_all_invisible_and_strided_rows():
    dev = device()
    s = np.full((2, 64), -np.inf, dtype=np.float32)
    s[1, 10] = 1.0
    big = torch.full((2, 80), 5.0, dtype=torch.float32, device=dev)
    big[:, :64] = torch.from_numpy(s).to(dev)
    idx = torch.empty((2, 4), dtype=torch.int32, device=dev)
    F.csa2_topk(big[:, :64], 4, idx)
    assert idx.cpu().tolist() == [[-1, -1, -1, -1], [10, -1, -1, -1]]


def test_topk_with_index_map_and_padding():
    dev = device()
    rng = np.random.default_rng(3)
    R, N, k = 3, 4000, 300
    s = _synthetic_scores(rng, R, N, tie_frac=0.5)
    pos = np.stack([np.sort(rng.choice(10 ** 6, N, replace=False)) for _ in range(R)]).astype(np.int32)
    pos[:, -50:] = -1
    idx = torch.empty((R, k), dtype=torch.int32, device=dev)
    F.csa2_topk(torch.from_numpy(s).to(dev), k, idx, index_map=torch.from_numpy(pos).to(dev))
    gi = idx.cpu().numpy()
    for r in range(R):
        assert np.array_equal(gi[r], OT.topk(s[r].astype(np.float64), k, index_map=pos[r]))


def test_full_scores_then_topk_swap_rule():
    """Top-K of the GPU's fp32 scores vs Top-K of the exact scores (1e-6 swap rule)."""
    dev = device()
    B, T, K = 2, 20000, 256
    k = torch.stack([W.fp8_normal(15, (T, 64), chunk_index=b) for b in range(B)])
    q = W.fp8_normal(16, (B, 64))
    scores = torch.empty((B, T), dtype=torch.float32, device=dev)
    F.csa2_index_full(q.to(dev), k.to(dev), scores)
    idx = torch.empty((B, K), dtype=torch.int32, device=dev)
    F.csa2_topk(scores, K, idx)
    for b in range(B):
        exact = OI.full_scores(q[b].numpy(), k[b].numpy())
        ref = OT.topk(exact, K)
        assert_topk_swap_rule(idx[b].cpu().numpy(), ref, lambda p: exact[p], f"row {b}")


@pytest.mark.parametrize("R,N,k", [(2, 32768, 2048), (3, 32772, 100), (8, 1 << 20, 16384)])
def test_topk_paths_boundaries_bit_exact(R, N, k):
    # 32768 = largest LDS-resident row; 32772 and 1M take the candidate-compaction path
    dev = device()
    rng = np.random.default_rng(N % 1000 + k)
    s = _synthetic_scores(rng, R, N)
    idx = torch.empty((R, k), dtype=torch.int32, device=dev)
    so = torch.empty((R, k), dtype=torch.float32, device=dev)
    F.csa2_topk(torch.from_numpy(s).to(dev), k, idx, score_out=so)
    gi, gs = idx.cpu().numpy(), so.cpu().numpy()
    for r in range(R):
        ri, rs = OT.topk_with_scores(s[r].astype(np.float64), k)
        assert np.array_equal(gi[r], ri), r
        assert np.array_equal(gs[r][~np.isnan(rs)], rs[~np.isnan(rs)].astype(np.float32))


@pytest.mark.parametrize("N", [4096, 8192, 16384, 32768, 65536])
@pytest.mark.parametrize("kind", ["k1000", "cut", "all"])
def test_topk_massive_ties(N, kind):
    # few distinct values: the k-th key is shared by thousands of slots and,
    # for "cut" and "all", larger keys are selected beside the tied ones;
    # ties go to the lowest slots.  Covers every register-layout width of the
    # one-workgroup path (N <= 32768) and the long-row path.
    dev = device()
    rng = np.random.default_rng(N)
    R = 3
    k = {"k1000": 1000, "cut": N * 3 // 8, "all": N}[kind]
    s = rng.integers(0, 4, (R, N)).astype(np.float32)
    s[1] = 7.0                                           # every slot equal
    s[2, ::3] = -np.inf
    idx = torch.empty((R, k), dtype=torch.int32, device=dev)
    F.csa2_topk(torch.from_numpy(s).to(dev), k, idx)
    gi = idx.cpu().numpy()
    for r in range(R):
        assert np.array_equal(gi[r], OT.topk(s[r].astype(np.float64), k)), r
    assert gi[1].tolist() == list(range(k))


def test_topk_multipass_path_sampled_rows():
    # R * N * 8 bytes above the candidate budget -> three full histogram passes
    dev = device()
    R, N, k = 1040, 131072, 2048
    g = torch.Generator(device=dev).manual_seed(5)
    s = torch.randn((R, N), generator=g, device=dev) * 8
    s[:, ::7] = torch.round(s[:, ::7])
    idx = torch.empty((R, k), dtype=torch.int32, device=dev)
    F.csa2_topk(s, k, idx)
    for r in (0, 519, R - 1):
        row = s[r].cpu().numpy().astype(np.float64)
        assert np.array_equal(idx[r].cpu().numpy(), OT.topk(row, k)), r


@pytest.mark.parametrize("R,N,k_pool,k_top,ties", [
    (8, 16384, 4096, 512, False),          # one-workgroup path (two selections in one launch)
    (5, 3000, 700, 700, True),             # one-workgroup path, k_top == k_pool (one selection, two outputs)
    (4, 20000, 2048, 100, True),           # one-workgroup path, heavy ties in both selections
    (4, 131072, 16384, 2048, False),       # candidate-list path, both selections from one list
    (3, 65536, 20000, 20000, True),        # k_top == k_pool, heavy ties
    (2, 1 << 20, 16384, 2048, False),      # the 1M-context pool shape
])
def test_topk_pool_matches_two_selections(R, N, k_pool, k_top, ties):
    dev = device()
    g = torch.Generator(device=dev).manual_seed(N + k_pool)
    if ties:
        s = torch.randint(0, 6, (R, N), device=dev, generator=g).to(torch.float32)
        s[0, ::5] = -float("inf")
    else:
        s = torch.randn((R, N), device=dev, generator=g) * 8
    pool = torch.empty((R, k_pool), dtype=torch.int32, device=dev)
    pool_s = torch.empty((R, k_pool), dtype=torch.float32, device=dev)
    top = torch.empty((R, k_top), dtype=torch.int32, device=dev)
    F.csa2_topk_pool(s, k_pool, k_top, pool, top, pool_scores=pool_s)
    sh = s.cpu().numpy().astype(np.float64)
    gp, gs, gt = pool.cpu().numpy(), pool_s.cpu().numpy(), top.cpu().numpy()
    for r in range(R):
        ref_pool = OT.topk(sh[r], k_pool)
        assert np.array_equal(gp[r], ref_pool), r
        valid = ref_pool >= 0
        assert np.array_equal(gs[r][valid], sh[r][ref_pool[valid]].astype(np.float32)), r
        assert np.all(np.isnan(gs[r][~valid]))
        assert np.array_equal(gt[r], OT.topk(sh[r], k_top)), r


def test_topk_pool_with_index_map_and_long_rows_path():
    # long rows beyond the candidate-list budget (two multipass selections), sampled rows
    dev = device()
    R, N, k_pool, k_top = 520, 131072, 4096, 256
    g = torch.Generator(device=dev).manual_seed(77)
    s = torch.randn((R, N), device=dev, generator=g)
    imap = torch.arange(N, dtype=torch.int32, device=dev).repeat(R, 1) * 3 + 1
    imap[:, 7::11] = -1
    pool = torch.empty((R, k_pool), dtype=torch.int32, device=dev)
    top = torch.empty((R, k_top), dtype=torch.int32, device=dev)
    F.csa2_topk_pool(s, k_pool, k_top, pool, top, index_map=imap)
    for r in (0, 259, 519):
        sh = s[r].cpu().numpy().astype(np.float64)
        mh = imap[r].cpu().numpy()
        assert np.array_equal(pool[r].cpu().numpy(), OT.topk(sh, k_pool, index_map=mh)), r
        assert np.array_equal(top[r].cpu().numpy(), OT.topk(sh, k_top, index_map=mh)), r


@pytest.mark.parametrize("R,T,k_pool,k_top", [(8, 1 << 20, 16384, 2048), (3, 8192, 2048, 256), (2, 65540, 4000, 4000),
                                             (64, 131072, 2048, 2048)])
def test_index_full_pool_equals_separate_calls(R, T, k_pool, k_top):
    """Scores, pool (with scores) and Top-K of the fused call are bit-identical to
    csa2_index_full followed by csa2_topk_pool (long rows: the scoring pass builds
    the selection's histogram; short rows: the two calls)."""
    dev = device()
    k = torch.stack([W.fp8_normal(61, (T, 64), device=dev, chunk_index=b) for b in range(R)])
    q = W.fp8_normal(62, (R, 64), device=dev)
    s1 = torch.empty((R, T), dtype=torch.float32, device=dev)
    p1 = torch.empty((R, k_pool), dtype=torch.int32, device=dev)
    ps1 = torch.empty((R, k_pool), dtype=torch.float32, device=dev)
    t1 = torch.empty((R, k_top), dtype=torch.int32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in ev:
        e.record()
    F.csa2_index_full_pool(q, k, s1, k_pool, k_top, p1, t1, pool_scores=ps1, scan_events=ev)
    s2 = torch.empty_like(s1)
    p2, ps2, t2 = torch.empty_like(p1), torch.empty_like(ps1), torch.empty_like(t1)
    F.csa2_index_full(q, k, s2)
    F.csa2_topk_pool(s2, k_pool, k_top, p2, t2, pool_scores=ps2)
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) > 0.0
    assert torch.equal(s1, s2)
    assert torch.equal(p1, p2) and torch.equal(t1, t2)
    assert torch.equal(torch.nan_to_num(ps1, nan=7.0), torch.nan_to_num(ps2, nan=7.0))
    # without a scores output: the same selections
    p3, ps3, t3 = torch.empty_like(p1), torch.empty_like(ps1), torch.empty_like(t1)
    F.csa2_index_full_pool(q, k, None, k_pool, k_top, p3, t3, pool_scores=ps3)
    torch.cuda.synchronize()
    assert torch.equal(p1, p3) and torch.equal(t1, t3)
    assert torch.equal(torch.nan_to_num(ps1, nan=7.0), torch.nan_to_num(ps3, nan=7.0))
    # and against the oracle on one row
    sh = s1[0].cpu().numpy().astype(np.float64)
    assert np.array_equal(p1[0].cpu().numpy(), OT.topk(sh, k_pool))
    assert np.array_equal(t1[0].cpu().numpy(), OT.topk(sh, k_top))


@pytest.mark.parametrize("R,B,T,k_pool,k_top", [(96, 3, 40000, 4000, 1000), (64, 1, 65536, 2048, 2048),
                                                 (40, 2, 131072, 16384, 2048), (40, 40, 33000, 1024, 128)])
def test_index_full_pool_query_blocks_equal_separate_calls(R, B, T, k_pool, k_top):
    """Chunked-prefill rows (row_seq given, R >= 32): the query-block scan with 1,024-position
    candidate blocks gives the scores, pool (with scores) and Top-K of csa2_index_full +
    csa2_topk_pool bit for bit: interleaved sequences, a partial row group, a ragged last block,
    causal limits, an empty row, rows shorter than either selection, a limit beyond T, and a
    row group whose 32 rows all belong to different sequences (one pass per sequence)."""
    dev = device()
    k = torch.stack([W.fp8_normal(81, (T, 64), device=dev, chunk_index=b) for b in range(B)])
    q = W.fp8_normal(82, (R, 64), device=dev)
    row_seq = (torch.arange(R, dtype=torch.int32) % B).to(dev)
    rng = np.random.default_rng(R + T)
    lim_h = (T - 1 - rng.integers(0, T // 3, R)).astype(np.int64)
    lim_h[:4] = [-1, 100, k_pool + 5, T + 7]
    lim = torch.from_numpy(lim_h).to(dev)
    s1 = torch.empty((R, T), dtype=torch.float32, device=dev)
    p1 = torch.empty((R, k_pool), dtype=torch.int32, device=dev)
    ps1 = torch.empty((R, k_pool), dtype=torch.float32, device=dev)
    t1 = torch.empty((R, k_top), dtype=torch.int32, device=dev)
    F.csa2_index_full_pool(q, k, s1, k_pool, k_top, p1, t1, pool_scores=ps1, row_seq=row_seq, row_limit=lim)
    s2 = torch.empty_like(s1)
    p2, ps2, t2 = torch.empty_like(p1), torch.empty_like(ps1), torch.empty_like(t1)
    F.csa2_index_full(q, k, s2, row_seq=row_seq, row_limit=lim)
    F.csa2_topk_pool(s2, k_pool, k_top, p2, t2, pool_scores=ps2)
    p3, ps3, t3 = torch.empty_like(p1), torch.empty_like(ps1), torch.empty_like(t1)
    F.csa2_index_full_pool(q, k, None, k_pool, k_top, p3, t3, pool_scores=ps3, row_seq=row_seq, row_limit=lim)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    for p, ps, t in ((p1, ps1, t1), (p3, ps3, t3)):
        assert torch.equal(p, p2) and torch.equal(t, t2)
        assert torch.equal(torch.nan_to_num(ps, nan=7.0), torch.nan_to_num(ps2, nan=7.0))
    assert (p1[0] == -1).all() and (t1[0] == -1).all()
    assert (p1[1, :101] >= 0).all() and (p1[1, 101:] == -1).all()
    # two rows against the oracle's exact scores (bit-equal to the GPU's for unit-normal keys)
    for r in (2, R - 1):
        b = r % B
        exact = OI.full_scores(np_u8(q[r]), np_u8(k[b]), limit=int(lim_h[r]))
        sh = exact.astype(np.float32).astype(np.float64)
        assert np.array_equal(p1[r].cpu().numpy(), OT.topk(sh, k_pool)), r
        assert np.array_equal(t1[r].cpu().numpy(), OT.topk(sh, k_top)), r


def test_index_full_pool_prefill_shape_equals_scores_first():
    """4,096 causal rows over 262,144 positions, Top-2,048 (chunked prefill): the streaming
    selection over the query-block scan equals csa2_index_full + csa2_topk on every row."""
    dev = device()
    R, T, K = 4096, 262144, 2048
    k = W.fp8_normal(93, (1, T, 64), device=dev)
    q = W.fp8_normal(94, (R, 64), device=dev)
    row_seq = torch.zeros(R, dtype=torch.int32, device=dev)
    lim = torch.arange(T - R, T, dtype=torch.int64, device=dev)
    pool = torch.empty((R, K), dtype=torch.int32, device=dev)
    top = torch.empty((R, K), dtype=torch.int32, device=dev)
    F.csa2_index_full_pool(q, k, None, K, K, pool, top, row_seq=row_seq, row_limit=lim)
    s = torch.empty((R, T), dtype=torch.float32, device=dev)
    F.csa2_index_full(q, k, s, row_seq=row_seq, row_limit=lim)
    ref = torch.empty((R, K), dtype=torch.int32, device=dev)
    F.csa2_topk(s, K, ref)
    torch.cuda.synchronize()
    del s
    assert torch.equal(top, ref) and torch.equal(pool, ref)


def _stream_case_keys(kind, R, T, q, dev, S=4096):
    """Index keys for the streaming selection's special cases (uint8 E4M3 codes [R, T, 64])."""
    g = torch.Generator(device="cpu").manual_seed(71)
    small = ((torch.randint(0, 256, (R, T, 64), generator=g, dtype=torch.uint8) & 0x87) | 0x08)
    if kind == "fallback":
        # strided positions carry the query itself (large positive score), the rest tiny keys:
        # the sampled threshold lands above the k-th score and the row is rebuilt from its scores
        k = small.clone()
        i = torch.arange(S, dtype=torch.int64)
        pos = ((2 * i + 1) * T) // (2 * S)
        k[:, pos, :] = q.cpu()[:, None, :]
        return k.to(dev)
    if kind == "ties_all":
        return q.cpu()[:, None, :].expand(R, T, 64).contiguous().to(dev)
    if kind in ("ties_few", "ties_256"):
        n = 16 if kind == "ties_few" else 256
        pal = torch.randint(0, 256, (n, 64), generator=g, dtype=torch.uint8)
        pal[(pal & 0x7F) == 0x7F] = 0
        return pal[torch.randint(0, n, (R, T), generator=g)].to(dev)
    if kind == "nan_keys":
        k = torch.stack([W.fp8_normal(73, (T, 64), chunk_index=b) for b in range(R)])
        nan_rows = torch.rand((R, T), generator=g) < 0.2
        k[nan_rows, 5] = 0x7F
        return k.to(dev)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["fallback", "ties_all", "ties_few", "ties_256", "nan_keys", "limits"])
def test_index_full_pool_streaming_cases(kind):
    """The streaming pool selection (sampled threshold, block-ordered candidates from the scan,
    gather / finish / write) gives the same pool, pool scores and Top-K as csa2_index_full +
    csa2_topk_pool, with and without a scores output, and the oracle's selection on sampled rows:
    when the threshold misses (the row is rebuilt), under massive ties (a boundary bin larger than
    its list; ties go to the lowest positions), with NaN keys and with row limits (empty rows,
    rows shorter than the pool)."""
    dev = device()
    R, T, k_pool, k_top = 4, 131072, 16384, 2048
    q = W.fp8_normal(72, (R, 64), device=dev)
    lim = None
    if kind == "limits":
        k = torch.stack([W.fp8_normal(74, (T, 64), device=dev, chunk_index=b) for b in range(R)])
        lim = torch.tensor([T - 1, 5000, -1, 40000], dtype=torch.int64, device=dev)
    else:
        k = _stream_case_keys(kind, R, T, q, dev)
    s1 = torch.empty((R, T), dtype=torch.float32, device=dev)
    p1 = torch.empty((R, k_pool), dtype=torch.int32, device=dev)
    ps1 = torch.empty((R, k_pool), dtype=torch.float32, device=dev)
    t1 = torch.empty((R, k_top), dtype=torch.int32, device=dev)
    F.csa2_index_full_pool(q, k, s1, k_pool, k_top, p1, t1, pool_scores=ps1, row_limit=lim)
    s2 = torch.empty_like(s1)
    p2, ps2, t2 = torch.empty_like(p1), torch.empty_like(ps1), torch.empty_like(t1)
    F.csa2_index_full(q, k, s2, row_limit=lim)
    F.csa2_topk_pool(s2, k_pool, k_top, p2, t2, pool_scores=ps2)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(s1, nan=7.0), torch.nan_to_num(s2, nan=7.0))
    assert torch.equal(s1.isnan(), s2.isnan())
    assert torch.equal(p1, p2) and torch.equal(t1, t2)
    assert torch.equal(torch.nan_to_num(ps1, nan=7.0), torch.nan_to_num(ps2, nan=7.0))
    for r in (0, R - 1):
        sh = s1[r].cpu().numpy().astype(np.float64)
        assert np.array_equal(p1[r].cpu().numpy(), OT.topk(sh, k_pool))
        assert np.array_equal(t1[r].cpu().numpy(), OT.topk(sh, k_top))
    # without a scores output (the rebuild and overflow paths then rescore or read candidates only)
    p3, ps3, t3 = torch.empty_like(p1), torch.empty_like(ps1), torch.empty_like(t1)
    F.csa2_index_full_pool(q, k, None, k_pool, k_top, p3, t3, pool_scores=ps3, row_limit=lim)
    torch.cuda.synchronize()
    assert torch.equal(p1, p3) and torch.equal(t1, t3)
    assert torch.equal(torch.nan_to_num(ps1, nan=7.0), torch.nan_to_num(ps3, nan=7.0))
    if kind == "ties_all":
        assert np.array_equal(p1.cpu().numpy(), np.tile(np.arange(k_pool, dtype=np.int32), (R, 1)))
    if kind == "limits":
        assert (p1[2] == -1).all() and (t1[2] == -1).all()
        assert (p1[1, :5001] >= 0).all() and (p1[1, 5001:] == -1).all()


@pytest.mark.parametrize("kind", ["fallback", "ties_all", "ties_256", "nan_keys"])
def test_index_full_pool_query_blocks_streaming_cases(kind):
    """The streaming selection's special cases through the query-block scan (64 rows over 2
    sequences, each row with its sequence's query, so that what misleads one row's sample
    misleads all of them): threshold misses, massive ties, NaN keys; same outputs as
    csa2_index_full + csa2_topk_pool, with and without a scores output."""
    dev = device()
    B, R, T, k_pool, k_top = 2, 64, 131072, 16384, 2048
    qb = W.fp8_normal(72, (B, 64), device=dev)
    k = _stream_case_keys(kind, B, T, qb, dev)
    row_seq = (torch.arange(R, dtype=torch.int32) % B).to(dev)
    q = qb[row_seq.long()].contiguous()
    s1 = torch.empty((R, T), dtype=torch.float32, device=dev)
    p1 = torch.empty((R, k_pool), dtype=torch.int32, device=dev)
    ps1 = torch.empty((R, k_pool), dtype=torch.float32, device=dev)
    t1 = torch.empty((R, k_top), dtype=torch.int32, device=dev)
    F.csa2_index_full_pool(q, k, s1, k_pool, k_top, p1, t1, pool_scores=ps1, row_seq=row_seq)
    s2 = torch.empty_like(s1)
    p2, ps2, t2 = torch.empty_like(p1), torch.empty_like(ps1), torch.empty_like(t1)
    F.csa2_index_full(q, k, s2, row_seq=row_seq)
    F.csa2_topk_pool(s2, k_pool, k_top, p2, t2, pool_scores=ps2)
    p3, ps3, t3 = torch.empty_like(p1), torch.empty_like(ps1), torch.empty_like(t1)
    F.csa2_index_full_pool(q, k, None, k_pool, k_top, p3, t3, pool_scores=ps3, row_seq=row_seq)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(s1, nan=7.0), torch.nan_to_num(s2, nan=7.0))
    assert torch.equal(s1.isnan(), s2.isnan())
    for p, ps, t in ((p1, ps1, t1), (p3, ps3, t3)):
        assert torch.equal(p, p2) and torch.equal(t, t2)
        assert torch.equal(torch.nan_to_num(ps, nan=7.0), torch.nan_to_num(ps2, nan=7.0))
    sh = s1[R - 1].cpu().numpy().astype(np.float64)
    assert np.array_equal(p1[R - 1].cpu().numpy(), OT.topk(sh, k_pool))
    assert np.array_equal(t1[R - 1].cpu().numpy(), OT.topk(sh, k_top))
    if kind == "ties_all":
        assert np.array_equal(p1.cpu().numpy(), np.tile(np.arange(k_pool, dtype=np.int32), (R, 1)))
