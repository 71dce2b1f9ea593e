"""Pins for the oracle's sparse attention, sliding window, merge and layer roles.

Attention semantics follow the HN summary's key points (local sliding window
plus global sparse retrieval over shared KV) and the MarkTechPost retelling
(window of the last 128 tokens, paragraph 2; Full / Reindex / Reuse roles,
paragraph 3).  Pins: scipy's softmax / logsumexp as an independent dense
reference, closed-form special cases, the merge-equals-one-softmax identity,
the 128-token window bound, Reuse == Full on shared indices and sparse ==
dense when K covers the whole context.
"""
import numpy as np
import pytest
from scipy.special import logsumexp, softmax

from oracle import attention as A, pipeline as P, topk as T, formats as F


def _dense_ref(q, rows, sigma):
    s = sigma * (q @ rows.T)
    return softmax(s, axis=1) @ rows, logsumexp(s, axis=1)


def test_attend_matches_scipy_dense():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((16, 512)) * 0.5
    rows = rng.standard_normal((300, 512))
    o, lse = A.attend(q, rows, 1 / np.sqrt(128))
    o2, lse2 = _dense_ref(q, rows, 1 / np.sqrt(128))
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-13) and np.allclose(lse, lse2, rtol=1e-13)


def test_single_key_identical_rows_and_zero_query():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((4, 64))
    x = rng.standard_normal(64)
    o, lse = A.attend(q, x[None, :], 0.3)
    assert np.allclose(o, np.broadcast_to(x, o.shape), rtol=0, atol=1e-15)
    assert np.allclose(lse, 0.3 * q @ x, rtol=1e-14)
    o, lse = A.attend(q, np.tile(x, (9, 1)), 0.3)
    assert np.allclose(o, np.broadcast_to(x, o.shape), atol=1e-14)
    assert np.allclose(lse, 0.3 * q @ x + np.log(9), rtol=1e-13)
    rows = rng.standard_normal((33, 64))
    o, lse = A.attend(np.zeros((2, 64)), rows, 0.3)
    assert np.allclose(o, rows.mean(axis=0), atol=1e-14) and np.allclose(lse, np.log(33))


def test_permutation_invariance_and_padding():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((8, 32))
    cache = rng.standard_normal((100, 32))
    idx = np.array([5, 17, 40, 99, 3, -1, -1])
    o, lse = A.sparse_attend(q, cache, idx, 0.2)
    o2, lse2 = A.sparse_attend(q, cache, idx[[3, 0, 4, 2, 1]], 0.2)
    assert np.allclose(o, o2, atol=1e-14) and np.allclose(lse, lse2, atol=1e-14)
    o3, lse3 = _dense_ref(q, cache[[3, 5, 17, 40, 99]], 0.2)
    assert np.allclose(o, o3, atol=1e-13) and np.allclose(lse, lse3, atol=1e-13)


def test_empty_key_set():
    o, lse = A.attend(np.ones((3, 8)), np.zeros((0, 8)), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_merge_equals_one_softmax_over_union():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((16, 128)) * 0.5
    a = rng.standard_normal((70, 128))
    b = rng.standard_normal((40, 128)) * 3
    oa, la = A.attend(q, a, 0.1)
    ob, lb = A.attend(q, b, 0.1)
    o, lse = A.merge(oa, la, ob, lb)
    o2, lse2 = _dense_ref(q, np.concatenate([a, b]), 0.1)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-12) and np.allclose(lse, lse2, rtol=1e-13)
    # an empty side contributes nothing
    oe, le = A.attend(q, np.zeros((0, 128)), 0.1)
    o3, l3 = A.merge(oa, la, oe, le)
    assert np.array_equal(o3, oa) and np.array_equal(l3, la)


def test_window_length_and_bound():
    assert [A.window_len(t) for t in (0, 1, 126, 127, 128, 10 ** 6)] == [1, 2, 127, 128, 128, 128]
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, 64))
    state = rng.standard_normal((300, 64))
    start, length = 300 - 128, 128
    o, lse = A.attend(q, A.window_rows(state, start, length), 0.2)
    state2 = state.copy()
    state2[:start] = rng.standard_normal((start, 64)) * 100        # outside the window
    o2, lse2 = A.attend(q, A.window_rows(state2, start, length), 0.2)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    state3 = state.copy(); state3[start] += 1.0                      # inside the window
    o3, _ = A.attend(q, A.window_rows(state3, start, length), 0.2)
    assert not np.array_equal(o, o3)


def _layer_inputs(rng, T_ctx, H=4, S=128):
    import torch
    lat = torch.from_numpy(rng.standard_normal((T_ctx, 512))).to(torch.bfloat16).to(torch.float64).numpy()
    codes, scales = F.fp4_pack(lat)
    cache = F.fp4_unpack(codes, scales)
    k_idx = torch.from_numpy(rng.standard_normal((T_ctx, 64))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    def layer():
        return {"q_lat": rng.standard_normal((H, 512)) * 0.5,
                "q_idx": torch.from_numpy(rng.standard_normal(64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy(),
                "swa": rng.standard_normal((S, 512)), "swa_start": 0, "swa_len": min(S, T_ctx)}
    return cache, k_idx, layer


def test_reuse_equals_full_when_sharing_indices():
    rng = np.random.default_rng(5)
    cache, k_idx, layer = _layer_inputs(rng, 1000)
    L = layer()
    full = P.decode_layer("full", L["q_lat"], L["q_idx"], k_idx, cache, L["swa"], 0, 128, 64, 0.1)
    reuse = P.decode_layer("reuse", L["q_lat"], L["q_idx"], k_idx, cache, L["swa"], 0, 128, 64, 0.1,
                           prev_idx=full["idx"])
    assert np.array_equal(full["o"], reuse["o"]) and np.array_equal(full["lse"], reuse["lse"])


def test_sparse_equals_dense_when_k_covers_context():
    rng = np.random.default_rng(6)
    cache, k_idx, layer = _layer_inputs(rng, 300)
    L = layer()
    r = P.decode_layer("full", L["q_lat"], L["q_idx"], k_idx, cache, L["swa"], 0, 128, 512, 0.1)
    assert np.array_equal(r["idx"][:300], np.arange(300)) and np.all(r["idx"][300:] == -1)
    o, lse = _dense_ref(L["q_lat"], cache, 0.1)
    assert np.allclose(r["o_sparse"], o, atol=1e-12) and np.allclose(r["lse_sparse"], lse, atol=1e-12)


def test_reindex_with_whole_context_pool_equals_full():
    rng = np.random.default_rng(7)
    cache, k_idx, layer = _layer_inputs(rng, 500)
    L = layer()
    pool = np.arange(500)
    full = P.decode_layer("full", L["q_lat"], L["q_idx"], k_idx, cache, L["swa"], 0, 128, 50, 0.1)
    re = P.decode_layer("reindex", L["q_lat"], L["q_idx"], k_idx, cache, L["swa"], 0, 128, 50, 0.1, pool=pool)
    assert np.array_equal(full["idx"], re["idx"]) and np.array_equal(full["o"], re["o"])


def test_stack_roles_share_pool_and_indices():
    rng = np.random.default_rng(8)
    cache, k_idx, layer = _layer_inputs(rng, 3000)
    layers = [layer() for _ in range(4)]
    res = P.decode_stack(("full", "reindex", "reuse", "reuse"), layers, k_idx, cache, 64, 0.1, 256)
    pool = res[0]["pool"]
    assert pool.shape == (256,)
    assert np.array_equal(res[0]["idx"], T.topk(res[0]["scores"], 64))
    assert set(res[1]["idx"].tolist()) <= set(pool.tolist())
    assert np.array_equal(res[2]["idx"], res[1]["idx"]) and np.array_equal(res[3]["idx"], res[1]["idx"])
    # a Reindex layer's scores are exactly the Full scores of its own query on the pool
    from oracle import indexer as I
    assert np.array_equal(res[1]["scores"], I.full_scores(layers[1]["q_idx"], k_idx)[pool])


def _unabsorbed_heads(q_heads, rows, w_uk, w_uv, sigma):
    """Multi-head attention written directly: head h's keys W_UK,h x and values
    W_UV,h x for every latent row x, softmax over sigma q_h . k."""
    H = q_heads.shape[0]
    out = np.empty((H, w_uv.shape[1]))
    lse = np.empty(H)
    for h in range(H):
        k = rows @ w_uk[h].T                 # [n, 128]
        v = rows @ w_uv[h].T                 # [n, 128]
        s = sigma * (k @ q_heads[h])         # [n]
        out[h] = softmax(s) @ v
        lse[h] = logsumexp(s)
    return out, lse


def test_absorbed_equals_unabsorbed_mla():
    # associativity: (W_UK^T q) . x == q . (W_UK x) and W_UV (sum p x) == sum p (W_UV x)
    rng = np.random.default_rng(9)
    H, n = 6, 200
    q = rng.standard_normal((H, 128))
    w_uk = rng.standard_normal((H, 128, 512)) / np.sqrt(512)
    w_uv = rng.standard_normal((H, 128, 512)) / np.sqrt(512)
    rows = rng.standard_normal((n, 512))
    sigma = 1 / np.sqrt(128)
    o_lat, lse = A.attend(A.absorb(q, w_uk), rows, sigma)
    o = A.unabsorb(o_lat, w_uv)
    o2, lse2 = _unabsorbed_heads(q, rows, w_uk, w_uv, sigma)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-12) and np.allclose(lse, lse2, rtol=1e-12, atol=1e-12)


def test_absorb_orientation_one_hot_and_brute_force():
    rng = np.random.default_rng(10)
    H = 3
    w_uk = rng.standard_normal((H, 128, 512))
    w_uv = rng.standard_normal((H, 128, 512))
    # a one-hot head query picks one row of W_UK,h; a one-hot latent output one column of W_UV,h
    q = np.zeros((2, H, 128)); q[0, 1, 7] = 1.0; q[1, 2, 127] = -2.0
    ql = A.absorb(q, w_uk)
    assert ql.shape == (2, H, 512)
    assert np.array_equal(ql[0, 1], w_uk[1, 7]) and np.array_equal(ql[1, 2], -2.0 * w_uk[2, 127])
    assert np.all(ql[0, 0] == 0) and np.all(ql[1, 0] == 0)
    ol = np.zeros((1, H, 512)); ol[0, 0, 300] = 1.0
    o = A.unabsorb(ol, w_uv)
    assert o.shape == (1, H, 128) and np.array_equal(o[0, 0], w_uv[0, :, 300]) and np.all(o[0, 1:] == 0)
    # element-by-element sums on a small random case
    qs = rng.standard_normal((2, H, 128)); os_ = rng.standard_normal((2, H, 512))
    ql, oo = A.absorb(qs, w_uk), A.unabsorb(os_, w_uv)
    for r, h, c in [(0, 0, 0), (1, 2, 511), (0, 1, 260)]:
        assert np.isclose(ql[r, h, c], sum(qs[r, h, d] * w_uk[h, d, c] for d in range(128)), rtol=1e-13)
    for r, h, d in [(0, 0, 0), (1, 2, 127), (1, 1, 64)]:
        assert np.isclose(oo[r, h, d], sum(w_uv[h, d, c] * os_[r, h, c] for c in range(512)), rtol=1e-13)
