"""One CSA2 decode layer in Full / Reindex / Reuse role — oracle (test infrastructure only).

[MTP] ¶3: layers take Full, Reindex or Reuse roles; some build fresh indices,
others rescore a shared candidate set, many reuse what came before; the
decoder Full layer's candidate pool holds up to 16,384 positions.  [HN] (key
points): several layers share the same main KV and Top-K indices.  [FO] (What
you will learn): the modes share global KV and sparse selections while queries
and sliding-window state stay per layer.

Per layer and sequence:
  Full     scores every visible position; pool = top min(P, visible) of them
           (only when a later layer rescores it); idx = top K of the pool
           (the same set as the top K of all positions);
  Reindex  scores only the pool positions with its own indexer query; idx = the
           top K of those, mapped back to positions;
  Reuse    idx = the idx of the nearest preceding Full or Reindex layer;
then sparse attention over idx, window attention over the layer's last
min(128, t+1) rows, merged into one softmax.
"""
import numpy as np
from . import indexer, topk as tk, attention as at


def decode_layer(mode: str, q_lat, q_idx, k_idx, cache_rows, swa, swa_start, swa_len,
                 k: int, sigma: float, pool_size: int = 0, pool=None, prev_idx=None,
                 limit: int = None):
    """Run one layer for one query row.

    q_lat [H, C] float64; q_idx uint8 [64]; k_idx uint8 [T, 64];
    cache_rows [T, C] float64 (dequantised FP4 rows); swa [S, C] float64.
    Returns a dict with 'scores', 'pool', 'idx', 'o_sparse', 'lse_sparse',
    'o_swa', 'lse_swa', 'o', 'lse'.
    """
    out = {"scores": None, "pool": pool}
    if mode == "full":
        s = indexer.full_scores(q_idx, k_idx, limit)
        out["scores"] = s
        if pool_size:
            out["pool"] = tk.candidate_pool(s, pool_size)
            pool_scores = np.where(out["pool"] >= 0, s[np.clip(out["pool"], 0, None)], -np.inf)
            idx = tk.topk(pool_scores, k, index_map=out["pool"])
        else:
            idx = tk.topk(s, k)
    elif mode == "reindex":
        if pool is None:
            raise ValueError("reindex layer needs the candidate pool of a Full layer")
        s = indexer.reindex_scores(q_idx, k_idx, pool)
        out["scores"] = s
        idx = tk.topk(s, k, index_map=pool)
    elif mode == "reuse":
        if prev_idx is None:
            raise ValueError("reuse layer needs the indices of a preceding layer")
        idx = np.asarray(prev_idx)
    else:
        raise ValueError(mode)
    out["idx"] = idx
    o_s, l_s = at.sparse_attend(q_lat, cache_rows, idx, sigma)
    o_w, l_w = at.attend(q_lat, at.window_rows(swa, swa_start, swa_len), sigma)
    o, lse = at.merge(o_s, l_s, o_w, l_w)
    out.update(o_sparse=o_s, lse_sparse=l_s, o_swa=o_w, lse_swa=l_w, o=o, lse=lse)
    return out


def decode_stack(modes, layers, k_idx, cache_rows, k: int, sigma: float, pool_size: int,
                 limit: int = None):
    """Run a stack of layers for one query row.

    layers: list of dicts with 'q_lat', 'q_idx', 'swa', 'swa_start', 'swa_len'.
    Returns the list of per-layer result dicts.
    """
    results = []
    pool = None
    prev_idx = None
    needs_pool = "reindex" in modes
    for mode, L in zip(modes, layers):
        r = decode_layer(mode, L["q_lat"], L["q_idx"], k_idx, cache_rows, L["swa"],
                         L["swa_start"], L["swa_len"], k, sigma,
                         pool_size=pool_size if (mode == "full" and needs_pool) else 0,
                         pool=pool, prev_idx=prev_idx, limit=limit)
        if mode == "full" and r["pool"] is not None:
            pool = r["pool"]
        prev_idx = r["idx"]
        results.append(r)
    return results
