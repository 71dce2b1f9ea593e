"""Top-K and candidate-pool selection — oracle (test infrastructure only).

[HN] (key points): CSA2 layers share the same Top-K indices; a shallow
layer's candidate pool limits the deeper layers' search.  [MTP] ¶3: the
decoder Full layer's pool holds up to 16,384 positions.

Readings where the pages are silent: the K largest scores are taken, equal
scores go to the lower position, the result is listed in ascending position
order and padded with -1 when fewer than K candidates are visible (a score of
-inf marks an invisible candidate).  The pool is the min(16384, visible)
highest-scoring positions by the same rule; the Full layer's Top-K is the
top K of the pool (equal to the top K of all positions, since the pool holds
the top 16,384).
"""
import numpy as np

POOL_MAX = 16384


def topk(scores: np.ndarray, k: int, index_map: np.ndarray = None) -> np.ndarray:
    """Indices of the k largest finite scores, ascending, -1 padded to length k.

    scores: 1-D array (float64 or int).  Candidates with score -inf or NaN are
    not visible.  index_map: optional array mapping candidate slot -> position
    (the returned values are then positions); ties break on the mapped
    position.
    """
    s = np.asarray(scores)
    n = s.shape[0]
    slots = np.arange(n)
    pos = slots if index_map is None else np.asarray(index_map, dtype=np.int64)
    if np.issubdtype(s.dtype, np.floating):
        visible = np.isfinite(s) | (s == np.inf)
    else:
        visible = np.ones(n, dtype=bool)
    if index_map is not None:
        visible &= pos >= 0
    cand = slots[visible]
    # primary key: larger score first; secondary: lower position first
    order = np.lexsort((pos[cand], -s[cand].astype(np.float64)))
    take = cand[order[:min(k, cand.shape[0])]]
    out = np.sort(pos[take])
    return np.concatenate([out, np.full(k - out.shape[0], -1, dtype=np.int64)]).astype(np.int64)


def topk_with_scores(scores: np.ndarray, k: int, index_map: np.ndarray = None):
    """Like topk, plus the selected scores (NaN in padded slots), in output order."""
    idx = topk(scores, k, index_map)
    s = np.asarray(scores, dtype=np.float64)
    if index_map is None:
        vals = np.where(idx >= 0, s[np.clip(idx, 0, None)], np.nan)
    else:
        im = np.asarray(index_map, dtype=np.int64)
        slot_of = {int(p): i for i, p in enumerate(im) if p >= 0}
        vals = np.array([s[slot_of[int(p)]] if p >= 0 else np.nan for p in idx])
    return idx, vals


def candidate_pool(scores: np.ndarray, pool_size: int = POOL_MAX) -> np.ndarray:
    """Full-layer candidate pool: the top min(pool_size, visible) positions, ascending."""
    return topk(scores, pool_size)
