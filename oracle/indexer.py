"""Indexer scoring — oracle (test infrastructure only).

[MTP] ¶3: CSA2 layers take a Full, Reindex or Reuse role.  A Full layer builds
fresh indices over the context; a Reindex layer rescores a shared candidate
set; in the decoder the Full layer's candidate pool holds up to 16,384
positions so later layers score a bounded set.  [HN] (key points) adds that the
shallow-layer pool makes the deeper layers' cost constant in context length.

Readings where the pages are silent: the score of position j is the plain dot
product of the layer's 64-d E4M3 indexer query with position j's 64-d E4M3
indexer key (no activation, no head weights, no scale); keys are shared by all
layers, queries are per layer.

Every E4M3 value is an integer multiple of 2^-9 below 2^18 * 2^-9 in
magnitude, so each product is an integer multiple of 2^-18 and a 64-term sum
is an integer below 2^42 in those units: the score is computed exactly in
int64.  ``scores_exact`` returns those integers; ``scores_f64`` is the same
quantity through a float64 matrix product (exact for the same reason).
"""
import numpy as np
from .formats import e4m3_decode

SCORE_UNIT = 2.0 ** -18       # value of one integer score unit


def _e4m3_int(codes) -> np.ndarray:
    """E4M3 bytes -> exact integer multiples of 2^-9 (int64)."""
    v = e4m3_decode(codes)
    if np.isnan(v).any():
        raise ValueError("NaN E4M3 code in indexer input")
    return np.rint(v * 512.0).astype(np.int64)


def scores_exact(q_idx: np.ndarray, k_idx: np.ndarray) -> np.ndarray:
    """Exact indexer scores in units of 2^-18.

    q_idx: uint8 [D] or [R, D] E4M3;  k_idx: uint8 [T, D] E4M3.
    Returns int64 [T] or [R, T].
    """
    qi = _e4m3_int(q_idx)
    ki = _e4m3_int(k_idx)
    return qi @ ki.T if qi.ndim == 2 else ki @ qi


def scores_f64(q_idx: np.ndarray, k_idx: np.ndarray) -> np.ndarray:
    """The same scores as float64 values through a float64 matrix product."""
    q = e4m3_decode(q_idx)
    k = e4m3_decode(k_idx)
    return q @ k.T if q.ndim == 2 else k @ q


def full_scores(q_idx: np.ndarray, k_idx: np.ndarray, limit: int = None) -> np.ndarray:
    """Full-mode scores (float64) of one query over every visible position.

    limit: last visible position (causal prefill); None means all positions.
    Invisible positions get -inf.
    """
    s = scores_exact(q_idx, k_idx).astype(np.float64) * SCORE_UNIT
    if limit is not None:
        s = s.copy()
        s[np.arange(s.shape[-1]) > limit] = -np.inf
    return s


def reindex_scores(q_idx: np.ndarray, k_idx: np.ndarray, pool: np.ndarray) -> np.ndarray:
    """Reindex-mode scores (float64) of one query over the pool positions only.

    pool: int [P] positions, -1 for an empty slot (scored -inf).
    """
    pool = np.asarray(pool, dtype=np.int64)
    valid = pool >= 0
    out = np.full(pool.shape, -np.inf)
    if valid.any():
        out[valid] = scores_exact(q_idx, k_idx[pool[valid]]).astype(np.float64) * SCORE_UNIT
    return out
