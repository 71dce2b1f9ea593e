"""Sparse attention, sliding window and merge — oracle (test infrastructure only).

[HN] (key points): CSA2 combines local sliding windows, global sparse
retrieval and cross-layer reuse; layers share the same main KV.  [MTP] ¶2:
sliding-window attention runs in every layer and the decoder rebuilds its
window state from the last 128 tokens.  [FO] (What you will learn): queries
and sliding-window state stay layer-local.

Readings where the pages are silent:
  * the H heads of a layer attend over one shared 512-channel latent row per
    position, used as key and as value (absorbed multi-head latent attention);
    queries arrive already absorbed into that latent space, q_lat [H, 512];
  * softmax scale sigma is a parameter (1/sqrt(128) in the workloads);
  * the sliding window holds the layer's own bf16 latent rows of the last
    min(128, t+1) positions, kept apart from the FP4 global cache;
  * window and sparse parts form one softmax over the union of their keys
    (log-sum-exp merge), with no gate, sink or de-duplication.

  * the per-head query and output live in a 128-d head space: a head's key
    is W_UK,h x and its value W_UV,h x for a latent row x (W [128, 512] per
    head), so the query is absorbed as q_lat = W_UK,h^T q and the latent
    output is mapped back as o = W_UV,h o_lat (multi-head latent attention in
    absorbed form; the pages name the 512-channel latent and the 128-d heads,
    not the head mathematics).

All arithmetic is float64; lse is a natural logarithm.
"""
import numpy as np

WINDOW = 128


def attend(q: np.ndarray, rows: np.ndarray, sigma: float):
    """Softmax attention of H query vectors over n key/value rows.

    q: [H, C]; rows: [n, C] (the key and the value of each position).
    Returns (o [H, C], lse [H]).  With n == 0: o = 0, lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    H, C = q.shape
    if rows.shape[0] == 0:
        return np.zeros((H, C)), np.full(H, -np.inf)
    s = sigma * (q @ rows.T)                     # [H, n]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ rows) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def sparse_attend(q: np.ndarray, cache_rows: np.ndarray, idx: np.ndarray, sigma: float):
    """Attention over the cache rows named by idx (entries < 0 are skipped).

    cache_rows: [T, C] dequantised latent rows (float64).
    """
    idx = np.asarray(idx, dtype=np.int64)
    sel = idx[idx >= 0]
    return attend(q, cache_rows[sel], sigma)


def window_rows(swa: np.ndarray, start: int, length: int) -> np.ndarray:
    """The layer's window rows [start, start+length) of its SWA state."""
    return np.asarray(swa, dtype=np.float64)[start:start + length]


def window_len(t: int, window: int = WINDOW) -> int:
    """Number of window positions visible at position t: max(0, t-127)..t."""
    return min(window, t + 1)


def merge(o_a: np.ndarray, lse_a: np.ndarray, o_b: np.ndarray, lse_b: np.ndarray):
    """Combine two softmax results over disjoint key sets into one.

    lse = log(exp(lse_a) + exp(lse_b)); o = exp(lse_a-lse)*o_a + exp(lse_b-lse)*o_b.
    An empty side has lse = -inf and contributes nothing.
    """
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    lse = np.logaddexp(lse_a, lse_b)
    with np.errstate(invalid="ignore"):
        wa = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - lse))
        wb = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - lse))
    o = wa[:, None] * o_a + wb[:, None] * o_b
    return o, lse


def absorb(q: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """Absorbed queries: q_lat[..., h, c] = sum_d q[..., h, d] * w_uk[h, d, c].

    q: [..., H, 128] per-head queries; w_uk: [H, 128, 512], the map from a
    latent row to head h's key.  Returns float64 [..., H, 512].
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w_uk, dtype=np.float64)
    return np.einsum("...hd,hdc->...hc", q, w)


def unabsorb(o_lat: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """Head outputs: o[..., h, d] = sum_c w_uv[h, d, c] * o_lat[..., h, c].

    o_lat: [..., H, 512] attention outputs in the latent space; w_uv:
    [H, 128, 512], the map from a latent row to head h's value.  Returns
    float64 [..., H, 128].
    """
    o = np.asarray(o_lat, dtype=np.float64)
    w = np.asarray(w_uv, dtype=np.float64)
    return np.einsum("...hc,hdc->...hd", o, w)
