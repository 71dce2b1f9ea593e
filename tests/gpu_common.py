"""Helpers shared by the GPU parity tests: device selection, the tolerance
rules, and seeded device workloads built with the library's own pack call.

Tolerances (the design notes derive them):
  * FP4 codes, scales, unpacked bf16, Top-K over given scores: bit-exact;
  * indexer scores: |gpu - exact| <= 64 * 2^-24 * sum_d |q_d k_d| (fp32
    accumulation of 64 exact products);
  * Top-K sets from GPU scores vs exact scores: equal except swaps among
    scores within 1e-6 relative (checked on the exact scores);
  * attention: per (row, head) max_c |o - o_ref| / max_c |o_ref| <= 2e-3 and
    |lse - lse_ref| <= 1e-4 (absolute).
"""
import numpy as np
import pytest
import torch

import workloads as W
from fp4_sparse_attention_amd.decode import LayerIO, StackIO, pack_cache

ATTN_RTOL = 2e-3
LSE_TOL = 1e-4
SWAP_RTOL = 1e-6


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def np_u8(t):
    return t.detach().cpu().numpy().astype(np.uint8, copy=False)


def bf16_to_f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def assert_attention_close(o, lse, o_ref, lse_ref, what=""):
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    denom = np.abs(o_ref).max(axis=-1)
    err = np.abs(o - o_ref).max(axis=-1)
    empty = np.isneginf(lse_ref)
    rel = np.where(empty, err, err / np.maximum(denom, 1e-300))
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= ATTN_RTOL, f"{what}: max normwise relative error {worst:.3e} > {ATTN_RTOL}"
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty-set pattern differs"
    ok = ~empty
    if ok.any():
        lerr = np.abs(lse[ok] - lse_ref[ok])
        assert float(lerr.max()) <= LSE_TOL, f"{what}: lse error {float(lerr.max()):.3e}"
    return worst


def assert_topk_swap_rule(gpu_idx, ref_idx, exact_score_of, what=""):
    """gpu_idx / ref_idx: int arrays (with -1 padding); exact_score_of(pos) -> float."""
    g = [int(x) for x in np.asarray(gpu_idx) if x >= 0]
    o = [int(x) for x in np.asarray(ref_idx) if x >= 0]
    assert len(g) == len(set(g)), f"{what}: duplicate indices"
    assert len(g) == len(o), f"{what}: {len(g)} selected vs {len(o)}"
    assert list(np.asarray(gpu_idx)[:len(g)]) == sorted(g), f"{what}: not ascending / padding not at the end"
    extra = sorted(set(g) - set(o))
    missing = sorted(set(o) - set(g))
    for i in extra:
        si = exact_score_of(i)
        for j in missing:
            sj = exact_score_of(j)
            assert abs(si - sj) <= SWAP_RTOL * max(abs(si), abs(sj)), \
                f"{what}: swap {i} ({si}) for {j} ({sj}) beyond 1e-6"
    return len(extra)


class DecodeWorkload:
    """Seeded decode inputs on the GPU.  The FP4 cache is packed by the library
    (csa2_fp4_pack) from latent rows drawn chunk by chunk; host copies of any
    latent row can be regenerated for the oracle."""

    def __init__(self, B, T, H, n_layers, seed, window=128, chunk_rows=65536, dev=None):
        self.dev = dev or device()
        self.B, self.T, self.H, self.seed = B, T, H, seed
        self.chunk_rows = min(chunk_rows, T)
        self.n_chunks = (T + self.chunk_rows - 1) // self.chunk_rows
        self.outliers = W.outlier_channels(seed)
        self.codes = torch.empty((B, T, 256), dtype=torch.uint8, device=self.dev)
        self.scales = torch.empty((B, T, 32), dtype=torch.uint8, device=self.dev)
        pack_cache(self.codes, self.scales, self.latent_chunk, self.chunk_rows)
        self.k_idx = torch.stack([W.fp8_normal(seed, (T, 64), device=self.dev, chunk_index=b) for b in range(B)])
        S = window
        ds = [W.decode_layer_inputs(seed, li, B, H, S, B, device=self.dev, outliers=self.outliers)
              for li in range(n_layers)]
        ln = min(window, T)
        self.layers = [] if n_layers == 0 else StackIO(torch.stack([d["q_lat"] for d in ds]), torch.stack([d["q_idx"] for d in ds]),
                              torch.stack([d["swa"] for d in ds]),
                              torch.zeros((n_layers, B), dtype=torch.int32, device=self.dev),
                              torch.full((n_layers, B), ln, dtype=torch.int32, device=self.dev))
        torch.cuda.synchronize()

    def latent_chunk(self, b, c):
        n = min(self.chunk_rows, self.T - c * self.chunk_rows)
        return W.latent_rows(self.seed, n, device=self.dev, outliers=self.outliers,
                             chunk_index=b * self.n_chunks + c)

    def latent_host(self, b, positions):
        """float64 [len(positions), 512] latent rows of sequence b (regenerated)."""
        positions = np.asarray(positions, dtype=np.int64)
        out = np.empty((positions.shape[0], 512))
        chunk = positions // self.chunk_rows
        for c in np.unique(chunk):
            sel = chunk == c
            local = torch.from_numpy(positions[sel] - c * self.chunk_rows).to(self.dev)
            out[sel] = self.latent_chunk(b, int(c))[local].to(torch.float64).cpu().numpy()
        return out

    def k_idx_host(self, b):
        return np_u8(self.k_idx[b])
