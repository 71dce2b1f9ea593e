"""Composition of the libcsa2 calls into CSA2 decode layers.

The MarkTechPost retelling of DeepSeek-V4.1-Flash (paragraph on CSA2) gives
each layer a Full, Reindex or Reuse role: a Full layer builds fresh indices
and, in the decoder, a candidate pool of up to 16,384 positions; a Reindex
layer rescores that pool with its own indexer query; a Reuse layer takes the
previous layer's Top-K indices.  Every layer then attends sparsely over the
shared FP4 latent cache and merges a 128-token sliding window of its own
(paragraph 2; the HN summary's key points).

This module only allocates buffers and sequences the C calls on one stream;
every arithmetic step runs in the HIP kernels of libcsa2.
"""
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

from . import (csa2_fp4_pack, csa2_decode_append, csa2_index_full, csa2_index_reindex, csa2_topk,
               csa2_topk_workspace_size, csa2_topk_pool, csa2_topk_pool_workspace_size, csa2_sparse_swa_decode_layers,
               csa2_index_full_pool, csa2_index_full_pool_workspace_size,
               csa2_sparse_swa_decode_layers_workspace_size,
               csa2_sparse_decode, csa2_sparse_decode_workspace_size, csa2_swa_merge,
               csa2_swa_merge_workspace_size, csa2_sparse_swa_decode, csa2_sparse_swa_decode_workspace_size)

LATENT = 512
POOL_MAX = 16384


def pack_cache(codes: torch.Tensor, scales: torch.Tensor, latent_chunk, chunk_rows: int, stream=None):
    """Fill an FP4 cache codes [B, T, 256] / scales [B, T, 32] from bf16 latent rows.

    latent_chunk(b, c) returns bf16 [rows, 512] for rows [c*chunk_rows, ...) of
    sequence b (fewer rows for the last chunk).
    """
    B, T, _ = codes.shape
    n_chunks = (T + chunk_rows - 1) // chunk_rows
    for b in range(B):
        for c in range(n_chunks):
            x = latent_chunk(b, c)
            r0 = c * chunk_rows
            n = x.shape[0]
            csa2_fp4_pack(x, codes[b, r0:r0 + n], scales[b, r0:r0 + n], stream=stream)


@dataclass
class LayerIO:
    """Per-layer inputs: latent queries, indexer query, sliding-window state."""
    q_lat: torch.Tensor          # bf16 [B, H, 512]
    q_idx: torch.Tensor          # uint8 [B, 64]
    swa: torch.Tensor            # bf16 [B, S, 512]
    swa_start: torch.Tensor      # int32 [B]
    swa_len: torch.Tensor        # int32 [B]


class StackIO:
    """The per-layer inputs of all L layers in stacked tensors (layer-major):
    q_lat bf16 [L, B, H, 512], q_idx uint8 [L, B, 64], swa bf16 [L, B, S, 512],
    swa_start / swa_len int32 [L, B].  With stacked inputs every layer's
    attention runs in one launch; .layers gives per-layer views."""

    def __init__(self, q_lat, q_idx, swa, swa_start, swa_len):
        self.q_lat, self.q_idx, self.swa, self.swa_start, self.swa_len = q_lat, q_idx, swa, swa_start, swa_len
        self.layers = [LayerIO(q_lat[l], q_idx[l], swa[l], swa_start[l], swa_len[l]) for l in range(q_lat.shape[0])]

    def __len__(self):
        return len(self.layers)

    def __getitem__(self, l):
        return self.layers[l]


class Csa2DecodeStack:
    """Preallocated buffers and the call sequence of one decode step.

    modes: e.g. ("full",) or ("full", "reindex", "reuse", "reuse").  A pool of
    min(POOL_MAX, T) candidates is built by the Full layer only when a
    Reindex layer follows it.
    """

    def __init__(self, B: int, T: int, H: int, K: int, modes: Sequence[str], device="cuda",
                 pool_size: int = POOL_MAX, fused_attention: bool = True):
        self.B, self.T, self.H, self.K = B, T, H, K
        self.modes = tuple(modes)
        self.use_pool = "reindex" in self.modes
        self.P = min(pool_size, T) if self.use_pool else 0
        self.P = (self.P + 3) // 4 * 4
        dev = torch.device(device)
        f32, i32, u8 = torch.float32, torch.int32, torch.uint8
        self.scores = torch.empty((B, T), dtype=f32, device=dev)
        self.L = len(self.modes)
        self.idx = torch.empty((self.L, B, K), dtype=i32, device=dev)
        if self.use_pool:
            self.pool = torch.empty((B, self.P), dtype=i32, device=dev)
            self.pool_scores = torch.empty((B, self.P), dtype=f32, device=dev)
            self.re_scores = torch.empty((B, self.P), dtype=f32, device=dev)
        self.o = torch.empty((self.L, B, H, LATENT), dtype=f32, device=dev)
        self.lse = torch.empty((self.L, B, H), dtype=f32, device=dev)
        self.ws_topk_full = torch.empty(max(csa2_topk_workspace_size(B, T, K),
                                            csa2_index_full_pool_workspace_size(B, T, max(self.P, K))),
                                        dtype=u8, device=dev)
        # a Full layer with no Reindex after it selects its Top-K in the same streaming call (pool = Top-K);
        # the call's second output lands here
        self.top_twin = torch.empty((B, K), dtype=i32, device=dev)
        self.ws_topk_pool = (torch.empty(csa2_topk_workspace_size(B, self.P, K), dtype=u8, device=dev)
                             if self.use_pool else None)
        self.ws_sparse = torch.empty(csa2_sparse_decode_workspace_size(B, H, K), dtype=u8, device=dev)
        self.ws_swa = torch.empty(csa2_swa_merge_workspace_size(B, H), dtype=u8, device=dev)
        self.fused_attention = fused_attention
        self.ws_fused = torch.empty(csa2_sparse_swa_decode_workspace_size(B, H, K), dtype=u8, device=dev)
        self.ws_layers = torch.empty(csa2_sparse_swa_decode_layers_workspace_size(self.L, B, H, K), dtype=u8,
                                     device=dev)
        self.index_events = None
        self.attention_events = None
        # the current token's cache row (position T - 1) and position, for the decode-time append
        self.tok_rows = torch.arange(B, dtype=torch.int64, device=dev) * T + (T - 1)
        self.tok_pos = torch.full((B,), T - 1, dtype=torch.int64, device=dev)

    def step(self, codes, scales, k_idx, layers, sigma: float, new_rows: Optional[torch.Tensor] = None,
             stream=None, time_index: bool = False, new_keys: Optional[torch.Tensor] = None,
             new_window: Optional[torch.Tensor] = None, time_attention: bool = False):
        """Run every layer once.  layers: a StackIO (all layers' attention in one
        launch, after the selections) or a list of LayerIO (one attention call
        per layer).  new_rows (bf16 [B, 512]), if given, is the current token's
        latent row, appended first at position T-1 of each sequence
        (csa2_decode_append): packed into the FP4 cache, with its indexer key
        new_keys (E4M3 [B, 64]) copied into k_idx and, with a StackIO whose
        window rings hold 256 rows, its window rows new_window (bf16 [L, B, 512])
        written into each layer's ring (the window bounds are updated).

        time_index: record HIP events around the Full-layer index call on the
        stream (self.index_events holds the (start, end) pair).  time_attention:
        the same around the stacked attention launch (self.attention_events)."""
        B, T, K = self.B, self.T, self.K
        stacked = layers if isinstance(layers, StackIO) else None
        ios = layers.layers if stacked is not None else list(layers)
        if new_rows is not None:
            win = None
            if new_window is not None:
                if stacked is None:
                    raise ValueError("window rows are appended through a StackIO")
                win = stacked
            csa2_decode_append(new_rows, self.tok_rows, codes.view(-1, codes.shape[-1]),
                               scales.view(-1, scales.shape[-1]), new_keys=new_keys,
                               k_idx=k_idx.view(-1, k_idx.shape[-1]) if new_keys is not None else None,
                               new_window=new_window, swa=win.swa if win is not None else None,
                               tok_pos=self.tok_pos if win is not None else None,
                               swa_start=win.swa_start if win is not None else None,
                               swa_len=win.swa_len if win is not None else None, stream=stream)
        src = []                       # index slice used by each layer
        for li, (mode, io) in enumerate(zip(self.modes, ios)):
            idx = self.idx[li]
            if mode == "full":
                if self.use_pool and K <= self.P:
                    # the pool and this layer's Top-K (the top K of the pool) in one call; the
                    # scores themselves are not needed and not written
                    ev = self._scan_events() if time_index else None
                    csa2_index_full_pool(io.q_idx, k_idx, None, self.P, K, self.pool, idx,
                                         pool_scores=self.pool_scores, workspace=self.ws_topk_full,
                                         scan_events=ev, stream=stream)
                    if time_index:
                        self.index_events = ev
                    src.append(li)
                    continue
                if not self.use_pool:
                    # the Top-K straight from the streaming selection: no score array is written
                    ev = self._scan_events() if time_index else None
                    csa2_index_full_pool(io.q_idx, k_idx, None, K, K, idx, self.top_twin,
                                         workspace=self.ws_topk_full, scan_events=ev, stream=stream)
                    if time_index:
                        self.index_events = ev
                    src.append(li)
                    continue
                if time_index:
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                csa2_index_full(io.q_idx, k_idx, self.scores, stream=stream)
                if time_index:
                    e1.record()
                    self.index_events = (e0, e1)
                if self.use_pool:
                    csa2_topk(self.scores, self.P, self.pool, score_out=self.pool_scores,
                              workspace=self.ws_topk_full, stream=stream)
                    csa2_topk(self.scores, K, idx, workspace=self.ws_topk_full, stream=stream)
                else:
                    csa2_topk(self.scores, K, idx, workspace=self.ws_topk_full, stream=stream)
                src.append(li)
            elif mode == "reindex":
                csa2_index_reindex(io.q_idx, k_idx, self.pool, self.re_scores, stream=stream)
                csa2_topk(self.re_scores, K, idx, index_map=self.pool, workspace=self.ws_topk_pool, stream=stream)
                src.append(li)
            elif mode == "reuse":
                if not src:
                    raise ValueError("a Reuse layer needs a preceding Full or Reindex layer")
                src.append(src[-1])
            else:
                raise ValueError(mode)
        if stacked is not None and self.fused_attention:
            ev = self._event_pair() if time_attention else None
            if ev:
                ev[0].record(stream)
            csa2_sparse_swa_decode_layers(stacked.q_lat, codes, scales, self.idx, src, stacked.swa, stacked.swa_start,
                                          stacked.swa_len, sigma, self.o, self.lse, workspace=self.ws_layers,
                                          stream=stream)
            if ev:
                ev[1].record(stream)
                self.attention_events = ev
            return self.o, self.lse
        for li, io in enumerate(ios):
            idx = self.idx[src[li]]
            if self.fused_attention:
                csa2_sparse_swa_decode(io.q_lat, codes, scales, idx, io.swa, io.swa_start, io.swa_len, sigma,
                                       self.o[li], self.lse[li], workspace=self.ws_fused, stream=stream)
            else:
                csa2_sparse_decode(io.q_lat, codes, scales, idx, sigma, self.o[li], self.lse[li],
                                   workspace=self.ws_sparse, stream=stream)
                csa2_swa_merge(io.q_lat, io.swa, io.swa_start, io.swa_len, sigma, self.o[li], self.lse[li],
                               o_sparse=self.o[li], lse_sparse=self.lse[li], workspace=self.ws_swa, stream=stream)
        return self.o, self.lse

    @staticmethod
    def _event_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def _scan_events(self):
        # a fresh, already-created pair of timing events (the library records them)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        e1.record()
        return e0, e1

    def layer_idx(self, li: int) -> torch.Tensor:
        """Indices used by layer li (a Reuse layer reports the indices it took)."""
        j = li
        while self.modes[j] == "reuse":
            j -= 1
        return self.idx[j]
