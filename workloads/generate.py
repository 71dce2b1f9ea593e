"""Seeded synthetic inputs.

Each tensor role draws from its own torch.Generator seeded with
``seed * 1000 + role`` so that a tensor does not depend on which other tensors
were drawn first.  On a CUDA/HIP device torch uses its Philox generator, on the
CPU its Mersenne-Twister one, so the same seed gives different values on the
two devices; every comparison feeds one drawn tensor to both sides.

Recipe (values are standard normal before the cast):
  * latent KV rows: bf16, with ``floor(1% * channels)`` outlier channels (picked by
    a seeded permutation, fixed for every row) scaled by 8 before the cast;
  * indexer keys and queries: 64-d OCP E4M3FN (torch cast, round-to-nearest-even);
  * latent queries: bf16 with std 0.5, the spread a unit-normal 128-d head query
    has after absorption into the 512-channel latent by N(0, 1/512) weights;
  * sliding-window rows: bf16, same outlier channels as the latent KV;
  * per-head queries (128-d, before absorption): bf16 N(0, 1);
  * absorption weights W_UK, W_UV [heads, 128, 512]: bf16 N(0, 1/512).
"""
import numpy as np
import torch

# role ids for per-tensor generator seeds
_ROLE_OUTLIER, _ROLE_LATENT, _ROLE_KIDX, _ROLE_QIDX, _ROLE_QLAT, _ROLE_SWA, _ROLE_MISC = range(7)
_ROLE_QHEAD, _ROLE_WUK, _ROLE_WUV = 7, 8, 9


def _gen(seed: int, role: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed) * 1000 + role)
    return g


def outlier_channels(seed: int, channels: int = 512, frac: float = 0.01) -> torch.Tensor:
    """Sorted channel ids of the outlier channels (CPU int64)."""
    n = int(np.floor(frac * channels))
    g = _gen(seed, _ROLE_OUTLIER, "cpu")
    return torch.sort(torch.randperm(channels, generator=g)[:n]).values


def latent_rows(seed: int, n: int, channels: int = 512, device="cpu", role_offset: int = 0,
                outliers: torch.Tensor = None, chunk_index: int = 0) -> torch.Tensor:
    """bf16 [n, channels] latent rows, N(0,1) with outlier channels x8.

    ``chunk_index`` selects an independent stream so large caches can be drawn
    chunk by chunk without holding the fp32 draw for the whole cache.
    """
    if outliers is None:
        outliers = outlier_channels(seed, channels)
    g = _gen(seed * 7919 + chunk_index, _ROLE_LATENT + role_offset, device)
    x = torch.randn((n, channels), generator=g, device=device, dtype=torch.float32)
    if outliers.numel():
        x[:, outliers.to(x.device)] *= 8.0
    return x.to(torch.bfloat16)


def fp8_normal(seed: int, shape, device="cpu", role: int = _ROLE_KIDX, chunk_index: int = 0) -> torch.Tensor:
    """uint8 E4M3FN bit patterns of N(0,1) draws (torch cast, RNE)."""
    g = _gen(seed * 7919 + chunk_index, role, device)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def bf16_normal(seed: int, shape, std: float = 1.0, device="cpu", role: int = _ROLE_MISC,
                chunk_index: int = 0) -> torch.Tensor:
    g = _gen(seed * 7919 + chunk_index, role, device)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32) * std
    return x.to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 numpy view of a bf16 tensor's bit patterns (copied to host)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def fp8_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().astype(np.uint8, copy=False)


def bits_to_bf16_float(bits: np.ndarray) -> np.ndarray:
    """float64 values of uint16 bf16 bit patterns (exact widening)."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode_layer_inputs(seed: int, layer: int, rows: int, heads: int, window_rows: int,
                        batch: int, channels: int = 512, index_dim: int = 64, device="cpu",
                        outliers: torch.Tensor = None):
    """Per-layer decode inputs: latent queries, indexer query, sliding-window rows.

    Returns a dict of tensors on ``device``:
      q_lat  bf16 [rows, heads, channels]
      q_idx  uint8 (E4M3FN) [rows, index_dim]
      swa    bf16 [batch, window_rows, channels]
    """
    if outliers is None:
        outliers = outlier_channels(seed, channels)
    q_lat = bf16_normal(seed, (rows, heads, channels), std=0.5, device=device, role=_ROLE_QLAT,
                        chunk_index=layer)
    q_idx = fp8_normal(seed, (rows, index_dim), device=device, role=_ROLE_QIDX, chunk_index=layer)
    g = _gen(seed * 7919 + layer, _ROLE_SWA, device)
    swa = torch.randn((batch, window_rows, channels), generator=g, device=device, dtype=torch.float32)
    if outliers.numel():
        swa[:, :, outliers.to(swa.device)] *= 8.0
    return {"q_lat": q_lat, "q_idx": q_idx, "swa": swa.to(torch.bfloat16)}


def head_queries(seed: int, layer: int, rows: int, heads: int, head_dim: int = 128, device="cpu"):
    """bf16 [rows, heads, head_dim] per-head queries, N(0, 1), before absorption."""
    return bf16_normal(seed, (rows, heads, head_dim), std=1.0, device=device, role=_ROLE_QHEAD,
                       chunk_index=layer)


def absorb_weights(seed: int, layer: int, heads: int, head_dim: int = 128, channels: int = 512,
                   device="cpu"):
    """(W_UK, W_UV): bf16 [heads, head_dim, channels] each, N(0, 1/channels)."""
    std = float(1.0 / np.sqrt(channels))
    w_uk = bf16_normal(seed, (heads, head_dim, channels), std=std, device=device, role=_ROLE_WUK,
                       chunk_index=layer)
    w_uv = bf16_normal(seed, (heads, head_dim, channels), std=std, device=device, role=_ROLE_WUV,
                       chunk_index=layer)
    return w_uk, w_uv
