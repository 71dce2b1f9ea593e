"""Workload shapes.

Every size here is a synthetic stand-in chosen to match the scale the
DeepSeek-V4.1-Flash write-ups describe: up to one million positions of context
(Hugging Face paper page, abstract), a decoder Full layer that fills a pool of
up to 16,384 candidates and later layers in Reindex or Reuse role (MarkTechPost
retelling, paragraph on CSA2), and a 128-token sliding window (same retelling,
paragraphs on the encoder/decoder split and on the KV cache).
"""
from dataclasses import dataclass, field
from typing import Tuple

LATENT_CHANNELS = 512      # latent KV width shared by every head
INDEX_DIM = 64             # indexer key / query width (fp8)
SWA_WINDOW = 128           # sliding-window length
POOL_MAX = 16384           # Full-layer candidate pool bound
HEAD_DIM = 128             # per-head query width before absorption


@dataclass(frozen=True)
class TinyDecode:
    """Single Full-mode decode layer, batch 1, 4,096 positions."""
    name: str = "tiny_decode"
    batch: int = 1
    context: int = 4096
    heads: int = 16
    topk: int = 256
    window: int = SWA_WINDOW
    modes: Tuple[str, ...] = ("full",)
    pool: int = 0
    seed: int = 0


@dataclass(frozen=True)
class PackStream:
    """FP4 pack then unpack of 1,048,576 latent rows (memory-bound stream)."""
    name: str = "pack_1m"
    rows: int = 1 << 20
    channels: int = LATENT_CHANNELS
    seed: int = 2


@dataclass(frozen=True)
class FullDecode:
    """Full-mode decode, batch 64, 131,072 positions per sequence."""
    name: str = "full_decode_b64"
    batch: int = 64
    context: int = 131072
    heads: int = 64
    topk: int = 2048
    window: int = SWA_WINDOW
    modes: Tuple[str, ...] = ("full",)
    pool: int = 0
    seed: int = 1


@dataclass(frozen=True)
class DecodeStack:
    """Four CSA2 layers [Full, Reindex, Reuse, Reuse] at 1M context, batch 8."""
    name: str = "stack_1m_b8"
    batch: int = 8
    context: int = 1 << 20
    heads: int = 64
    topk: int = 2048
    window: int = SWA_WINDOW
    modes: Tuple[str, ...] = ("full", "reindex", "reuse", "reuse")
    pool: int = POOL_MAX
    seed: int = 4


@dataclass(frozen=True)
class ChunkedPrefill:
    """4,096 causal query rows over a 262,144-position cache."""
    name: str = "prefill_4k_256k"
    batch: int = 1
    context: int = 262144
    queries: int = 4096
    heads: int = 64
    topk: int = 2048
    window: int = SWA_WINDOW
    seed: int = 3

    def query_positions(self):
        """The last `queries` positions of the cache, oldest first."""
        return range(self.context - self.queries, self.context)


CONFIGS = (TinyDecode(), PackStream(), FullDecode(), DecodeStack(), ChunkedPrefill())


def by_name(name: str):
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)
