"""Seeded synthetic workloads for CSA2 FP4 sparse-attention decode.

This module holds the workload shapes and the seeded random generators that
feed both the HIP path and the CPU oracle.  It contains none of the method's
arithmetic: no FP4 encoding, no scoring, no selection, no attention.  Values
are drawn from a normal distribution with torch's generator and rounded to the
storage dtype with torch's own casts (bf16 round-to-nearest-even, OCP E4M3FN
round-to-nearest-even); the FP4 cache itself is built by whichever side is
under test.

The shapes follow the DeepSeek-V4.1-Flash write-ups (MarkTechPost retelling,
paragraphs on CSA2 and on the KV cache format): a 512-channel latent KV shared
by all heads, a 128-token sliding window and a candidate pool of up to 16,384
positions.
"""
from .configs import (CONFIGS, TinyDecode, PackStream, FullDecode, DecodeStack,
                      ChunkedPrefill, by_name)
from .generate import (outlier_channels, latent_rows, fp8_normal, bf16_normal,
                       bf16_bits, fp8_bits, bits_to_bf16_float, decode_layer_inputs,
                       head_queries, absorb_weights)

__all__ = [
    "CONFIGS", "TinyDecode", "PackStream", "FullDecode", "DecodeStack", "ChunkedPrefill",
    "by_name", "outlier_channels", "latent_rows", "fp8_normal", "bf16_normal", "bf16_bits",
    "fp8_bits", "bits_to_bf16_float", "decode_layer_inputs", "head_queries", "absorb_weights",
]
