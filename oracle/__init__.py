"""CPU oracle for CSA2 FP4 sparse-attention decode — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the hot path
computes, in float64 and exact integers.  Only the test suite, the package's
smoke check and the benchmark's CPU-baseline leg may import it.  The HIP
library never calls, links or imports anything here, and nothing here imports
the HIP library or its binding.

Sources (cited by title and block; the pages have no numbered sections):
  [HN]  "DeepSeek-v4.1 Flash: Pushing the Limits of KV Cache Compression"
        (hackernews.kjhq.dev summary), block "key points".
  [HF]  "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
        (Hugging Face paper page), abstract.
  [MTP] "DeepSeek AI Released DeepSeek-V4.1-Flash with 1M Context, FP4 KV
        Cache, and Cross-Layer Attention Reuse" (retelling of MarkTechPost),
        paragraphs 1-5.
  [FO]  "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
        (fanout.sh lesson), block "What you will learn".
  [OCP] OCP Microscaling Formats (MX) v1.0 specification: element encodings
        E2M1 (FP4) and E4M3 (FP8), which the NVFP4 layout named in [MTP] ¶4
        builds on.

Module map:
  formats    E2M1 / E4M3 codecs and the FP4 block pack/unpack     [MTP] ¶4
  indexer    exact indexer scores, Full and Reindex scoring          [MTP] ¶3, [HN]
  topk       Top-K / candidate-pool selection                         [HN], [MTP] ¶3
  attention  sparse attention, sliding window, log-sum-exp merge,     [HN], [MTP] ¶2, [FO]
             query absorption / output unabsorption (per-head MLA maps)
  pipeline   one decode layer in Full / Reindex / Reuse role          [MTP] ¶3, [FO]
  paging     logical view of a paged global KV pool                    [HF] abstract

Parity pins: every function is checked by tests marked "not gpu" against
closed forms, brute force, library routines or invariants; see the test files
named test_oracle_*.py.  No function here is "parity unpinned".
"""
from . import formats, indexer, topk, attention, pipeline, paging  # noqa: F401
