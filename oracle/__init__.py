"""CPU oracle for query/Forecast-conditioned block selection and block-sparse attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package: only the tests, the package's smoke check and the
benchmark's CPU-baseline leg use it. It shares no code with the HIP library
and never imports it; it receives plain numpy arrays.

It is a slow, plain restatement of the method on the page "SparDA: Sparse
Decoupled Attention for Efficient Long-Context LLM Inference" (picx.dev
summary), section "Theoretical Foundation" (Eq. 1 block union, Eq. 2
mean-pooled compressed keys) and section "Methodology" (Eq. 4 Forecast-driven
top-k, Eq. 5 attention over the chosen blocks, "Compact Forecast Indexer", and
the Eq. 6 group-summed softmax form of the query-driven selector), plus the
token-level variant with one index shared across layers (oracle.token: the
CLSA abstract and the JSSA item) and the selection-quality measures
(oracle.quality), and the second-order block statistic read from the COBS
abstract (oracle.cobs, parity unpinned by the pages). Arithmetic is
fp64 from the compressed keys onward; the compressed keys themselves are formed
in a fixed fp32 order and rounded to the key dtype, so they are one exact value;
the second-order block statistics are fp64 mean and variance rounded once.

Pinned by the tests under tests/ marked "not gpu" (closed forms, library
special cases, invariants and brute force). Parity unpinned by the pages: which
compressed entries belong to a 64-token block (pinned only by brute force over
that definition, see oracle.select), and the whole of oracle.cobs (the pages
give no formula for the second-order statistic; pinned only by the mathematics
of the cumulant expansion and by the first-order block path).
"""
from .numerics import bf16_round, round_to, round_once
from .compress import n_compressed, n_blocks, compressed_keys, append_compressed_keys
from .select import (SOFTMAX_SUM, RAW_SUM, entry_scores, block_scores, block_entries,
                     candidate_sets, top_k_blocks, select_blocks, SelectParams)
from .attention import sparse_attention, lse_merge, split_attention_partials
from .decode import decode_step, decode_unit
from .prefill import prefill_tile_select, prefill_attention, prefill_chunk, tile_attention
from .crosslayer import crosslayer_step
from .quality import block_mass, recall, rest_bucket_distribution, mass_optimal_blocks
from .token import (token_candidates, token_scores, top_k_tokens, select_tokens,
                    token_decode_unit, token_crosslayer_step)
from .cobs import block_stats, cobs_log_mass, cobs_block_scores, select_blocks_cobs

__all__ = [
    "bf16_round", "round_to", "round_once", "n_compressed", "n_blocks", "compressed_keys",
    "append_compressed_keys", "SOFTMAX_SUM", "RAW_SUM", "entry_scores", "block_scores",
    "block_entries", "candidate_sets", "top_k_blocks", "select_blocks", "SelectParams",
    "sparse_attention", "lse_merge", "split_attention_partials", "decode_step", "decode_unit",
    "prefill_tile_select", "prefill_attention", "prefill_chunk", "tile_attention",
    "crosslayer_step",
    "block_mass", "recall", "rest_bucket_distribution", "mass_optimal_blocks",
    "token_candidates", "token_scores", "top_k_tokens", "select_tokens", "token_decode_unit",
    "token_crosslayer_step", "block_stats", "cobs_log_mass", "cobs_block_scores",
    "select_blocks_cobs",
]
