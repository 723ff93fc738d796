"""CPU oracles for Multi-Segment Attention, the KV write, the Eq. 5 latency
model and the eviction order -- test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the HIP path.
"""
from .evict_oracle import EvictOracle, block_cost, lambda_from_lifespan, weight
from .kv_write_oracle import write_kv
from .latency_oracle import chunk_blocks, delta_b, fit_latency, latency, model_terms
from .msa_oracle import attend, gather_context, masked_softmax_attention, merge_partials

__all__ = ["EvictOracle", "block_cost", "lambda_from_lifespan", "weight", "attend", "gather_context", "masked_softmax_attention", "merge_partials", "write_kv",
           "chunk_blocks", "delta_b", "fit_latency", "latency", "model_terms"]
