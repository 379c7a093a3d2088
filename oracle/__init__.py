"""CPU fp64 oracle of the attention-mass top-k prefill path.

TEST INFRASTRUCTURE ONLY: this package is the checker. Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it. The HIP library and its Python binding never do; the product path
raises when the HIP extension is missing instead of falling back to this.
"""
from .attention_mass import (OracleLayer, IndexerOracle, KLDistillOracle, row_logits,
                             log_sum_exp, head_mass, top_units, kth_score, block_masses, tokens_of_blocks,
                             support_attention, dense_attention, causal_sparsity,
                             default_scale, kv_head, query_block_rows, captured_mass,
                             support_overlap)

__all__ = ["OracleLayer", "IndexerOracle", "KLDistillOracle", "row_logits", "log_sum_exp",
           "head_mass", "top_units", "kth_score", "block_masses", "tokens_of_blocks", "support_attention",
           "dense_attention", "causal_sparsity", "default_scale", "kv_head", "query_block_rows",
           "captured_mass", "support_overlap"]
