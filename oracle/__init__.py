"""CPU oracle of the MSA forward (test infrastructure only: tests, smoke check and
the benchmark's CPU-baseline leg).  Nothing in the product path imports it."""
from .msa_oracle import (block_maxima, select_from_maxima, index_select, sparse_attention,  # noqa: F401
                         msa_forward, dense_causal_attention, token_set)
