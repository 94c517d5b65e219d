"""CPU reference for the CSA decode path.  Test infrastructure only: imported by
tests/, __graft_entry__.smoke() and the CPU-baseline leg of bench.py, never by
the library or its binding."""
from .csa_oracle import (bf16_to_f64, visible_blocks, indexer_scores,  # noqa: F401
                         select_top_blocks, gather_rows, shared_kv_attention,
                         csa_token, hca_token)
from .fp8_oracle import (e4m3_to_f64, quantize_rows_e4m3, quantize_rows_e4m3_scalar,  # noqa: F401
                         indexer_scores_e4m3, prefilter_count, select_prefiltered,
                         csa_token_e4m3)
from . import producer_oracle  # noqa: F401
