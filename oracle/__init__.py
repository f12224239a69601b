"""fp64 CPU oracle for the blockwise ring-attention step (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import this
package; the product path never does.
"""
from .attention import (LAYOUTS, attend, attention_bwd, attention_fwd, attention_partial,
                        bwd_delta, chunk_of_token, document_ids, lse_merge, positions,
                        ring_schedule)

__all__ = ["LAYOUTS", "attend", "attention_bwd", "attention_fwd", "attention_partial",
           "bwd_delta", "chunk_of_token", "document_ids", "lse_merge", "positions",
           "ring_schedule"]
