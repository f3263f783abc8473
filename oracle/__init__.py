"""CPU oracle for fused exact attention (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The library under exact_io_aware_51_amd never does.
"""
from .attention import (attention_backward, attention_backward_terms, attention_backward_dropout, attention_backward_kv,
                        attention_backward_rows, attention_backward_sparse, attention_forward,
                        attention_forward_dropout, attention_forward_fp8, attention_forward_kv, attention_forward_panel,
                        attention_forward_rows,
                        attention_forward_sparse, attention_forward_sparse_rows, attention_probs, dropout_keep, dropout_threshold, e4m3_decode, e5m2_decode,
                        philox4x32)

__all__ = ["attention_forward", "attention_backward", "attention_backward_terms", "attention_probs",
           "attention_forward_rows", "attention_forward_panel", "attention_backward_rows",
           "attention_forward_kv", "attention_backward_kv",
           "attention_forward_sparse", "attention_backward_sparse", "attention_forward_sparse_rows",
           "attention_forward_dropout", "attention_backward_dropout", "dropout_keep", "dropout_threshold",
           "philox4x32", "e4m3_decode", "e5m2_decode", "attention_forward_fp8"]
