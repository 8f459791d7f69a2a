"""fp64 CPU oracle for attention (forward and backward): TEST INFRASTRUCTURE ONLY.

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg,
never by the GPU library.  See oracle/attention.py for the definitions and the
passages of the pages they follow.
"""

from .attention import (alibi_bias, aligned_key_position, as_f64, attention_backward,  # noqa: F401
                        attention_backward_varlen, attention_forward, attention_kvcache, attention_sampled, attention_varlen,
                        brute_force, combine, head_rows, rotary, round_bf16, round_fp16, slope_table,
                        softmax_rows, split_bounds, splitkv_partials, visible_mask)
