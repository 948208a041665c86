"""fp64 CPU oracle for the exact attention forward pass.

TEST INFRASTRUCTURE ONLY: imported by tests/, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``, never by the product path.
"""
from .attention import (as_f64, attention_backward, attention_backward_sampled,
                        attention_forward, attention_partial,
                        backward_error_bound,
                        boundary_scale, causal_offset, decode_e4m3, dequantize_fp8,
                        forward_error_bound_16, fp8_weight_error_bound,
                        merge_partials, split_attention, streaming_attention,
                        weight_rounding_error_bound, ROUNDING_16)

__all__ = ["as_f64", "attention_backward", "attention_backward_sampled", "attention_forward",
           "attention_partial",
           "backward_error_bound", "boundary_scale",
           "causal_offset", "decode_e4m3", "dequantize_fp8", "forward_error_bound_16",
           "fp8_weight_error_bound", "merge_partials", "split_attention",
           "streaming_attention", "weight_rounding_error_bound", "ROUNDING_16"]
