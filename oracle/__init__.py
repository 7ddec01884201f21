"""CPU oracle (test infrastructure only): see fljsd_oracle's module docstring."""
from .fljsd_oracle import (REDUCTIONS, reduction_scale, log_softmax, jsd_rows,
                           generalized_jsd, jsd_logprob, tvd, fused_linear_jsd,
                           fused_linear_jsd_rows, cross_entropy_rows, ce_reduction_scale,
                           fused_linear_cross_entropy)

__all__ = ["REDUCTIONS", "reduction_scale", "log_softmax", "jsd_rows",
           "generalized_jsd", "jsd_logprob", "tvd", "fused_linear_jsd",
           "fused_linear_jsd_rows", "cross_entropy_rows", "ce_reduction_scale",
           "fused_linear_cross_entropy"]
