"""CPU oracle (test infrastructure only): see fljsd_oracle's module docstring."""
from .fljsd_oracle import (REDUCTIONS, reduction_scale, log_softmax, jsd_rows,
                           generalized_jsd, jsd_logprob, tvd, fused_linear_jsd,
                           fused_linear_jsd_rows)

__all__ = ["REDUCTIONS", "reduction_scale", "log_softmax", "jsd_rows",
           "generalized_jsd", "jsd_logprob", "tvd", "fused_linear_jsd",
           "fused_linear_jsd_rows"]
