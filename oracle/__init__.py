"""CPU fp64 oracle (test infrastructure only; never on the product path)."""

from .attention import (attention_backward, attention_forward, attention_probs,
                        attention_rows, default_scale, row_dvec)

__all__ = ["attention_forward", "attention_backward", "attention_rows",
           "attention_probs", "default_scale", "row_dvec"]
