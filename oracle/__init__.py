"""CPU float64 oracle for the SQA forward pass and its gradients (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import
this package. The HIP library and its Python binding never do.
"""
from .sqa_oracle import (round_bf16, kv_head_for, split_heads, softmax_probs, attention_rows,
                         sqa_forward, sqa_forward_rows, sqa_forward_varlen, sqa_forward_varlen_rows)
from .bruteforce import sqa_forward_bruteforce
from .backward import (attention_head_backward, softmax_backward, sqa_backward, sqa_backward_rows,
                       sqa_backward_dy_rows)

__all__ = ["round_bf16", "kv_head_for", "split_heads", "softmax_probs", "attention_rows",
           "sqa_forward", "sqa_forward_rows", "sqa_forward_varlen", "sqa_forward_varlen_rows",
           "sqa_forward_bruteforce", "attention_head_backward", "softmax_backward", "sqa_backward",
           "sqa_backward_rows", "sqa_backward_dy_rows"]
