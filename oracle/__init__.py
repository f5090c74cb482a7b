"""CPU oracle of the MoE FFN layer forward and backward (float64 numpy) -- test infrastructure.

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline leg may
import this package. The GPU library never does and shares no code with it.
"""
from .moe_backward import aux_loss, backward, gate_backward, router_probabilities, silu_grad, swiglu_backward
from .moe_oracle import (SIGMOID, SOFTMAX, combine, dequantize_rows, e4m3_value, expert_capacity,
                         forward, fp8_expert, gate_values, grouped_mlp, permute, route, router_logits,
                         select_topk, shared_mlp, silu, swiglu_ffn, token_outputs)

__all__ = ["SIGMOID", "SOFTMAX", "combine", "dequantize_rows", "e4m3_value", "expert_capacity",
           "forward", "fp8_expert", "gate_values", "grouped_mlp", "permute", "route", "router_logits",
           "select_topk", "shared_mlp", "silu", "swiglu_ffn", "token_outputs",
           "aux_loss", "backward", "gate_backward", "router_probabilities", "silu_grad", "swiglu_backward"]
