"""CPU oracle of the K2 MoE layer forward -- test infrastructure only.

Imported by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py``; never by the product path.  See ``moe_oracle`` for the
definition it implements and the readings it takes.
"""
from .moe_oracle import (RSF_K2, combine, dequant_fp8, dequant_q4, e4m3_value, expert_param_count, moe_forward,
                         moe_forward_given_routing, permute, route, router_logits, sigmoid, silu, swiglu_expert)

__all__ = ["RSF_K2", "combine", "dequant_fp8", "dequant_q4", "e4m3_value", "expert_param_count", "moe_forward",
           "moe_forward_given_routing", "permute", "route", "router_logits", "sigmoid", "silu", "swiglu_expert"]
