"""CPU oracle of the SwitchFFN forward pass -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The HIP product path never does.
"""
from .switchffn_oracle import (  # noqa: F401
    aux_loss,
    backward,
    capacity,
    dispatch,
    dispatch_topk,
    expert_ffn,
    forward,
    forward_reroute,
    gelu,
    near_tie_second,
    near_tie_tokens,
    round_to_bf16,
    round_to_dtype,
    router,
    reroute_overflow,
    router_logits,
    second_choice,
    softmax,
    top1,
)
