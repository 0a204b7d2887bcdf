"""CPU oracle of the Switch FFN layer forward (test infrastructure only).

Only tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the HIP path.
"""

from .switch_oracle import (  # noqa: F401
    assign_slots,
    combine,
    dispatch,
    expert_capacity,
    expert_ffn,
    forward,
    load_balancing_loss,
    router_logits,
    softmax,
    top1,
)
