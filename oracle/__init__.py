"""CPU oracle for the sigmoid Top-K MoE router and its expert-bias load balancer.

TEST INFRASTRUCTURE.  This package is the plain, slow, obviously correct statement of
what the GPU library computes, evaluated in float64 with numpy, one definition per
function, each citing the passage it follows.  Only the test suite, the package's smoke
check and the benchmark's CPU-baseline leg may import it.  The GPU library never does,
and the two share no code: not a kernel, a header, a helper or a constant table.

Sources, cited by page title and section/equation:
  * "SMEBU Load Balancing" (AI Engineer Exhaustive study note on Arcee Trinity),
    section "How it works", equations (17) and (20)-(28);
  * "Arcee Trinity Large Technical Report" (paperlayer.ai summary), section 2.3
    "Mixture-of-Experts";
  * "Arcee Halts 400B Blackwell Model Collapse With Dynamic Router Biases" (summary of
    the Ai4 talk), section "The MaxVio Metric and the Day-4 Crisis";
  * the hotdry blog post on Trinity Large MoE routing and load balancing, section on
    sigmoid routing and Top-K selection.

Parity status of every function is listed in the functions' docstrings; all are pinned
by tests under tests/ (closed forms, brute force, invariants, library routines).
"""

from .backward import RouterGrads, logit_grads, router_backward, router_loss  # noqa: F401
from .balance import BalanceStep, balance_layers, balance_step, normalized_violation  # noqa: F401
from .loads import dispatch_permutation, expert_loads, max_violation  # noqa: F401
from .router import (  # noqa: F401
    Route,
    gate_values,
    route,
    router_logits,
    select_topk,
    sigmoid_scores,
    widen,
)
from .moe import combine, permute_rows  # noqa: F401
from .zloss import router_z_loss, z_loss_from_lse  # noqa: F401
