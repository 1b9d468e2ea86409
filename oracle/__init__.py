"""CPU oracle for the memory-efficient linear GRPO loss — TEST INFRASTRUCTURE.

A plain, slow, fp64 NumPy statement of what the loss computes, written from the
pages and checked against closed forms, brute force and finite differences in
``tests/``.  It materialises every row's full vocabulary of logits and shares
no code with the HIP path.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never calls it.

Parity status: every function here is pinned (see the tests named in each
docstring); none is "parity unpinned".
"""

from .grpo_oracle import (  # noqa: F401
    DEFAULT,
    E4M3_MAX,
    dequantize_e4m3_rows,
    e4m3_codes,
    e4m3_round,
    quantize_e4m3_rows,
    advantage_term,
    grad_factor,
    logits,
    Variant,
    forward_kl_k3,
    kl_grad_q,
    kl_value,
    reverse_kl_q,
    token_weights,
    backward,
    dw_rows,
    forward,
    found_inf,
    group_advantages,
    log_softmax_rows,
    logit_grad,
    policy_grad,
    reverse_kl_k3,
    surrogate_objective,
    token_loss,
)
