"""CPU oracle of the TTT layer hot path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does.
"""
from .oracle import (  # noqa: F401
    build,
    load,
    ln_fwd,
    ln_l2_grad,
    rope_row,
    gelu,
    gelu_grad,
    linear_chain,
    linear_chain_dual,
    mlp_chain,
    mlp_chain_dual,
    linear_batch,
    mlp_batch,
    max_threads,
    post_proj,
    set_threads,
)
