"""fp64 CPU oracle for Sketch Attention compression (test infrastructure).

Only the tests, the smoke check and the bench's CPU-baseline leg use this
package.  The GPU library never imports it, and it imports nothing from the
GPU library; the two share only the seeded inputs of ``synth``.
"""
from .sa_oracle import (  # noqa: F401
    allocations,
    logits,
    normalised_rows_batch,
    sketch_batch,
    sketch_one,
)
from .sa_oracle_grad import sketch_batch_grad, sketch_one_grad  # noqa: F401,E402
from .sa_oracle_target import target_attention_batch, target_attention_one  # noqa: F401,E402
